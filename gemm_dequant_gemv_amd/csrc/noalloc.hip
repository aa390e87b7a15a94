// The statically allocated scratch behind qmoe_grouped_noalloc: a file-scope
// device array that stands in for the caller's workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).
//
// Every GPU the library runs on holds its own copy of the array, from the
// moment the code object is loaded on it until the process ends.  In host code
// the array's name is only a host-side stand-in, never a device address: the
// address of each device's copy is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept in a table, and only
// that address is ever handed to kernels.
#include <mutex>

#include "qmm_internal.h"

namespace qmm {
namespace {

__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

}  // namespace

hipError_t noalloc_scratch(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace qmm
