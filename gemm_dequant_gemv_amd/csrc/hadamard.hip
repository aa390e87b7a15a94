// The EXL3 rotation stages around an inner product ("TurboEXL3" section 3.1:
// prepare scales the input by the input-channel vector and applies the
// Hadamard transform one 128-element block at a time; finish applies the
// transform to the output and then scales it by the output-channel vector;
// section 2.3: the transforms are sign-randomized Hadamard transforms in
// blocks of 128, and the two 16-bit channel vectors are the only scales).
//
// The transform is the orthonormal one, H_128 / sqrt(128) with H_128 in
// Sylvester's natural order (entry (i, j) = (-1)^popcount(i & j)); the random
// signs travel in the sign bits of the float16 channel scales.
//
// One wave per (row, block of 128): lane l holds elements l and l + 64
// (hadamard128_wave; qgemv_hadamard runs the same routine on its staged
// activations).  Prepare reads bf16 and writes bf16 (rounded to nearest
// even); finish reads float32 and writes float32 or bf16.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace {

struct HadArgs {
  const void *in;         // bf16 (prepare) or float32 (finish) [rows][len]
  const uint16_t *scale;  // float16 [len] or null (all ones)
  void *out;              // bf16 (prepare), float32 or bf16 (finish) [rows][len]
  uint32_t units;         // rows * len / 128
  uint32_t blocks;        // len / 128
  uint32_t len;
  int out_bf16;
};

template <bool PREPARE>
__global__ __launch_bounds__(256) void hadamard_kernel(HadArgs a) {
  const uint32_t unit = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (unit >= a.units) return;  // whole wave
  const int lane = threadIdx.x & 63;
  const uint32_t row = unit / a.blocks, blk = unit - row * a.blocks;
  const size_t base = (size_t)row * a.len + (size_t)blk * 128;
  const uint32_t c0 = blk * 128u + (uint32_t)lane, c1 = c0 + 64u;  // channels
  float v0, v1;
  if constexpr (PREPARE) {
    const uint16_t *x = (const uint16_t *)a.in;
    v0 = bf_lo(x[base + lane]);
    v1 = bf_lo(x[base + lane + 64]);
    if (a.scale) {  // scale first, then transform
      v0 *= half_to_float(a.scale[c0]);
      v1 *= half_to_float(a.scale[c1]);
    }
  } else {
    const float *y = (const float *)a.in;
    v0 = y[base + lane];
    v1 = y[base + lane + 64];
  }
  hadamard128_wave(v0, v1, lane);
  if constexpr (!PREPARE) {
    if (a.scale) {  // transform first, then scale
      v0 *= half_to_float(a.scale[c0]);
      v1 *= half_to_float(a.scale[c1]);
    }
  }
  if (PREPARE || a.out_bf16) {
    uint16_t *o = (uint16_t *)a.out;
    o[base + lane] = (uint16_t)float_to_bf16(v0);
    o[base + lane + 64] = (uint16_t)float_to_bf16(v1);
  } else {
    float *o = (float *)a.out;
    o[base + lane] = v0;
    o[base + lane + 64] = v1;
  }
}

}  // namespace

hipError_t launch_hadamard(bool prepare, const void *in, int rows, int len, const void *scale,
                           void *out, int out_bf16, hipStream_t s) {
  HadArgs a;
  a.in = in;
  a.scale = (const uint16_t *)scale;
  a.out = out;
  a.blocks = (uint32_t)(len / 128);
  a.units = (uint32_t)rows * a.blocks;
  a.len = (uint32_t)len;
  a.out_bf16 = out_bf16;
  const dim3 grid((a.units + 3) / 4);
  if (prepare)
    hipLaunchKernelGGL(hadamard_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(hadamard_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace qmm
