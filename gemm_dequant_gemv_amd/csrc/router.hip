// qmoe_router: the MoE router's top-k and softmax ("TurboEXL3" section 4.2,
// the decode chain folds the router's top-k and softmax into its first
// launch; section 3.1 and the model description: each token picks 10 of 512
// routed experts by router score, weighted by a softmax).  One wave per
// token; the per-token work is router::topk_softmax_wave (router_device.h).
#include "qmm_device.h"
#include "qmm_internal.h"
#include "router_device.h"

namespace qmm {
namespace {

constexpr int kRouterWaves = 4;  // tokens per workgroup

struct RouterArgs {
  const float *logits;  // [t][e]
  int t, e, k;
  int32_t *ids;  // [t][k]
  float *w;      // [t][k]
};

template <int PER>
__global__ __launch_bounds__(64 * kRouterWaves) void moe_router_kernel(RouterArgs a) {
  const int tok = blockIdx.x * kRouterWaves + (int)(threadIdx.x >> 6);
  if (tok >= a.t) return;  // the whole wave
  int id;
  float w;
  router::topk_softmax_wave<PER>(a.logits + (size_t)tok * a.e, a.e, a.k, id, w);
  const int lane = threadIdx.x & 63;
  if (lane < a.k) {
    a.ids[(size_t)tok * a.k + lane] = id;
    a.w[(size_t)tok * a.k + lane] = w;
  }
}

template <int PER>
hipError_t launch_router_per(const RouterArgs &a, hipStream_t s) {
  const int blocks = (a.t + kRouterWaves - 1) / kRouterWaves;
  hipLaunchKernelGGL(moe_router_kernel<PER>, dim3(blocks), dim3(64 * kRouterWaves), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const float *logits, int t, int e, int k, int32_t *ids, float *w,
                         hipStream_t s) {
  const RouterArgs a{logits, t, e, k, ids, w};
  const int per = (e + 63) / 64;
  if (per <= 1) return launch_router_per<1>(a, s);
  if (per <= 2) return launch_router_per<2>(a, s);
  if (per <= 4) return launch_router_per<4>(a, s);
  if (per <= 8) return launch_router_per<8>(a, s);
  if (per <= 16) return launch_router_per<16>(a, s);
  if (per <= 32) return launch_router_per<32>(a, s);
  return launch_router_per<64>(a, s);
}

}  // namespace qmm
