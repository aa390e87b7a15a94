// qmoe_router: the MoE router's top-k and softmax ("TurboEXL3" section 4.2,
// the decode chain folds the router's top-k and softmax into its first
// launch; section 3.1 and the model description: each token picks 10 of 512
// routed experts by router score, weighted by a softmax).
//
// One wave per token.  Lane l holds the logits l, l + 64, l + 128, ... of its
// token as order keys (a float32 mapped to a uint32 whose unsigned order is
// the float order, -0 taken as +0).  Each of the k rounds finds the largest
// key not yet taken: every lane its own best (ascending index, so an equal
// key keeps the lower index), then the maximum over (key, inverted index)
// across the wave (DPP inside each row of 16 lanes, then the four rows), so
// equal logits go to the lower expert id; the owner lane
// marks the winner taken.  Lane r keeps round r's expert and logit, so the
// list comes out in descending logit order (each winner's logit is read back
// from its key).  The weights are the softmax of
// the k chosen logits in float32: e_r = exp(l_r - l_0), divided by their sum,
// taken over a fixed tree (the same bits on every run).
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace {

constexpr int kRouterWaves = 4;  // tokens per workgroup

struct RouterArgs {
  const float *logits;  // [t][e]
  int t, e, k;
  int32_t *ids;  // [t][k]
  float *w;      // [t][k]
};

__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// (hi, lo) = the larger of itself and the pair DPP brings from another lane
// of its row of 16
template <int CTRL>
__device__ __forceinline__ void dpp_max_u64(uint32_t &hi, uint32_t &lo) {
  const uint32_t oh = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, CTRL, 0xF, 0xF, false);
  const uint32_t ol = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, CTRL, 0xF, 0xF, false);
  if (oh > hi || (oh == hi && ol > lo)) {
    hi = oh;
    lo = ol;
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     CTRL, 0xF, 0xF, false));
}

template <int PER>
__global__ __launch_bounds__(64 * kRouterWaves) void moe_router_kernel(RouterArgs a) {
  const int lane = threadIdx.x & 63;
  const int tok = blockIdx.x * kRouterWaves + (int)(threadIdx.x >> 6);
  if (tok >= a.t) return;  // the whole wave
  const float *lg = a.logits + (size_t)tok * a.e;
  uint32_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = lane + 64 * j;
    key[j] = i < a.e ? order_key(lg[i]) : 0u;  // 0: below every finite key
  }
  uint64_t taken = 0;
  int my_id = 0;
  float my_logit = 0.0f;
  for (int r = 0; r < a.k; ++r) {
    uint64_t best = 0;  // (key << 32) | (0xFFFFFFFF - index); 0: none
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = lane + 64 * j;
      const uint64_t c = ((uint64_t)key[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
      if (i < a.e && !((taken >> j) & 1ull) && c > best) best = c;
    }
    // the maximum inside each row of 16 lanes (DPP), then over the four rows
    // (one lane of each, uniform)
    uint32_t bh = (uint32_t)(best >> 32), bl = (uint32_t)best;
    dpp_max_u64<kDppQuadXor1>(bh, bl);
    dpp_max_u64<kDppQuadXor2>(bh, bl);
    dpp_max_u64<kDppHalfMirror>(bh, bl);
    dpp_max_u64<kDppMirror>(bh, bl);
    uint32_t kw = (uint32_t)__builtin_amdgcn_readlane((int)bh, 0);
    uint32_t iw = (uint32_t)__builtin_amdgcn_readlane((int)bl, 0);
#pragma unroll
    for (int row = 1; row < 4; ++row) {
      const uint32_t h = (uint32_t)__builtin_amdgcn_readlane((int)bh, 16 * row);
      const uint32_t l = (uint32_t)__builtin_amdgcn_readlane((int)bl, 16 * row);
      if (h > kw || (h == kw && l > iw)) {
        kw = h;
        iw = l;
      }
    }
    const int win = (int)(0xFFFFFFFFu - iw);
    if ((win & 63) == lane) taken |= 1ull << (win >> 6);
    if (lane == r) {  // the logit back from its key: no reload from memory
      my_id = win;
      my_logit = __uint_as_float((kw & 0x80000000u) ? (kw & 0x7FFFFFFFu) : ~kw);
    }
  }
  // softmax of the k chosen logits (lane r holds round r's; lane 0 the largest)
  const float top = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_logit), 0));
  const float e = lane < a.k ? expf(my_logit - top) : 0.0f;
  // sum: a fixed tree (rows of 16 by DPP, then the four rows), the same in
  // every lane and on every run
  float rs = dpp_add<kDppQuadXor1>(e);
  rs = dpp_add<kDppQuadXor2>(rs);
  rs = dpp_add<kDppHalfMirror>(rs);
  rs = dpp_add<kDppMirror>(rs);
  float r4[4];
#pragma unroll
  for (int row = 0; row < 4; ++row)
    r4[row] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rs), 16 * row));
  const float sum = (r4[0] + r4[1]) + (r4[2] + r4[3]);
  if (lane < a.k) {
    a.ids[(size_t)tok * a.k + lane] = my_id;
    a.w[(size_t)tok * a.k + lane] = e / sum;
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
