// The router's top-k and softmax for one token, computed by one wave; shared
// by the router kernel (router.hip) and the decode-form gate/up launch that
// folds the router in (moe_gemv.hip), so both give the same bits.
//
// Lane l holds the logits l, l + 64, l + 128, ... of the token as order keys
// (a float32 mapped to a uint32 whose unsigned order is the float order, -0
// taken as +0).  Each of the k rounds finds the largest key not yet taken:
// every lane its own best (ascending index, so an equal key keeps the lower
// index), then the maximum over (key, inverted index) across the wave (DPP
// inside each row of 16 lanes, then the four rows), so equal logits go to the
// lower expert id; the owner lane marks the winner taken.  Lane r keeps round
// r's expert and logit (read back from its key), so the list comes out in
// descending logit order.  The weights are the softmax of the k chosen logits
// in float32: e_r = exp(l_r - l_0), divided by their sum, taken over a fixed
// tree (the same bits on every run and in every lane).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {
namespace router {

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

// Token logits lg[0 .. e) (e <= 64 PER, k <= min(64, e)): lanes r < k get
// (id, weight) of round r; other lanes get (0, 0).
template <int PER>
__device__ __forceinline__ void topk_softmax_wave(const float *lg, int e, int k, int &out_id,
                                                  float &out_w) {
  const int lane = (int)(threadIdx.x & 63);
  uint32_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = lane + 64 * j;
    key[j] = i < e ? order_key(lg[i]) : 0u;  // 0: below every finite key
  }
  uint64_t taken = 0;
  int my_id = 0;
  float my_logit = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0;  // (key << 32) | (0xFFFFFFFF - index); 0: none
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = lane + 64 * j;
      const uint64_t c = ((uint64_t)key[j] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
      if (i < e && !((taken >> j) & 1ull) && c > best) best = c;
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
  const float e_ = lane < k ? expf(my_logit - top) : 0.0f;
  // sum: a fixed tree (rows of 16 by DPP, then the four rows), the same in
  // every lane and on every run
  float rs = dpp_add<kDppQuadXor1>(e_);
  rs = dpp_add<kDppQuadXor2>(rs);
  rs = dpp_add<kDppHalfMirror>(rs);
  rs = dpp_add<kDppMirror>(rs);
  float r4[4];
#pragma unroll
  for (int row = 0; row < 4; ++row)
    r4[row] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rs), 16 * row));
  const float sum = (r4[0] + r4[1]) + (r4[2] + r4[3]);
  out_id = lane < k ? my_id : 0;
  out_w = lane < k ? e_ / sum : 0.0f;
}

}  // namespace router
}  // namespace qmm
