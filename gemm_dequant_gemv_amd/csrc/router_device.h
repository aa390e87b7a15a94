// The router's top-k and softmax for one token, computed by one wave; shared
// by the router kernel (router.hip) and the decode-form gate/up launch that
// folds the router in (moe_gemv.hip), so both give the same bits.
//
// Lane l holds the logits l, l + 64, l + 128, ... of the token as order keys
// (a float32 mapped to a uint32 whose unsigned order is the float order, -0
// taken as +0).  Each of the k rounds finds the largest key not yet taken:
// every lane its own maximum, then the maximum across the wave (DPP inside
// each row of 16 lanes, then the four rows); the lowest index holding it
// (ballots over the lane's keys in index order), so equal logits go to the
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

// the larger of v and the value DPP brings from another lane of its row of 16
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
  return o > v ? o : v;
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
  // live keys: taken or absent ones are 0, below every finite key
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (lane + 64 * j >= e) key[j] = 0u;
  int my_id = 0;
  float my_logit = 0.0f;
  for (int r = 0; r < k; ++r) {
    // the largest live key: each lane's, then inside each row of 16 (DPP),
    // then over the four rows (uniform)
    uint32_t mx = key[0];
#pragma unroll
    for (int j = 1; j < PER; ++j) mx = key[j] > mx ? key[j] : mx;
    mx = dpp_max_u32<kDppQuadXor1>(mx);
    mx = dpp_max_u32<kDppQuadXor2>(mx);
    mx = dpp_max_u32<kDppHalfMirror>(mx);
    mx = dpp_max_u32<kDppMirror>(mx);
    uint32_t kw = (uint32_t)__builtin_amdgcn_readlane((int)mx, 0);
#pragma unroll
    for (int row = 1; row < 4; ++row) {
      const uint32_t h = (uint32_t)__builtin_amdgcn_readlane((int)mx, 16 * row);
      kw = h > kw ? h : kw;
    }
    // the lowest index holding it (index = lane + 64 j: the first j with a
    // lane at kw, its lowest such lane), so equal logits go to the lower id
    int win = 0;
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {
      const uint64_t b = __ballot(key[j] == kw);
      if (b != 0ull) win = 64 * j + (int)__builtin_ctzll(b);
    }
    const int wj = win >> 6, wl = win & 63;  // uniform
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (j == wj && lane == wl) key[j] = 0u;
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
