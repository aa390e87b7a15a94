// Per-lane arithmetic shared by the two GEMV kernels: one row's 32 weights
// (16 code bytes, plus their scales) against the matching 32 activations of
// each of the M lanes, accumulated in float32.
#pragma once

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

template <int FMT>
struct FmtTraits {
  // sums of x kept per 32-value chunk: affine 1 (per chunk), Q6_K 2 (per
  // 16-value sub-block), E2M1 formats none.
  static constexpr int kSums = FMT == QMM_AFFINE4_G64 ? 1 : (FMT == QMM_Q6_K ? 2 : 0);
  // activations staged in (i, i+4) pair order for the nibble-into-mantissa
  // unpack, natural pair order for the hardware FP4 conversion.
  static constexpr bool kPermute = FMT == QMM_AFFINE4_G64 || FMT == QMM_Q6_K;
  // K values per byte of the `scales` plane
  static constexpr int kKPerScaleByte = FMT == QMM_MXFP4 ? 32 : 16;
};


// One row's data for one step.
struct RowData {
  uint4 q;      // 32 codes (Q6_K: low nibbles)
  uint2 h;      // Q6_K high bits
  uint32_t s;   // affine (scale, bias) / E8M0 / two E4M3 / two int8 sc
  uint32_t d;   // Q6_K super-block scale
};

// The nibble-into-mantissa unpack: two 4-bit codes at bits 4p and 4p + 16 of
// a word of eight become the bfloat16 pair (128 + q_p, 128 + q_{p+4}) by
// landing in the low mantissa bits of 128.0 (0x4300), with no conversion
// instruction.  Its constants are held in registers: gfx9 VOP3
// instructions take no literal operand, so with the masks in an SGPR and the
// bfloat16 128.0 pair in a VGPR each (v, v+4) pair is one v_and_or_b32 (plus
// a shift) instead of a shift, an and and an or.
struct UnpackK {
  uint32_t lo;     // 0x000F000F
  uint32_t hi;     // 0x00300030
  uint32_t magic;  // 0x43004300: bfloat16 128.0 in both halves
};

__device__ __forceinline__ UnpackK unpack_consts() {
  UnpackK k{0x000F000Fu, 0x00300030u, 0x43004300u};
  asm volatile("" : "+s"(k.lo));
  asm volatile("" : "+s"(k.hi));
  asm volatile("" : "+v"(k.magic));
  return k;
}

// (a & mask) | b as one v_and_or_b32 (left to itself the compiler turns the
// nested Q6_K form into two ands and an or3)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t b) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(b));
  return r;
}

// acc[m] += (this row's 32 weights of the chunk) . (x[m] chunk)
template <int FMT, int M>
__device__ __forceinline__ void row_step(const RowData &rd, const uint32_t (&X)[M][16],
                                         const float (&S)[M][2], float (&acc)[M],
                                         const UnpackK &K) {
  const uint32_t w[4] = {rd.q.x, rd.q.y, rd.q.z, rd.q.w};
  if constexpr (FMT == QMM_AFFINE4_G64) {
    const float s = half_to_float(rd.s & 0xFFFFu), b = half_to_float(rd.s >> 16);
    float d[M];
#pragma unroll
    for (int m = 0; m < M; ++m) d[m] = -128.0f * S[m][0];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t p0 = and_or(w[j], K.lo, K.magic), p1 = and_or(w[j] >> 4, K.lo, K.magic);
      const uint32_t p2 = and_or(w[j] >> 8, K.lo, K.magic), p3 = and_or(w[j] >> 12, K.lo, K.magic);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        d[m] = dot2(p0, X[m][4 * j + 0], d[m]);
        d[m] = dot2(p1, X[m][4 * j + 1], d[m]);
        d[m] = dot2(p2, X[m][4 * j + 2], d[m]);
        d[m] = dot2(p3, X[m][4 * j + 3], d[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      acc[m] = __builtin_fmaf(s, d[m], acc[m]);
      acc[m] = __builtin_fmaf(b, S[m][0], acc[m]);
    }
  } else if constexpr (FMT == QMM_MXFP4 || FMT == QMM_NVFP4) {
    float d0[M], d1[M];
#pragma unroll
    for (int m = 0; m < M; ++m) d0[m] = d1[m] = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t p0 = e2m1x2_to_bf16x2<0>(w[j]), p1 = e2m1x2_to_bf16x2<1>(w[j]);
      const uint32_t p2 = e2m1x2_to_bf16x2<2>(w[j]), p3 = e2m1x2_to_bf16x2<3>(w[j]);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float &d = (FMT == QMM_NVFP4 && j >= 2) ? d1[m] : d0[m];
        d = dot2(p0, X[m][4 * j + 0], d);
        d = dot2(p1, X[m][4 * j + 1], d);
        d = dot2(p2, X[m][4 * j + 2], d);
        d = dot2(p3, X[m][4 * j + 3], d);
      }
    }
    if constexpr (FMT == QMM_MXFP4) {
      const float sc = e8m0_to_float(rd.s);
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = __builtin_fmaf(sc, d0[m], acc[m]);
    } else {
      float s0, s1;
      e4m3x2_to_float(rd.s, s0, s1);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        acc[m] = __builtin_fmaf(s0, d0[m], acc[m]);
        acc[m] = __builtin_fmaf(s1, d1[m], acc[m]);
      }
    }
  } else {  // Q6_K
    const float dd = half_to_float(rd.d);
    const uint32_t hw[2] = {rd.h.x, rd.h.y};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t A = w[2 * j], B = w[2 * j + 1];
      // high-bit bytes reordered to (values 0-3, 8-11, 4-7, 12-15) so that one
      // shift puts the high bits of a (v, v+4) pair at bits 4-5 and 20-21.
      const uint32_t H = __builtin_amdgcn_perm(hw[j], hw[j], 0x03010200u);
      const uint32_t a0 = and_or(H << 4, K.hi, and_or(A, K.lo, K.magic));
      const uint32_t a1 = and_or(H << 2, K.hi, and_or(A >> 4, K.lo, K.magic));
      const uint32_t a2 = and_or(H, K.hi, and_or(A >> 8, K.lo, K.magic));
      const uint32_t a3 = and_or(H >> 2, K.hi, and_or(A >> 12, K.lo, K.magic));
      const uint32_t b0 = and_or(H >> 4, K.hi, and_or(B, K.lo, K.magic));
      const uint32_t b1 = and_or(H >> 6, K.hi, and_or(B >> 4, K.lo, K.magic));
      const uint32_t b2 = and_or(H >> 8, K.hi, and_or(B >> 8, K.lo, K.magic));
      const uint32_t b3 = and_or(H >> 10, K.hi, and_or(B >> 12, K.lo, K.magic));
      const float dsc = dd * (float)(int8_t)(rd.s >> (8 * j));
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float d = -160.0f * S[m][j];
        d = dot2(a0, X[m][8 * j + 0], d);
        d = dot2(a1, X[m][8 * j + 1], d);
        d = dot2(a2, X[m][8 * j + 2], d);
        d = dot2(a3, X[m][8 * j + 3], d);
        d = dot2(b0, X[m][8 * j + 4], d);
        d = dot2(b1, X[m][8 * j + 5], d);
        d = dot2(b2, X[m][8 * j + 6], d);
        d = dot2(b3, X[m][8 * j + 7], d);
        acc[m] = __builtin_fmaf(dsc, d, acc[m]);
      }
    }
  }
}

// ---- the matrix-core form for 2 to 8 activation rows

// A row's 32 weights as 16 bfloat16 pairs, in the order row_step multiplies
// them: pair p meets activation word p of the chunk (affine and Q6_K: 128 +
// q, the zero points left to the caller; E2M1: the exact values).
template <int FMT>
__device__ __forceinline__ void unpack_pairs(const RowData &rd, uint32_t (&P)[16],
                                             const UnpackK &K) {
  const uint32_t w[4] = {rd.q.x, rd.q.y, rd.q.z, rd.q.w};
  if constexpr (FMT == QMM_AFFINE4_G64) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      P[4 * j + 0] = and_or(w[j], K.lo, K.magic);
      P[4 * j + 1] = and_or(w[j] >> 4, K.lo, K.magic);
      P[4 * j + 2] = and_or(w[j] >> 8, K.lo, K.magic);
      P[4 * j + 3] = and_or(w[j] >> 12, K.lo, K.magic);
    }
  } else if constexpr (FMT == QMM_MXFP4 || FMT == QMM_NVFP4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      P[4 * j + 0] = e2m1x2_to_bf16x2<0>(w[j]);
      P[4 * j + 1] = e2m1x2_to_bf16x2<1>(w[j]);
      P[4 * j + 2] = e2m1x2_to_bf16x2<2>(w[j]);
      P[4 * j + 3] = e2m1x2_to_bf16x2<3>(w[j]);
    }
  } else {  // Q6_K
    const uint32_t hw[2] = {rd.h.x, rd.h.y};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t A = w[2 * j], B = w[2 * j + 1];
      const uint32_t H = __builtin_amdgcn_perm(hw[j], hw[j], 0x03010200u);
      P[8 * j + 0] = and_or(H << 4, K.hi, and_or(A, K.lo, K.magic));
      P[8 * j + 1] = and_or(H << 2, K.hi, and_or(A >> 4, K.lo, K.magic));
      P[8 * j + 2] = and_or(H, K.hi, and_or(A >> 8, K.lo, K.magic));
      P[8 * j + 3] = and_or(H >> 2, K.hi, and_or(A >> 12, K.lo, K.magic));
      P[8 * j + 4] = and_or(H >> 4, K.hi, and_or(B, K.lo, K.magic));
      P[8 * j + 5] = and_or(H >> 6, K.hi, and_or(B >> 4, K.lo, K.magic));
      P[8 * j + 6] = and_or(H >> 8, K.hi, and_or(B >> 8, K.lo, K.magic));
      P[8 * j + 7] = and_or(H >> 10, K.hi, and_or(B >> 12, K.lo, K.magic));
    }
  }
}

typedef short mf_v4s_t __attribute__((ext_vector_type(4)));
typedef float mf_v4f_t __attribute__((ext_vector_type(4)));

// One v_mfma_f32_4x4x4_16b_bf16: 16 independent 4 x 4 x 4 products, block b
// in lanes 4b .. 4b+3.  Lane 4b+i supplies row i of A (4 bfloat16: words a0,
// a1) and column i of B (words b0, b1); lane 4b+j receives column j of D,
// D[i] in element i.  (Layout checked on the GPU against a CPU product.)
__device__ __forceinline__ mf_v4f_t mfma4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                          mf_v4f_t c) {
  const mf_v4s_t A = __builtin_bit_cast(mf_v4s_t, make_uint2(a0, a1));
  const mf_v4s_t B = __builtin_bit_cast(mf_v4s_t, make_uint2(b0, b1));
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(A, B, c, 0, 0, 0);
}

// x moved within each group of four lanes by a DPP quad permutation
template <int CTRL>
__device__ __forceinline__ float quad_perm(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// v + (v moved by one DPP pattern): quad permutations, half-row and row
// mirrors, row broadcasts of lane 15 and lane 31 (rows without the mask bit
// add zero).
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  int r;
  switch (ctrl_sel) {
    case 0: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false); break;
    case 1: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false); break;
    case 3: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false); break;
  }
  return v + __builtin_bit_cast(float, r);
}

// Sums over each quarter-wave (16-lane DPP row), returned uniform: the quad,
// half-row and row mirrors give every lane its row's sum.
__device__ __forceinline__ void quarter_sums(float v, float (&s)[4]) {
  v = dpp_add(v, 0);  // quad_perm [1,0,3,2]
  v = dpp_add(v, 1);  // quad_perm [2,3,0,1]
  v = dpp_add(v, 2);  // row_half_mirror
  v = dpp_add(v, 3);  // row_mirror
#pragma unroll
  for (int r = 0; r < 4; ++r)
    s[r] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16 * r + 15));
}

// Sums over each half-wave (lanes 0-31 and 32-63), returned uniform: DPP
// quad, half-row and row mirrors give every lane its row's sum, and a row
// broadcast adds row 0 into row 1 and row 2 into row 3.
__device__ __forceinline__ void half_sums(float v, float &s0, float &s1) {
  v = dpp_add(v, 0);  // quad_perm [1,0,3,2]
  v = dpp_add(v, 1);  // quad_perm [2,3,0,1]
  v = dpp_add(v, 2);  // row_half_mirror
  v = dpp_add(v, 3);  // row_mirror
  v = dpp_add(v, 4);  // row_bcast:15 into rows 1 and 3
  s0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
  s1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

}  // namespace qmm
