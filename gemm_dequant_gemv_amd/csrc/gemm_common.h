// Pieces shared by the two GEMM kernels: the argument block, the 32-weight
// piece loads and their decode to bfloat16 pairs.
#pragma once

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace gemm {

constexpr int kBK = 64;          // K values per slice
constexpr int kLdsPad = 8;       // bf16 of padding per LDS row (keeps MFMA operand reads conflict-free)
constexpr int kRowH = kBK + kLdsPad;  // bf16 per LDS row

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// What a workgroup's rows are, and where its results go.
enum GemmMode {
  kDense = 0,   // y[m][n] = x[m] . w[n]; rows of x are rows of y
  kMoeGateUp = 1,  // grouped: x rows gathered by token, weight rows interleaved
                   // (gate i, up i); the epilogue applies SwiGLU and writes bf16 h
  kMoeDown = 2,    // grouped: rows of h, one expert per tile; writes float32 d
};

struct GemmArgs {
  const uint8_t *codes;
  const uint8_t *codes_hi;
  const uint8_t *scales;
  const uint8_t *scales2;
  const float *tensor_scale;
  const uint16_t *x;
  const uint16_t *residual;
  uint16_t *y;
  int m, n, k;
  // dense split-K: workgroup (tile, split) sums slices [split * sps, ...) and
  // leaves float32 partials; the last of a tile's splits adds them in order
  int splits, sps;
  float *partials;     // [splits][m][n]
  uint32_t *counters;  // [tiles], zero between calls
  int wrows;                     // rows of the weight planes (all experts)
  // grouped (MoE) modes
  const uint32_t *tiles;         // [max_tiles][3] = (expert, first grouped row, rows)
  const uint32_t *n_tiles;       // device count of valid tiles
  const uint32_t *token_of_row;  // grouped row -> token (gate/up gather)
  uint16_t *h;                   // bf16 [rows][inter]   (gate/up output, down input)
  float *d;                      // float32 [rows][n]    (down output)
  int inter;                     // I: gate/up rows are 2I
};

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2v_t;

// Two floats -> a bfloat16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2v_t));
}

// Raw bytes of one 32-weight piece of a row (codes and scales).
struct Piece {
  u32x4_t q;
  uint2 h;
  uint32_t s, d;
};

template <int FMT>
__device__ __forceinline__ Piece load_piece(const GemmArgs &a, int row, int kc) {
  const size_t k = (size_t)a.k, r = (size_t)row;
  Piece p;
  p.q = __builtin_nontemporal_load((const u32x4_t *)(a.codes + r * (k / 2) + kc / 2));
  if constexpr (FMT == QMM_AFFINE4_G64) {
    p.s = *(const uint32_t *)(a.scales + (r * (k / 64) + kc / 64) * 4);
  } else if constexpr (FMT == QMM_MXFP4) {
    p.s = a.scales[r * (k / 32) + kc / 32];
  } else if constexpr (FMT == QMM_NVFP4) {
    p.s = *(const uint16_t *)(a.scales + r * (k / 16) + kc / 16);
  } else {
    p.h = *(const uint2 *)(a.codes_hi + r * (k / 4) + kc / 4);
    p.s = *(const uint16_t *)(a.scales + r * (k / 16) + kc / 16);
    p.d = *(const uint16_t *)(a.scales2 + (r * (k / 256) + kc / 256) * 2);
  }
  return p;
}

// The piece's 32 weights as 16 bf16 pairs in natural order.
template <int FMT>
__device__ __forceinline__ void decode_piece(const Piece &p, uint32_t (&o)[16]) {
  const uint32_t w[4] = {p.q[0], p.q[1], p.q[2], p.q[3]};
  if constexpr (FMT == QMM_AFFINE4_G64) {
    const float s = half_to_float(p.s & 0xFFFFu), b = half_to_float(p.s >> 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // even codes to the bytes of one word, odd codes to the bytes of another,
      // so that each code becomes a float with one v_cvt_f32_ubyteN (the
      // empty asm keeps the compiler from folding the mask into a bit-field
      // extract per code)
      uint32_t ev = w[j] & 0x0F0F0F0Fu, od = (w[j] >> 4) & 0x0F0F0F0Fu;
      asm volatile("" : "+v"(ev));
      asm volatile("" : "+v"(od));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __builtin_fmaf(s, (float)((ev >> (8 * i)) & 0xFFu), b);
        const float hi = __builtin_fmaf(s, (float)((od >> (8 * i)) & 0xFFu), b);
        o[4 * j + i] = pack_bf16(lo, hi);
      }
    }
  } else if constexpr (FMT == QMM_MXFP4) {
    const float sc = e8m0_to_float(p.s);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[4 * j + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 0));
      o[4 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 1));
      o[4 * j + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 2));
      o[4 * j + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 3));
    }
  } else if constexpr (FMT == QMM_NVFP4) {
    float s0, s1;
    e4m3x2_to_float(p.s, s0, s1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float sc = j < 2 ? s0 : s1;
      // E2M1 pair -> two float32 (hardware conversion, unit scale), times the
      // E4M3 block scale (exact), -> bfloat16 pair (exact)
      const f32x2_t e[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 0),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 1),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 2),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 3)};
#pragma unroll
      for (int i = 0; i < 4; ++i) o[4 * j + i] = pack_bf16(e[i][0] * sc, e[i][1] * sc);
    }
  } else {  // Q6_K
    const float dd = half_to_float(p.d);
    const uint32_t hw[2] = {p.h.x, p.h.y};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float dsc = dd * (float)(int8_t)(p.s >> (8 * (j / 2)));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v0 = 8 * j + 2 * i;  // value index within the piece (even)
        const uint32_t q0 = ((w[j] >> (8 * i)) & 15u) | (((hw[v0 / 16] >> (2 * (v0 % 16))) & 3u) << 4);
        const uint32_t q1 = ((w[j] >> (8 * i + 4)) & 15u) |
                            (((hw[(v0 + 1) / 16] >> (2 * ((v0 + 1) % 16))) & 3u) << 4);
        o[4 * j + i] = pack_bf16(dsc * (float)((int)q0 - 32), dsc * (float)((int)q1 - 32));
      }
    }
  }
}

}  // namespace gemm
}  // namespace qmm
