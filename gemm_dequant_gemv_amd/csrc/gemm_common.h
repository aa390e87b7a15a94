// Pieces of the GEMM kernels: the argument block, the 32-weight piece loads
// and their decode to bfloat16 pairs.
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
  int n_begin;         // dense: first weight row (output column) of the launch's tiles
  float *partials;     // [splits][m][n]
  uint32_t *counters;  // [tiles], cleared ahead of each split launch
  int wrows;                     // rows of the weight planes (all experts)
  // grouped (MoE) modes
  const uint32_t *tiles;         // [max_tiles][3] = (expert, first grouped row, rows)
  const uint32_t *n_tiles;       // device count of valid tiles
  const uint32_t *token_of_row;  // grouped row -> token (gate/up gather)
  const uint32_t *slot_of_row;   // grouped row -> token slot = row of d (down)
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

// Per-piece scale terms of decode_part, computed once per piece.
struct PieceScale {
  float a, b;  // affine: scale, bias; MXFP4: scale; NVFP4: the two block scales; Q6_K: d
};

template <int FMT>
__device__ __forceinline__ PieceScale piece_scale(const Piece &p) {
  if constexpr (FMT == QMM_AFFINE4_G64) {
    return {half_to_float(p.s & 0xFFFFu), half_to_float(p.s >> 16)};
  } else if constexpr (FMT == QMM_MXFP4) {
    return {e8m0_to_float(p.s), 0.0f};
  } else if constexpr (FMT == QMM_NVFP4) {
    PieceScale r;
    e4m3x2_to_float(p.s, r.a, r.b);
    return r;
  } else {
    return {half_to_float(p.d), 0.0f};
  }
}

// Weights 8j + 2i and 8j + 2i + 1 of the piece (code word j) as one bf16
// pair.
template <int FMT>
__device__ __forceinline__ uint32_t decode_word(const Piece &p, const PieceScale &sc, int j, int i) {
  const uint32_t w = p.q[j];
  if constexpr (FMT == QMM_AFFINE4_G64) {
    // even codes to the bytes of one word, odd codes to the bytes of another,
    // so that each code becomes a float with one v_cvt_f32_ubyteN (the empty
    // asm keeps the compiler from folding the mask into a bit-field extract
    // per code)
    uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;
    asm("" : "+v"(ev));
    asm("" : "+v"(od));
    const float lo = __builtin_fmaf(sc.a, (float)((ev >> (8 * i)) & 0xFFu), sc.b);
    const float hi = __builtin_fmaf(sc.a, (float)((od >> (8 * i)) & 0xFFu), sc.b);
    return pack_bf16(lo, hi);
  } else if constexpr (FMT == QMM_MXFP4) {
    // the conversions take the byte index as an immediate
    switch (i) {
      case 0: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc.a, 0));
      case 1: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc.a, 1));
      case 2: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc.a, 2));
      default: return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc.a, 3));
    }
  } else if constexpr (FMT == QMM_NVFP4) {
    const float bs = j < 2 ? sc.a : sc.b;
    // E2M1 pair -> two float32 (hardware conversion, unit scale), times the
    // E4M3 block scale (exact), -> bfloat16 pair (exact)
    const f32x2_t e = i == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0)
                    : i == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1)
                    : i == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2)
                             : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    return pack_bf16(e[0] * bs, e[1] * bs);
  } else {  // Q6_K
    const uint32_t hw[2] = {p.h.x, p.h.y};
    const float dsc = sc.a * (float)(int8_t)(p.s >> (8 * (j / 2)));
    const int v0 = 8 * j + 2 * i;  // value index within the piece (even)
    const uint32_t q0 = ((w >> (8 * i)) & 15u) | (((hw[v0 / 16] >> (2 * (v0 % 16))) & 3u) << 4);
    const uint32_t q1 = ((w >> (8 * i + 4)) & 15u) |
                        (((hw[(v0 + 1) / 16] >> (2 * ((v0 + 1) % 16))) & 3u) << 4);
    return pack_bf16(dsc * (float)((int)q0 - 32), dsc * (float)((int)q1 - 32));
  }
}

// Weights 8j .. 8j+7 of the piece (code word j) as 4 bf16 pairs in natural
// order.
template <int FMT>
__device__ __forceinline__ void decode_part(const Piece &p, const PieceScale &sc, int j,
                                            uint32_t (&o)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = decode_word<FMT>(p, sc, j, i);
}

// The piece's 32 weights as 16 bf16 pairs in natural order.
template <int FMT>
__device__ __forceinline__ void decode_piece(const Piece &p, uint32_t (&o)[16]) {
  const PieceScale sc = piece_scale<FMT>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t t[4];
    decode_part<FMT>(p, sc, j, t);
#pragma unroll
    for (int i = 0; i < 4; ++i) o[4 * j + i] = t[i];
  }
}

}  // namespace gemm
}  // namespace qmm
