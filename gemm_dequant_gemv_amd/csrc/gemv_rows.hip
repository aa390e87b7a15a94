// qgemv, row-streaming form: decode matrix-vector products for 1-4 activation
// rows (and qgemm's 5-8), weights dequantized in registers ("TurboEXL3"
// section 2.2: W4A16, each weight expanded to 16 bits in the kernel, 16-bit
// products, 32-bit sums).  The products are v_dot2 per activation row for 1,
// 2 (and 5) rows, and the matrix cores' 4 x 4 x 4 form for more (below).
//
// One workgroup of 16 waves (8 for 5-8 rows) per compute unit.  The workgroup first stages the
// whole activation block x [M][K] in LDS (one padded record per 32-value
// chunk: its x in pair order, then its block sums), then its waves stream
// weight rows:
//   * rows go in pairs (2p, 2p+1), one per half-wave, dealt out in one of two
//     ways: round-robin, in rounds of W pairs (W = waves in the grid, 16 G
//     for G workgroups): in round r wave w of workgroup g owns pair
//     r W + 16 g + w, so that the grid streams one contiguous band of rows
//     and a workgroup's waves neighbouring pairs, except in the last, partial
//     round, where it owns pair r W + w G + g (wave-major: every workgroup
//     gets its share of that round, give or take one pair); or balanced,
//     where workgroup g owns the contiguous pairs [g P / G, (g+1) P / G) (P
//     pairs) and splits their units (below), pair-major, evenly over its
//     waves (the form for fewer pairs than waves and long rows);
//   * a unit is one step of one pair: 1024 values (512 code bytes) of each
//     row, one 16-byte load per lane (lane c of a half holds values 32c ..
//     32c+31), so every load instruction reads whole 128-byte lines of two
//     rows, and K = 5120 or 17408 is a whole number of steps;
//   * every load address is a per-lane constant (the lane's half and chunk)
//     plus a wave-uniform offset (pair and step) passed in the buffer
//     instruction's scalar offset, so addressing costs no vector ALU work;
//   * a wave's units form one software pipeline with U units of loads in
//     flight; each unit brings the codes of two rows, their block scales and
//     one residual value per output;
//   * when a wave is done with a pair, each half-wave's sums are reduced with
//     DPP row operations and lanes 0 .. 2M-1 write the pair's 2 x M outputs;
//     in the balanced form a pair cut by a wave boundary leaves its sums in an
//     LDS slot instead, and after the last barrier the wave that did the
//     pair's last step adds the slots in wave order and writes the outputs;
//   * a wave lowers its issue priority at each quarter of its units, so that
//     the waves sharing a SIMD progress together instead of oldest first.
// Nothing crosses workgroups, so there is no split-K finish and no workspace,
// and every sum has a fixed order: the result does not depend on timing.
//
// The waves of a workgroup need not end together: the compute unit's memory
// throughput sets the pace, and a copy of the kernel that handed out units
// to the waves at run time (chunks of 4 from an LDS counter, sums kept per
// chunk and added in chunk order) so that they all ended within a chunk of
// each other was 1-12% slower on every decode shape.  What matters is that
// every workgroup gets the same work, which the wave-major last round gives.
//
// The activations must fit in LDS (K * M * 2 bytes plus block sums); the host
// falls back to the split-K kernel otherwise.
#include <algorithm>
#include <atomic>
#include <cstdlib>

#include "gemv_step.h"

namespace qmm {
namespace {

constexpr int kStepK = 1024;       // values of one row per step (32 lanes x 32)

// Waves per workgroup (one workgroup per compute unit) and the 16-byte
// activation pieces each thread stages at most.  Up to 4 activation rows: 16
// waves (at most 128 registers each); 5 to 8 rows: 8 waves, so that a wave
// can hold the 8 x 32 activation values of a unit (256 registers each).
template <int M>
struct RowsShape {
  static constexpr int kWaves = M <= 4 ? 16 : 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kXPieces = M <= 4 ? 9 : 18;
};
constexpr size_t kLdsLimit = 160 * 1024 - 2048;  // dynamic part; the static part is <= 1 KB

// Where the matrix-core form runs (below).  Measured against the v_dot2 form
// on the decode shapes (cold weights, events around 4 x copies launches, two
// runs): 4 rows 6-17% faster, 3 rows 0-6%, 6-8 rows (17408 x 5120) 5-27%;
// 2 rows 0-4% slower (half of each product's columns idle against 32 v_dot2
// per unit), 5 rows 3-6% slower for affine and NVFP4 (5 of 8 columns used)
// and 2-4% faster for Q6_K.
constexpr bool use_mfma(int format, int m) {
  return m >= 3 && (m != 5 || format == QMM_Q6_K);
}

template <int M>
struct MfShape {
  static constexpr int kG = M <= 2 ? 1 : (M + 3) / 4;  // groups of 4 activation rows
  static constexpr int kH = M <= 2 ? 1 : 2;            // chunk halves per lane
};

// LDS image of the activations, one record per 32-value chunk: the chunk's
// x (16-byte pieces, in pair order for the nibble-into-mantissa formats),
// then its block sums of x (M x NS floats), then padding.
//   v_dot2 form: row m's four pieces at 64 m + 16 q; the 8 lanes of one
//     ds_read_b128 group read consecutive records at the same offset, and a
//     stride that is an odd multiple of 16 bytes sends them to 8 distinct
//     groups of 4 banks.
//   matrix-core form: piece q of row 4g + j at 256 g + 64 q + 16 j
//     (piece-major within each group of 4 rows), stride 16 (4k + 2) bytes.
//     Lanes 4b + j read piece q of row 4g + j of record 2b (+ h): within 16
//     lanes the records add 0, 4, 8, 12 (mod 16) 16-byte units and j adds
//     0-3, and within 8 lanes 0 and 4 (mod 8): distinct bank groups under
//     either grouping.  (Row-major pieces at that stride measured 2-4-way
//     conflicts.)
// Every read of a unit is one lane base plus an immediate offset.
constexpr int record_pad(int m, int ns) {
  return m * ns * 4 <= 16 ? 16 : m * ns * 4 <= 48 ? 48 : m * ns * 4 <= 80 ? 80 : 112;
}
constexpr int mf_stride(int bytes) {
  int u = (bytes + 15) / 16;
  while (u % 4 != 2) ++u;
  return 16 * u;
}

template <int M, int NS, bool MFL>
struct XLayout {
  static constexpr int kXBytes = MFL ? 256 * MfShape<M>::kG : 64 * M;
  static constexpr int kSumOff = kXBytes;  // bytes
  static constexpr int kStride = MFL ? mf_stride(kXBytes + M * NS * 4) : 64 * M + record_pad(M, NS);
  static constexpr int piece(int m, int q) {
    return MFL ? 256 * (m / 4) + 64 * q + 16 * (m % 4) : 64 * m + 16 * q;
  }
  static_assert(kSumOff + M * NS * 4 <= kStride, "record layout");
  static_assert(MFL ? (kStride / 16) % 4 == 2 : (kStride / 16) % 2 == 1, "record stride");
};

// How the waves share the rows (above): round-robin pairs, or each
// workgroup's units split evenly over its waves.
constexpr int kSplitRR = 0, kSplitBal = 1;

constexpr int sums_per_chunk(int format) {
  return format == QMM_AFFINE4_G64 ? 1 : (format == QMM_Q6_K ? 2 : 0);
}

struct RowsArgs {
  const uint8_t *codes;
  const uint8_t *codes_hi;
  const uint8_t *scales;
  const uint8_t *scales2;
  const float *tensor_scale;
  const uint16_t *x;
  const uint16_t *residual;
  void *y;
  uint32_t codes_bytes, hi_bytes, scales_bytes, scales2_bytes, residual_bytes;
  int n, k, steps, y_bf16;
};

// ---- the matrix-core form (2 to 8 activation rows)
//
// v_mfma_f32_4x4x4_16b_bf16 runs 16 independent 4 x 4 x 4 products, block b
// in lanes 4b .. 4b+3.  Lane 4b + i loads row (i >> 1) of the pair at chunk
// 2b + (i & 1) of the step (the same 2 x 512 contiguous bytes per load
// instruction as the scalar form) and supplies that row's weights as row i
// of A; as column i of B it supplies activations: for M = 2 row (i & 1) of x
// at chunk 2b + (i >> 1), for M >= 3 row 4g + i at chunk 2b + h, one product
// per (h, g).  An entry D[i][j] is a useful partial sum where A's chunk is
// B's chunk (half of them); lane 4b + j receives column j, so it holds its
// activation row's partial sums for both weight rows.  Per k-step of 4
// values a lane issues 1 (M = 2), 2 (M = 3, 4) or 4 (M = 5..8) products
// instead of 2, 4 or 8 v_dot2 per activation row, and reads from LDS only
// its own activation row's 64 bytes per chunk instead of every row's.  The
// block scales are applied per chunk in float32 after the product, taken
// from the loading lane by DPP quad permutations.
constexpr int kXSlack = 256;  // LDS bytes after the last record (reads of rows past M)

// The scale terms of the lane's own (row, chunk): affine (s, b - 128 s),
// MXFP4 (scale, -), NVFP4 (s0, s1), Q6_K (d sc0, d sc1).
template <int FMT>
__device__ __forceinline__ void mf_scales(const RowData &rd, float &t0, float &t1) {
  if constexpr (FMT == QMM_AFFINE4_G64) {
    t0 = half_to_float(rd.s & 0xFFFFu);
    t1 = __builtin_fmaf(-128.0f, t0, half_to_float(rd.s >> 16));
  } else if constexpr (FMT == QMM_MXFP4) {
    t0 = e8m0_to_float(rd.s);
    t1 = 0.0f;
  } else if constexpr (FMT == QMM_NVFP4) {
    e4m3x2_to_float(rd.s, t0, t1);
  } else {
    const float dd = half_to_float(rd.d);
    t0 = dd * (float)(int8_t)(rd.s & 0xFFu);
    t1 = dd * (float)(int8_t)((rd.s >> 8) & 0xFFu);
  }
}

// acc += the chunk's partial sum of one weight row: D0 (and D1, the second
// 16-value sub-block or the odd k-steps) scaled by the row's terms t0, t1,
// with the block sums Sx0, Sx1 of the activation row for the zero points.
template <int FMT>
__device__ __forceinline__ float mf_apply(float acc, float d0, float d1, float t0, float t1,
                                          float sx0, float sx1) {
  if constexpr (FMT == QMM_AFFINE4_G64) {
    acc = __builtin_fmaf(t0, d0 + d1, acc);
    return __builtin_fmaf(t1, sx0, acc);
  } else if constexpr (FMT == QMM_MXFP4) {
    return __builtin_fmaf(t0, d0 + d1, acc);
  } else if constexpr (FMT == QMM_NVFP4) {
    acc = __builtin_fmaf(t0, d0, acc);
    return __builtin_fmaf(t1, d1, acc);
  } else {
    acc = __builtin_fmaf(t0, __builtin_fmaf(-160.0f, sx0, d0), acc);
    return __builtin_fmaf(t1, __builtin_fmaf(-160.0f, sx1, d1), acc);
  }
}

// One unit in the matrix-core form.  xb / sb: this lane's activation words
// and block sums in the unit's record (B role); P: the lane's unpacked
// weights (A role); t0, t1 its scale terms.
template <int FMT, int M, int STRIDE>
__device__ __forceinline__ void mf_unit(const uint32_t (&P)[16], float t0, float t1,
                                        const char *xb, const char *sb, int qi,
                                        float (&acc)[MfShape<M>::kG][2]) {
  using MS = MfShape<M>;
  constexpr bool kTwoSub = FMT == QMM_NVFP4 || FMT == QMM_Q6_K;
  constexpr int kNS = FmtTraits<FMT>::kSums;
#pragma unroll
  for (int h = 0; h < MS::kH; ++h) {
#pragma unroll
    for (int g = 0; g < MS::kG; ++g) {
      const char *xr = xb + h * STRIDE + g * 256;
      uint32_t X[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = *(const uint4 *)(xr + 64 * q);
        X[4 * q + 0] = v.x;
        X[4 * q + 1] = v.y;
        X[4 * q + 2] = v.z;
        X[4 * q + 3] = v.w;
      }
      float sx0 = 0.0f, sx1 = 0.0f;
      if constexpr (kNS > 0) {
        const float *sr = (const float *)(sb + h * STRIDE + g * 16 * kNS);
        sx0 = sr[0];
        if constexpr (kNS > 1) sx1 = sr[1];
      }
      // two chains: the sub-blocks (k-steps 0-3, 4-7), or even and odd k-steps
      mf_v4f_t D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int s0 = kTwoSub ? st : 2 * st, s1 = kTwoSub ? st + 4 : 2 * st + 1;
        D0 = mfma4(P[2 * s0], P[2 * s0 + 1], X[2 * s0], X[2 * s0 + 1], D0);
        D1 = mfma4(P[2 * s1], P[2 * s1 + 1], X[2 * s1], X[2 * s1 + 1], D1);
      }
      // useful entries: weight row r at this lane's chunk, D[2r + chunk half]
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        float d0, d1, a0, a1;
        if constexpr (M <= 2) {
          const bool odd = (qi >> 1) != 0;  // B chunk half of this lane
          d0 = odd ? D0[2 * r + 1] : D0[2 * r];
          d1 = odd ? D1[2 * r + 1] : D1[2 * r];
          a0 = r == 0 ? quad_perm<0x50>(t0) : quad_perm<0xFA>(t0);  // lanes [0,0,1,1] / [2,2,3,3]
          a1 = r == 0 ? quad_perm<0x50>(t1) : quad_perm<0xFA>(t1);
        } else {
          d0 = D0[2 * r + h];
          d1 = D1[2 * r + h];
          // the loading lane 2r + h of the quad
          constexpr int kC0 = 0x00, kC1 = 0x55, kC2 = 0xAA, kC3 = 0xFF;
          if (2 * r + h == 0) { a0 = quad_perm<kC0>(t0); a1 = quad_perm<kC0>(t1); }
          else if (2 * r + h == 1) { a0 = quad_perm<kC1>(t0); a1 = quad_perm<kC1>(t1); }
          else if (2 * r + h == 2) { a0 = quad_perm<kC2>(t0); a1 = quad_perm<kC2>(t1); }
          else { a0 = quad_perm<kC3>(t0); a1 = quad_perm<kC3>(t1); }
        }
        acc[g][r] = mf_apply<FMT>(acc[g][r], d0, d1, a0, a1, sx0, sx1);
      }
    }
  }
}

// v + v rotated by 4 or 8 lanes within each row of 16 (DPP row_ror)
template <int CTRL>
__device__ __forceinline__ float ror_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                           0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// A pair's outputs in the matrix-core form: each partial sum is added over
// its copies (the 16 blocks, and for M = 2 the two chunk halves of a quad)
// in a fixed order; lane 2m + r returns weight row r of activation row m.
template <int M>
__device__ __forceinline__ float mf_finish(float (&acc)[MfShape<M>::kG][2], int lane) {
  float out = 0.0f;
  const int m = lane >> 1, r_out = lane & 1;
#pragma unroll
  for (int g = 0; g < MfShape<M>::kG; ++g) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float v = acc[g][r];
      acc[g][r] = 0.0f;
      if constexpr (M <= 2) v += quad_perm<0x4E>(v);  // lanes [2,3,0,1]: the other half
      v = ror_add<0x124>(v);                          // row_ror:4
      v = ror_add<0x128>(v);                          // row_ror:8
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      // every lane at quad position j now holds the total of activation row
      // (M = 2: j & 1; else 4g + j)
      const float t = __shfl(v, M <= 2 ? (m & 1) : (m & 3));
      if (r_out == r && m < M && (M <= 2 || (m >> 2) == g)) out = t;
    }
  }
  return out;
}

template <int FMT, int M, int U, int SPLIT>
__global__ __launch_bounds__(RowsShape<M>::kThreads) void gemv_rows_kernel(RowsArgs a) {
  constexpr bool BAL = SPLIT == kSplitBal;
  constexpr int kWaves = RowsShape<M>::kWaves;
  constexpr int kThreads = RowsShape<M>::kThreads;
  constexpr int kXPieces = RowsShape<M>::kXPieces;
  using T = FmtTraits<FMT>;
  constexpr int kNS = T::kSums;
  constexpr bool MF = use_mfma(FMT, M);
  using XL = XLayout<M, kNS, MF>;
  static_assert(kNS == sums_per_chunk(FMT), "sums per chunk");
  constexpr int kChunks = kStepK / 32;  // chunks per step
  constexpr int kOut = 2 * M;           // outputs of one pair
  extern __shared__ __align__(16) uint32_t smem[];
  const int nch = a.k / 32;
  char *xs = (char *)smem;  // [nch] records of XL::kStride bytes

  const int tid = threadIdx.x;
  const int lane = tid & 63, hf = lane >> 5, c = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.steps;
  const uint32_t k = (uint32_t)a.k;
  // The wave walks its pairs pair_of(j) from j = j0, step st0, for `units`
  // units.
  const int npairs = (a.n + 1) / 2;
  int pbase, pstride, units, j0 = 0, st0 = 0, L = 0, rfull = 0, plast = 0;
  if constexpr (BAL) {
    // the workgroup's pairs [pbase, pbase + L / S) and their L units
    pbase = (int)((long long)blockIdx.x * npairs / gridDim.x);
    L = ((int)((long long)(blockIdx.x + 1) * npairs / gridDim.x) - pbase) * S;
    pstride = 1;
    const int u0 = wave * L / kWaves;
    units = (wave + 1) * L / kWaves - u0;
    j0 = u0 / S;
    st0 = u0 - j0 * S;
  } else {
    // round r < rfull: pair r W + 16 g + w of the grid's W = 16 G waves; the
    // last, partial round: pair rfull W + w G + g (wave-major), so that every
    // workgroup gets the same number of pairs give or take one
    pbase = blockIdx.x * kWaves + wave;
    pstride = gridDim.x * kWaves;
    rfull = npairs / pstride;
    plast = rfull * pstride + wave * (int)gridDim.x + (int)blockIdx.x;
    units = (rfull + (plast < npairs ? 1 : 0)) * S;
  }
  __shared__ float part[BAL ? kWaves : 1][2][kOut];  // sums of pairs cut by wave boundaries

  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes, a.codes_bytes);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.codes_hi, a.hi_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales, a.scales_bytes);
  const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(a.scales2, a.scales2_bytes);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.residual, a.residual_bytes);

  // the lane's loads: row 2p + rA of the pair, chunk cA of the step
  // (scalar form: one row per half-wave; matrix-core form: see mf_unit)
  const int qb = lane >> 2, qi = lane & 3;  // matrix-core block and position
  const int rA = MF ? (qi >> 1) : hf;
  const int cA = MF ? 2 * qb + (qi & 1) : c;
  const uint32_t v_code = rA * (k / 2) + 16 * cA;
  const uint32_t v_scale = FMT == QMM_AFFINE4_G64 ? rA * (k / 16) + (cA / 2) * 4
                         : FMT == QMM_MXFP4 ? rA * (k / 32) + cA
                         : rA * (k / 16) + 2 * cA;
  const uint32_t v_hi = rA * (k / 4) + 8 * cA;
  const uint32_t v_d = (rA * (k / 256) + cA / 8) * 2;
  // output lane i = 2m + h writes row 2p + h of activation row m
  const int o_h = lane & 1, o_m = min(lane >> 1, M - 1);
  const uint32_t v_res = ((uint32_t)o_m * a.n + o_h) * 2;

  // 0. the NVFP4 tensor scale (used at every pair's store)
  float gscale = (FMT == QMM_NVFP4 && a.tensor_scale) ? a.tensor_scale[0] : 1.0f;

  // 1. the activations, first, so that they do not queue behind the codes.
  //    Every thread issues kXPieces loads (so the compiler counts outstanding
  //    loads exactly); a load with no piece to fetch points past the end of
  //    the buffer and returns zeros without a memory access (clamping it to
  //    the last piece instead queued copies from every wave of the grid on
  //    the one L2 channel holding that piece).
  const int pieces = nch * 4 * M;
  const uint32_t x_bytes = (uint32_t)pieces * 16u;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, x_bytes);
  uint4 xv[kXPieces];
#pragma unroll
  for (int j = 0; j < kXPieces; ++j) {
    const int i = j * kThreads + tid;
    const int ch = i / (4 * M), m = (i >> 2) % M, part_ = i & 3;
    const uint32_t off = i < pieces ? ((uint32_t)m * k + ch * 32 + part_ * 8) * 2u : x_bytes;
    xv[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
  }
  __builtin_amdgcn_sched_barrier(0);

  // 2. the first U units of weights.  Every load is unconditional, so that
  //    the compiler can count outstanding loads exactly: a unit past the
  //    wave's range points every load past the end of its buffer, which
  //    returns zeros at once without touching memory (re-reading real data
  //    there delayed each wave's exit by a memory round trip); the row past n
  //    of an odd n and lanes past K read whatever the buffer holds there, or
  //    zeros beyond its end, and their results are never used.
  // the wave's j-th pair
  auto pair_of = [&](int j) -> int {
    if constexpr (BAL) return pbase + j;
    return j < rfull ? pbase + j * pstride : plast;
  };
  auto load_unit = [&](int t, int j, int s, RowData &rd, uint32_t &res) {
    const bool past = t >= units;  // uniform
    const uint32_t row0 = 2u * (uint32_t)pair_of(j);
    auto at = [past](uint32_t off, uint32_t bytes) { return past ? bytes : off; };
    rd.q = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
        rc, v_code, at(row0 * (k / 2) + (uint32_t)s * (kStepK / 2), a.codes_bytes), 2));
    if constexpr (FMT == QMM_AFFINE4_G64) {
      rd.s = __builtin_amdgcn_raw_buffer_load_b32(
          rs, v_scale, at(row0 * (k / 16) + (uint32_t)s * (kStepK / 16), a.scales_bytes), 0);
    } else if constexpr (FMT == QMM_MXFP4) {
      rd.s = __builtin_amdgcn_raw_buffer_load_b8(
          rs, v_scale, at(row0 * (k / 32) + (uint32_t)s * (kStepK / 32), a.scales_bytes), 0);
    } else {
      rd.s = __builtin_amdgcn_raw_buffer_load_b16(
          rs, v_scale, at(row0 * (k / 16) + (uint32_t)s * (kStepK / 16), a.scales_bytes), 0);
    }
    if constexpr (FMT == QMM_Q6_K) {
      rd.h = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
          rh, v_hi, at(row0 * (k / 4) + (uint32_t)s * (kStepK / 4), a.hi_bytes), 2));
      rd.d = __builtin_amdgcn_raw_buffer_load_b16(
          rs2, v_d, at((row0 * (k / 256) + (uint32_t)s * (kStepK / 256)) * 2, a.scales2_bytes), 0);
    }
    // a null residual has a zero-sized buffer, whose loads return 0
    res = __builtin_amdgcn_raw_buffer_load_b16(rr, v_res, at(row0 * 2u, a.residual_bytes), 0);
  };

  // Every wave of the workgroup has issued its activation loads before any
  // issues a weight load: otherwise the activations of the waves dispatched
  // last queue behind the first waves' weights (per-wave timestamps: the
  // first waves had their x after 0.5 us, the median wave after ~2 us), and
  // the staging barrier waits for the last of them.  An issue barrier only:
  // nothing is waited for.  (Interleaved A/B on cold weights, two boxes: the
  // FP4 5120- and 6144-row shapes 2-8% faster, the decode shapes from 1.5%
  // slower to 7% faster, the mid band within 1.5%.)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  RowData buf[U];
  uint32_t res[U];
  int lj = j0, ls = st0;  // next unit to load: pair index, step
#pragma unroll
  for (int j = 0; j < U; ++j) {
    load_unit(j, lj, ls, buf[j], res[j]);
    if (++ls == S) { ls = 0; ++lj; }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 3. stage x in LDS: pair order for the nibble-into-mantissa formats, and
  //    the sums of x per 32 (affine) or 16 (Q6_K) values
  // the block sums of x of one piece's chunk (called by every lane of the
  // wave: the sums cross lanes)
  auto stage_sums = [&](const uint4 &v, char *rec, int m, int part_, bool ok) {
    if constexpr (kNS > 0) {
      float sm = ((bf_lo(v.x) + bf_hi(v.x)) + (bf_lo(v.y) + bf_hi(v.y))) +
                 ((bf_lo(v.z) + bf_hi(v.z)) + (bf_lo(v.w) + bf_hi(v.w)));
      sm += __shfl_xor(sm, 1);
      float *sums = (float *)(rec + XL::kSumOff);
      if constexpr (kNS == 1) {
        sm += __shfl_xor(sm, 2);
        if (ok && part_ == 0) sums[m] = sm;
      } else {
        if (ok && (part_ & 1) == 0) sums[m * 2 + (part_ >> 1)] = sm;
      }
    }
  };
#pragma unroll
  for (int j = 0; j < kXPieces; ++j) {
    if (j * kThreads >= pieces) break;  // uniform
    const int i = j * kThreads + tid;
    const bool ok = i < pieces;
    const int ch = i / (4 * M), m = (i >> 2) % M, part_ = i & 3;
    const uint4 v = xv[j];
    char *rec = xs + ch * XL::kStride;
    stage_sums(v, rec, m, part_, ok);
    if (ok) {
      uint4 o = v;
      if constexpr (T::kPermute) {
        o.x = (v.x & 0xFFFFu) | (v.z << 16);
        o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
        o.z = (v.y & 0xFFFFu) | (v.w << 16);
        o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
      }
      *(uint4 *)(rec + XL::piece(m, part_)) = o;
    }
  }
  // records past the last chunk, up to a whole step, and the slack after
  // them are zero: lanes past K read them as activations
  {
    const int nchp = (nch + kChunks - 1) / kChunks * kChunks;
    const int n16 = ((nchp - nch) * XL::kStride + kXSlack) / 16;
    uint4 *z = (uint4 *)(xs + (size_t)nch * XL::kStride);
    for (int i = tid; i < n16; i += kThreads) z[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  // A bare barrier: this wave's LDS writes are complete (lgkmcnt), while its
  // weight loads stay in flight.  __syncthreads() would also wait for those
  // (vmcnt(0)), so that every wave drained its pipeline here and restarted it
  // from empty.
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  const UnpackK K = unpack_consts();
  // gscale's load completed before the barrier above (loads complete in
  // order and x was loaded after it); the empty asm tells the compiler so,
  // which keeps it from waiting for every load in flight at each pair's store
  asm volatile("" : "+v"(gscale));
  auto store = [&](int row, float v) {
    if (a.y_bf16)
      ((uint16_t *)a.y)[(size_t)o_m * a.n + row] = (uint16_t)float_to_bf16(v);
    else
      ((float *)a.y)[(size_t)o_m * a.n + row] = v;
  };
  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;
  const char *xs_lane = xs + c * XL::kStride;
  // matrix-core form: accumulators per (group of 4 activation rows, weight
  // row) and the lane's activation words and block sums (B role)
  float accv[MfShape<M>::kG][2];
#pragma unroll
  for (int g = 0; g < MfShape<M>::kG; ++g) accv[g][0] = accv[g][1] = 0.0f;
  const int mB = M <= 2 ? (qi & 1) : qi;
  const int cB = M <= 2 ? 2 * qb + (qi >> 1) : 2 * qb;
  const char *xb_lane = xs + cB * XL::kStride + XL::piece(mB, 0);
  const char *sb_lane = xs + cB * XL::kStride + XL::kSumOff + mB * 4 * (kNS > 0 ? kNS : 1);

  // one unit's products into the lane's sums (step cs of the unit in b)
  auto compute_unit = [&](const RowData &b, int cs) {
    if constexpr (MF) {
      // every lane takes part in the products; a lane whose chunk is past
      // K multiplies zero activations and gets zero scale terms
      RowData rd = b;
      if (cs * kChunks + cA >= nch) {
        rd.s = 0u;
        rd.d = 0u;
      }
      uint32_t P[16];
      unpack_pairs<FMT>(rd, P, K);
      float t0s, t1s;
      mf_scales<FMT>(rd, t0s, t1s);
      const int off = cs * (kChunks * XL::kStride);
      mf_unit<FMT, M, XL::kStride>(P, t0s, t1s, xb_lane + off, sb_lane + off, qi, accv);
    } else if (cs * kChunks + c < nch) {
      // this lane's record of step cs: lane base + a wave-uniform offset
      const char *rec = xs_lane + cs * (kChunks * XL::kStride);
      uint32_t X[M][16];
      float Sx[M][2];
#pragma unroll
      for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = *(const uint4 *)(rec + XL::piece(m, q));
          X[m][4 * q + 0] = v.x;
          X[m][4 * q + 1] = v.y;
          X[m][4 * q + 2] = v.z;
          X[m][4 * q + 3] = v.w;
        }
        const float *sums = (const float *)(rec + XL::kSumOff);
        Sx[m][0] = kNS > 0 ? sums[m * (kNS > 0 ? kNS : 1)] : 0.0f;
        Sx[m][1] = kNS > 1 ? sums[m * 2 + 1] : 0.0f;
      }
      row_step<FMT, M>(b, X, Sx, acc, K);
    }
  };
  // the pair's sums so far, reduced over the wave: lane 2m + h gets row 2p + h
  // of activation row m (lanes < kOut); the lane sums restart from zero
  auto take_sums = [&]() -> float {
    float out = 0.0f;
    if constexpr (MF) {
      out = mf_finish<M>(accv, lane);
    } else {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float s0, s1;
        half_sums(acc[m], s0, s1);
        acc[m] = 0.0f;
        if (lane == 2 * m) out = s0;
        if (lane == 2 * m + 1) out = s1;
      }
    }
    return out;
  };

  int cj = j0, cs = st0;  // unit being computed: pair index, step
  float fin_res = 0.0f;    // balanced: residual of the cut pair this wave finishes
  // Issue priority falls as the wave gets through its units.  The arbiter of
  // a SIMD favours its oldest wave; left alone, the four waves of a SIMD
  // finish one after another and the last ones run with little memory in
  // flight.  Lowering the priority of waves that are ahead lets the ones
  // behind catch up, so that the waves of a SIMD end close together.
  __builtin_amdgcn_s_setprio(3);
  const int q1 = units / 4, q2 = units / 2, q3 = (3 * units) / 4;
  for (int t0 = 0; t0 < units; t0 += U) {
    if (t0 >= q1 && t0 - U < q1) __builtin_amdgcn_s_setprio(2);
    if (t0 >= q2 && t0 - U < q2) __builtin_amdgcn_s_setprio(1);
    if (t0 >= q3 && t0 - U < q3) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (t0 + j < units) {  // uniform
        compute_unit(buf[j], cs);
        if (cs == S - 1 || (BAL && t0 + j == units - 1)) {  // the wave is done with the pair
          const float out = take_sums();
          if (cs == S - 1 && (!BAL || cj != j0 || st0 == 0)) {  // the whole pair
            const int row = 2 * pair_of(cj) + o_h;
            if (lane < kOut && row < a.n) store(row, out * gscale + bf_lo(res[j]));
          } else {  // a cut pair, the wave's first (slot 0) or last (slot 1)
            if (lane < kOut) part[BAL ? wave : 0][cj == j0 ? 0 : 1][lane] = out;
            if (cs == S - 1) fin_res = bf_lo(res[j]);
          }
        }
        if (++cs == S) { cs = 0; ++cj; }
      }
      load_unit(t0 + j + U, lj, ls, buf[j], res[j]);
      if (++ls == S) { ls = 0; ++lj; }
    }
  }

  if constexpr (BAL) {
    // A wave that starts inside a pair and does that pair's last step adds
    // the parts of every wave that shared the pair, in wave order.
    __syncthreads();
    const int u0 = wave * L / kWaves;
    if (st0 != 0 && units > 0 && u0 + units >= (j0 + 1) * S && lane < kOut) {
      int wa = wave - 1;  // the wave holding the pair's first unit
      while (wa * L / kWaves > j0 * S) --wa;
      float sum = 0.0f;
      for (int w = wa; w <= wave; ++w) {
        const int b0 = w * L / kWaves;
        if ((w + 1) * L / kWaves > b0) sum += part[w][b0 / S == j0 ? 0 : 1][lane];
      }
      const int row = 2 * (pbase + j0) + o_h;
      if (row < a.n) store(row, sum * gscale + fin_res);
    }
  }
}

template <int FMT, int M, int U, int SPLIT>
hipError_t launch_rows_cfg(const RowsArgs &a, size_t lds, int grid, hipStream_t s) {
  constexpr int kThreads = RowsShape<M>::kThreads;
  // the dynamic LDS limit is raised once per device for each instantiation
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(raised.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void *)gemv_rows_kernel<FMT, M, U, SPLIT>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
    if (e != hipSuccess) return e;
    raised.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((gemv_rows_kernel<FMT, M, U, SPLIT>), dim3(grid), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

#ifdef QMM_TUNE
#define QMM_ROWS_CONFIGS(X) X(1) X(2) X(3) X(4) X(6)
#else
#define QMM_ROWS_CONFIGS(X) X(2) X(3) X(4)
#endif

template <int FMT, int M>
hipError_t launch_rows_fm(const RowsArgs &a, const GemvPlan &p, hipStream_t s) {
  int split = p.balanced;
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_ROWS_SPLIT")) split = atoi(e);
#endif
#define QMM_CASE(UU)                                                                          \
  if (p.depth == UU)                                                                          \
    return split == kSplitBal ? launch_rows_cfg<FMT, M, UU, kSplitBal>(a, p.lds_bytes, p.tiles, s) \
                              : launch_rows_cfg<FMT, M, UU, kSplitRR>(a, p.lds_bytes, p.tiles, s);
  QMM_ROWS_CONFIGS(QMM_CASE)
#undef QMM_CASE
  return hipErrorInvalidConfiguration;
}

template <int FMT>
hipError_t launch_rows_f(const RowsArgs &a, int m, const GemvPlan &p, hipStream_t s) {
  switch (m) {
    case 1: return launch_rows_fm<FMT, 1>(a, p, s);
    case 2: return launch_rows_fm<FMT, 2>(a, p, s);
    case 3: return launch_rows_fm<FMT, 3>(a, p, s);
    case 4: return launch_rows_fm<FMT, 4>(a, p, s);
    case 5: return launch_rows_fm<FMT, 5>(a, p, s);
    case 6: return launch_rows_fm<FMT, 6>(a, p, s);
    case 7: return launch_rows_fm<FMT, 7>(a, p, s);
    default: return launch_rows_fm<FMT, 8>(a, p, s);
  }
}

int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int v = cached[dev & 63].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 0;
  cached[dev & 63].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace

size_t gemv_rows_lds(int format, int k, int m) {
  const int ns = sums_per_chunk(format);
  const size_t nchp = (size_t)(k / 32 + kStepK / 32 - 1) / (kStepK / 32) * (kStepK / 32);
  const int g = m <= 2 ? 1 : (m + 3) / 4;
  const int stride = use_mfma(format, m) ? mf_stride(256 * g + m * ns * 4) : 64 * m + record_pad(m, ns);
  return nchp * (size_t)stride + kXSlack;
}

bool plan_gemv_rows(int format, int n, int k, int m, GemvPlan &p) {
  if (m < 1 || m > kRowsMaxM) return false;
  const size_t lds = gemv_rows_lds(format, k, m);
  const size_t threads = m <= 4 ? RowsShape<4>::kThreads : RowsShape<8>::kThreads;
  const size_t pieces = m <= 4 ? RowsShape<4>::kXPieces : RowsShape<8>::kXPieces;
  if (lds > kLdsLimit || (size_t)k / 32 * 4 * m > pieces * threads) return false;
  const int cus = cu_count();
  if (cus <= 0) return false;
  p = GemvPlan{};
  p.kind = 1;
  p.rows_per_lane = 1;
  p.lanes_k = 32;
  p.steps = (k + kStepK - 1) / kStepK;
  p.tiles = cus;  // one workgroup per compute unit
  p.splits = 1;
  p.lds_bytes = lds;
  // The split and the units of loads in flight per wave (cold weights, events
  // around back-to-back launches, the settings interleaved in one process):
  //   * balanced where the grid has more waves than pairs and the rows are
  //     long: 5120 x 17408 3-9% faster than round-robin (Q6_K from 1 row,
  //     affine from 2), which leaves 6 of 16 waves per compute unit idle
  //     there; on 5120 x 5120 and 6144 x 5120 balanced is 14-18% slower (its
  //     cut-pair finish and barrier cost more than the idle waves);
  //   * round-robin elsewhere: on 17408 x 5120 8-14% faster than balanced and
  //     14-19% faster than round-robin without the wave-major last round
  //     (which gave an eighth of the workgroups half as many pairs again);
  //   * 2 units in flight on the decode shapes (3 and 4 were 2-9% slower on
  //     17408 x 5120; on 5120 x 17408 at 1 row 3 was faster until the x loads
  //     were issued ahead of every weight load, and is now 3% slower), 4 on
  //     long streams of at least 8 rounds (the 248320 x 5120 projection 3-5%
  //     faster than with 2), 3 for 5 to 8 rows.
  const size_t waves = (size_t)cus * (m <= 4 ? RowsShape<4>::kWaves : RowsShape<8>::kWaves);
  const size_t npairs = ((size_t)n + 1) / 2;
  p.balanced = npairs < waves && p.steps >= 8 ? kSplitBal : kSplitRR;
  if (m >= 5)
    p.depth = 3;
  else if (p.balanced == kSplitBal)
    p.depth = 2;
  else
    p.depth = npairs >= 8 * waves ? 4 : 2;
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_ROWS_U")) p.depth = atoi(e);
#endif
  return true;
}

hipError_t launch_gemv_rows(const qmm_weight &w, const void *x, int m, const void *residual,
                            void *y, int y_dtype, const GemvPlan &p, hipStream_t s) {
  RowsArgs a;
  a.codes = (const uint8_t *)w.codes;
  a.codes_hi = (const uint8_t *)w.codes_hi;
  a.scales = (const uint8_t *)w.scales;
  a.scales2 = (const uint8_t *)w.scales2;
  a.tensor_scale = w.tensor_scale;
  const size_t rows = (size_t)w.batch * w.n;
  a.codes_bytes = (uint32_t)(rows * (size_t)(w.k / 2));
  a.hi_bytes = w.codes_hi ? (uint32_t)(rows * (size_t)(w.k / 4)) : 0u;
  a.scales_bytes = (uint32_t)(rows * (size_t)(w.k / (w.format == QMM_MXFP4 ? 32 : 16)));
  a.scales2_bytes = w.scales2 ? (uint32_t)(rows * (size_t)(w.k / 256) * 2) : 0u;
  a.residual_bytes = residual ? (uint32_t)((size_t)m * w.n * 2) : 0u;
  a.x = (const uint16_t *)x;
  a.residual = (const uint16_t *)residual;
  a.y = y;
  a.n = w.n;
  a.k = w.k;
  a.steps = p.steps;
  a.y_bf16 = y_dtype == QMM_BF16;
  switch (w.format) {
    case QMM_AFFINE4_G64: return launch_rows_f<QMM_AFFINE4_G64>(a, m, p, s);
    case QMM_MXFP4: return launch_rows_f<QMM_MXFP4>(a, m, p, s);
    case QMM_NVFP4: return launch_rows_f<QMM_NVFP4>(a, m, p, s);
    default: return launch_rows_f<QMM_Q6_K>(a, m, p, s);
  }
}

}  // namespace qmm

namespace qmm {

// qgemm's mid band, 5 to 8 activation rows ("TurboEXL3" section 4.3, the
// trunk: 5 to 16 rows take a GEMV chain that decodes each weight once per
// chunk of up to 8 rows): the row-streaming kernel, which reads and decodes
// the weights once, with the exact weights (no bfloat16 rounding of the
// weights, unlike the MFMA tiles) and a bfloat16 y.  Measured on 17408 x 5120
// (cold weights, us, GEMV with v_dot2 products / MFMA tiles): affine 5 rows
// 23.9 / 38.0, 8 rows 28.9 / 38.0; NVFP4 23.0 / 37.6, 27.1 / 38.2; Q6_K
// 31.6 / 55.6, 37.3 / 55.3; MXFP4 21.8 / 37.2, 26.4 / 37.5; with the
// matrix-core products from 6 rows (5 for Q6_K), 8 rows take affine ~22,
// NVFP4 ~20, Q6_K ~27 us.  Two chunks for 9 to 16 rows lost to the MFMA tiles
// (affine 9 rows 42.2 / 38.2, 16 rows 56.7 / 40.3), so those rows stay there.
bool gemm_rows_fits(const qmm_weight &w, int m) {
  if (m < 5 || m > kRowsMaxM || w.batch != 1) return false;
  GemvPlan p;
  return plan_gemv_rows(w.format, w.n, w.k, m, p);
}

hipError_t launch_gemm_rows(const qmm_weight &w, const void *x, int m, const void *residual,
                            void *y, hipStream_t s) {
  GemvPlan p;
  if (!plan_gemv_rows(w.format, w.n, w.k, m, p)) return hipErrorInvalidValue;
  return launch_gemv_rows(w, x, m, residual, y, QMM_BF16, p, s);
}

}  // namespace qmm
