// qgemm and the grouped MoE multiplies: each weight decoded once per tile into
// bfloat16 ("TurboEXL3" section 4.1: decode once, multiply many times), bf16
// MFMA with float32 sums over K in slice order, on this data path:
//
//   * the activation tile (32 TM rows) goes from memory straight into LDS
//     (buffer_load_dwordx4 ... lds), three 64-wide K slices in flight, with no
//     register staging; its 16-byte chunks are XOR-swizzled by row so that the
//     MFMA operand reads of a lane group fall on distinct LDS bank groups;
//   * the weights never pass through LDS: each wave owns 32 rows of the tile,
//     loads their codes and scales itself (registers, three slices ahead) and
//     decodes them straight into its MFMA A operands.  The K order inside a
//     slice is permuted (lane half h of a 32-lane row holds K values 32h ..
//     32h+31, 8 of them for each of the slice's four k-steps) and the
//     activation operand is read in the same order, so each lane decodes one
//     contiguous 32-weight run of one row with one 16-byte code load;
//   * a wave computes TM v_mfma_f32_32x32x16_bf16 tiles (its 32 W rows x 32 TM
//     rows of X).  From 257 rows of X on: 8 waves of 32 W rows x 256 X rows
//     (TM = 8), so that each decoded weight feeds 8 MFMAs per k-step, as do
//     the grouped MoE modes (256 rows is the routing table's tile height), or
//     x 192 rows (TM = 6) where that fills the last round of workgroups
//     better; up to 256 rows: 4 waves of 32 x 128 (more workgroups for small
//     calls).  A wave holds at most 128 float32 accumulators; two waves share
//     a SIMD.
//
// Per slice and wave (dense, TM = 8): 32 MFMAs, 32 decoded weights per lane,
// 32 KB of LDS operand reads; per workgroup 32 KB of activations and 9-14 KB
// of weight codes from memory, about half of what 128 x 128 tiles staged
// through LDS moved per flop.  (The 32 x 32 x 16 form against the 16 x 16 x 32
// one, same tiles: 3-15% faster up to 512 rows, the same from 2048 on, where
// the matrix cores' clock sets the pace: with random operands a bare MFMA
// loop runs both at ~1.75 PFLOP/s on MI355X, the clock falling to ~1.8 GHz.)
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <type_traits>

#include "gemm_common.h"
#include "swiglu_device.h"

namespace qmm {
namespace {

using namespace gemm;

constexpr int kStages = 3;  // LDS stages of X = slices in flight
// (6 or 8 stages for the 32- and 64-row tiles measured 10% faster unsplit but
// slower split, and the split form is the faster one for those calls)
constexpr int kXRow = kBK * 2;  // bytes of one X row in a slice

// Buffer descriptors and the per-lane constant parts of a lane's weight
// offsets (its row and half); the slice's part goes in the scalar offset.
struct WSrc {
  __amdgpu_buffer_rsrc_t rc, rh, rs, rs2;
  uint32_t v_code, v_hi, v_s, v_d;
};

// The lane's 32-weight run of slice s: values 32h .. 32h+31 of the slice
// (h = lane / 32), codes and what scales them.
template <int FMT>
__device__ __forceinline__ Piece load_run(const WSrc &w, int s) {
  Piece p;
  p.q = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(w.rc, w.v_code, s * (kBK / 2), 0));
  if constexpr (FMT == QMM_AFFINE4_G64) {
    p.s = __builtin_amdgcn_raw_buffer_load_b32(w.rs, w.v_s, s * 4, 0);
  } else if constexpr (FMT == QMM_MXFP4) {
    p.s = __builtin_amdgcn_raw_buffer_load_b8(w.rs, w.v_s, s * 2, 0);
  } else if constexpr (FMT == QMM_NVFP4) {
    p.s = __builtin_amdgcn_raw_buffer_load_b16(w.rs, w.v_s, s * 4, 0);
  } else {
    p.h = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(w.rh, w.v_hi, s * (kBK / 4), 0));
    p.s = __builtin_amdgcn_raw_buffer_load_b16(w.rs, w.v_s, s * 4, 0);
    p.d = __builtin_amdgcn_raw_buffer_load_b16(w.rs2, w.v_d, (s / 4) * 2, 0);
  }
  return p;
}

// Physical 16-byte chunk offset of X row `row` in LDS: logical chunk c sits at
// c ^ swz(row).  The 16 rows read by one ds_read_b128 lane group (same logical
// chunk) then land on distinct bank groups; measured on gfx950 at 119 TB/s of
// LDS reads against 71 TB/s for a plain (row / 2) swizzle.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int FMT>
constexpr int w_loads_per_run() { return FMT == QMM_Q6_K ? 4 : 2; }

// A wave owns 32 rows of W and computes them against the workgroup's BM =
// 32 TM rows of X as TM v_mfma_f32_32x32x16_bf16 tiles; the WAVES waves cover
// BN = 32 WAVES rows of W.  MODE (gemm_common.h): dense, or the grouped MoE
// gate/up (rows of x gathered by token, gate and up weight rows interleaved,
// SwiGLU epilogue) and down products over the routing tile table (tiles of BM
// grouped rows, one expert each).
template <int FMT, int TM, int WAVES, int MODE>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_big_kernel(GemmArgs a) {
  constexpr int kBN = 32 * WAVES;
  constexpr int BM = 32 * TM;
  constexpr int kXStage = BM * kXRow;   // bytes per LDS stage
  constexpr int XI = BM / (8 * WAVES);  // X load instructions per wave and slice (8 rows each)
  static_assert(XI >= 1 && XI * 8 * WAVES == BM, "every wave loads the same X rows per slice");
  extern __shared__ __align__(16) uint8_t lds[];  // kStages x [BM rows][128 bytes]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int m0, n0, mrows, wrow0 = 0, expert = 0, tile = 0, split = 0;
  if constexpr (MODE == kDense) {
    const int tiles_m = (a.m + BM - 1) / BM;
    tile = (int)blockIdx.x / a.splits;
    split = (int)blockIdx.x - tile * a.splits;
    m0 = (tile % tiles_m) * BM;
    n0 = a.n_begin + (tile / tiles_m) * kBN;
    mrows = a.m - m0;
  } else {
    // workgroup -> (routing tile, column block).  Workgroups go to the 8
    // XCDs in turn (workgroup w to XCD w % 8); the consecutive workgroups
    // of XCD x take the tile pair 2 (8 q + x), 2 (8 q + x) + 1 column block
    // by column block, so the pair's gathered activation slices (and the
    // weight rows of an expert with two tiles) are shared in that XCD's L2.
    // Measured (interleaved A/B, bit-identical): one tile per XCD run
    // against tiles fastest in a 2-D grid (a tile's column blocks on
    // different XCDs about two rounds apart, each gathering the tile again)
    // T = 8192 1.097 -> 1.019 ms per layer, T = 100-2048 2-4% faster; pairs
    // against single tiles T = 2048 7%, T = 512 4%, T = 8192 1% faster;
    // groups of 4 or 8 tiles 1-7% slower than pairs.  Any other XCD count
    // only changes which workgroups share an L2.
    const int ncb = (a.n + kBN - 1) / kBN, j = (int)blockIdx.x >> 3;
    const int q = j / (2 * ncb), r = j - q * 2 * ncb;
    const int tl = (q * 8 + ((int)blockIdx.x & 7)) * 2 + (r & 1), cb = r >> 1;
    if (tl >= *a.n_tiles) return;  // beyond this call's tiles (whole workgroup)
    const uint32_t *t = a.tiles + 3 * tl;
    expert = (int)t[0];
    m0 = (int)t[1];
    mrows = (int)t[2];
    n0 = cb * kBN;
    wrow0 = expert * a.n;  // first row of the expert's matrix
  }
  // this workgroup's slices [s_begin, s_end)
  const int slices = a.k / kBK;
  const int s_begin = MODE == kDense ? split * a.sps : 0;
  const int s_end = MODE == kDense ? min(s_begin + a.sps, slices) : slices;
  const uint32_t k = (uint32_t)a.k;
  const int lr = lane & 31, h = lane >> 5;

  // activations: wave w fills rows (BM/WAVES) w .. of a stage, 8 rows per
  // instruction; lane l of instruction i writes LDS chunk l % 8 of row
  // (BM/WAVES) w + 8i + l / 8, which holds the row's logical chunk
  // (l % 8) ^ swz(row) (grouped modes: the routing tables index valid rows
  // of x or h, whose extent the call does not pass; their descriptor spans
  // the 32-bit range)
  const __amdgpu_buffer_rsrc_t rx =
      MODE == kDense ? make_rsrc(a.x, (uint32_t)((size_t)a.m * a.k * 2))
                     : make_rsrc(MODE == kMoeGateUp ? (const void *)a.x : (const void *)a.h, 0xFFFFFFFFu);
  uint32_t v_x[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int row = (BM / WAVES) * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    const int rr = m0 + min(row, mrows - 1);
    const uint32_t src = MODE == kMoeGateUp ? a.token_of_row[rr] : (uint32_t)rr;
    v_x[i] = (src * k + (uint32_t)c * 8) * 2;
  }
  auto load_x = [&](int s) __attribute__((always_inline)) {
    uint8_t *st = lds + (s % kStages) * kXStage + wave * (BM / WAVES) * kXRow;
#pragma unroll
    for (int i = 0; i < XI; ++i)
      buffer_load_lds16(rx, st + i * 8 * kXRow, v_x[i], s * kXRow);
  };

  // weights: lane (lr, h) holds tile row j = 32 w + lr, values 32h .. 32h+31
  // of each slice; tile row j is weight row n0 + j, or in the gate/up mode
  // gate or up row n0/2 + j/2 of the expert (even j gate, odd j up)
  WSrc ws;
  {
    const size_t rows = (size_t)a.wrows;
    ws.rc = make_rsrc(a.codes, (uint32_t)(rows * (k / 2)));
    ws.rh = make_rsrc(a.codes_hi, a.codes_hi ? (uint32_t)(rows * (k / 4)) : 0u);
    ws.rs = make_rsrc(a.scales, (uint32_t)(rows * (k / (FMT == QMM_AFFINE4_G64 ? 16 : (FMT == QMM_MXFP4 ? 32 : 16)))));
    ws.rs2 = make_rsrc(a.scales2, a.scales2 ? (uint32_t)(rows * (k / 256) * 2) : 0u);
    const int j = 32 * wave + lr;
    uint32_t r;
    if constexpr (MODE == kMoeGateUp)
      r = (uint32_t)(wrow0 + ((j & 1) ? a.inter : 0) + min(n0 / 2 + j / 2, a.inter - 1));
    else
      r = (uint32_t)(wrow0 + min(n0 + j, a.n - 1));
    ws.v_code = r * (k / 2) + 16 * h;
    ws.v_hi = r * (k / 4) + 8 * h;
    ws.v_s = FMT == QMM_AFFINE4_G64 ? r * (k / 64) * 4
           : FMT == QMM_MXFP4       ? r * (k / 32) + h
                                    : r * (k / 16) + 2 * h;
    ws.v_d = r * (k / 256) * 2;
  }
  Piece wr[kStages];
  // down mode: the token slot (row of d) of each of this lane's TM rows, read
  // ahead of the pipeline so that the epilogue does not wait for it
  uint32_t drow_of[MODE == kMoeDown ? TM : 1];
  if constexpr (MODE == kMoeDown) {
#pragma unroll
    for (int t = 0; t < TM; ++t) drow_of[t] = a.slot_of_row[m0 + min(32 * t + lr, mrows - 1)];
  }

  f32x16_t acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;

  // operand reads of the activation tile for k-step st: row 32t + lr,
  // logical chunk 4h + st at physical chunk (4h + st) ^ swz(lr) (swz of
  // 32t + lr is swz(lr))
  uint32_t xo[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) xo[st] = (uint32_t)lr * kXRow + (uint32_t)(((4 * h + st) ^ swz(lr)) * 16);

  // slices 0 .. kStages-2 in flight; every iteration then issues one more
  // (the last slice again past the end, so that every wave issues the same
  // loads and the counts below hold)
  constexpr int kLoadsPerSlice = XI + w_loads_per_run<FMT>();
  // The waits below count loads, so the loads must issue slice by slice: the
  // scheduler is kept from regrouping them (left alone it can put every
  // slice's weight loads ahead of the first slice's activations, which the
  // first wait would then not cover).
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p) {
    const int sp = min(s_begin + p, s_end - 1);
    load_x(sp);
    wr[p] = load_run<FMT>(ws, sp);
    __builtin_amdgcn_sched_barrier(0);
  }

  // One slice: s is the slice, u its weight slot (s - s_begin) % kStages.
  auto slice = [&](const int s, auto uc) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    // this wave's share of slice s is in LDS once at most the loads issued
    // after it (kStages - 2 slices) are outstanding; the barrier then makes
    // every wave's share visible and frees the stage read in iteration s - 1
    // (whose operands are already in registers).  A bare s_barrier: the
    // fence of __syncthreads would also wait for the slices still in flight.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 2) * kLoadsPerSlice));
    __builtin_amdgcn_s_barrier();
    const int sn = min(s + kStages - 1, s_end - 1);
    load_x(sn);
    wr[(u + kStages - 1) % kStages] = load_run<FMT>(ws, sn);

    // the run's 32 weights: k-step st takes values 8 st .. 8 st + 7.  The
    // decode of k-step st + 1's weights is interleaved with k-step st's
    // MFMAs (each MFMA occupies the matrix core for many cycles, in which
    // the wave issues independent vector instructions), so that only the
    // first k-step's decode runs with the matrix core idle.
    const PieceScale sc = piece_scale<FMT>(wr[u]);
    uint32_t o[4];
    decode_part<FMT>(wr[u], sc, 0, o);
    bf16x8_t af = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});

    // Likewise the activation operands of k-step st + 1 are read from LDS
    // during k-step st's MFMAs, so that no k-step but the first waits on LDS.
    const uint8_t *stg = lds + (s % kStages) * kXStage;
    bf16x8_t bfr[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) bfr[t] = *(const bf16x8_t *)(stg + t * 32 * kXRow + xo[0]);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      // MFMA t, then one LDS read and part of the decode for k-step st + 1,
      // in this order (the scheduler is kept from regrouping them)
      __builtin_amdgcn_sched_barrier(0);
      uint32_t on[4] = {0u, 0u, 0u, 0u};
      bf16x8_t bfn[TM];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[t], acc[t], 0, 0, 0);
        if (st < 3) {
          bfn[t] = *(const bf16x8_t *)(stg + t * 32 * kXRow + xo[st + 1]);
#pragma unroll
          for (int i = t * 4 / TM; i < (t + 1) * 4 / TM; ++i) on[i] = decode_word<FMT>(wr[u], sc, st + 1, i);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      af = __builtin_bit_cast(bf16x8_t, u32x4_t{on[0], on[1], on[2], on[3]});
#pragma unroll
      for (int t = 0; t < TM; ++t) bfr[t] = bfn[t];
    }
  };
  // Whole groups of kStages slices, then the rest: the loop body has no exit
  // of its own, so that the compiler's wait analysis keeps track of the
  // weight loads' age across the back edge.
  static_assert(kStages == 3, "the slice loop is written out for three stages");
  int s = s_begin;
  for (; s + kStages <= s_end; s += kStages) {
    slice(s, std::integral_constant<int, 0>{});
    slice(s + 1, std::integral_constant<int, 1>{});
    slice(s + 2, std::integral_constant<int, 2>{});
  }
  if (s < s_end) slice(s, std::integral_constant<int, 0>{});
  if (s + 1 < s_end) slice(s + 1, std::integral_constant<int, 1>{});

  // The loads issued past the last slice (re-reads of it, so that the counts
  // above hold) may still be in flight; a workgroup must not end with LDS
  // writes pending, or they could land in the LDS of the next workgroup on
  // the compute unit.
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // epilogue: lane (lr, h) holds D[n = 8b + 4h + r][m = lr] of each tile as
  // value 4b + r: four consecutive W rows per b
  if constexpr (MODE == kDense) {
    if (a.splits > 1) {
      // split K: this split's float32 sums of the tile's valid rows go out as
      // 16-byte stores with the sc1 cache bit (written through to where every
      // XCD sees them, without flushing the L2s); every wave waits for its
      // stores before the barrier that precedes the counter increment, so the
      // workgroup that takes the count to splits - 1 sees every split's
      // partials (read with sc1 loads, which miss the non-coherent L2), adds
      // them in split order and runs the epilogue below on the sums.  n is a
      // multiple of 4 whenever the host splits.
      constexpr int kSc1 = 16;  // cache-policy bit of gfx950 buffer operations
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(a.partials, 0xFFFFFFFFu);
      const uint32_t split_off = (uint32_t)split * (uint32_t)a.m * (uint32_t)a.n;
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int ml = 32 * t + lr;
        if (ml >= mrows) continue;
        const uint32_t row_off = split_off + (uint32_t)(m0 + ml) * (uint32_t)a.n;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int nb = n0 + 32 * wave + 8 * b + 4 * h;
          if (nb < a.n)
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4_t, f32x4_t{acc[t][4 * b], acc[t][4 * b + 1], acc[t][4 * b + 2],
                                                    acc[t][4 * b + 3]}),
                rp, (row_off + (uint32_t)nb) * 4u, 0, kSc1);
        }
      }
      __shared__ int s_last;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (tid == 0)
        s_last = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(a.splits - 1);
      __syncthreads();
      if (!s_last) return;
      const uint32_t split_stride = (uint32_t)a.m * (uint32_t)a.n * 4u;
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int ml = 32 * t + lr;
        if (ml >= mrows) continue;
        const uint32_t row_off = (uint32_t)(m0 + ml) * (uint32_t)a.n;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int nb = n0 + 32 * wave + 8 * b + 4 * h;
          if (nb >= a.n) continue;
          f32x4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
          for (int sp = 0; sp < a.splits; ++sp) {
            v += __builtin_bit_cast(
                f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rp, (row_off + (uint32_t)nb) * 4u + sp * split_stride, 0, kSc1));
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[t][4 * b + r] = v[r];
        }
      }
    }
  }
  const float gs = (FMT == QMM_NVFP4 && a.tensor_scale) ? a.tensor_scale[expert] : 1.0f;
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const int ml = 32 * t + lr;
    if (ml >= mrows) continue;
    const int m = m0 + ml;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int nl = 32 * wave + 8 * b + 4 * h;  // tile row of v[0]
      float v[4] = {acc[t][4 * b] * gs, acc[t][4 * b + 1] * gs, acc[t][4 * b + 2] * gs,
                    acc[t][4 * b + 3] * gs};
      if constexpr (MODE == kMoeGateUp) {
        // (gate, up, gate, up) of two consecutive intermediate columns; SwiGLU
        // in float32: h = silu(g) * u, silu(g) = g / (1 + e^-g)
        const int col = n0 / 2 + nl / 2;  // even, and I is even
        if (col < a.inter) {
          const float h0 = silu_f32(v[0]) * v[1];
          const float h1 = silu_f32(v[2]) * v[3];
          *(uint32_t *)(a.h + (size_t)m * a.inter + col) = pack_bf16(h0, h1);
        }
        continue;
      } else if constexpr (MODE == kMoeDown) {
        // grouped row m goes to its token slot's row of d
        const size_t drow = (size_t)drow_of[t];
        const int nb = n0 + nl;
        if (nb + 3 < a.n) {
          *(float4 *)(a.d + drow * a.n + nb) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          for (int r = 0; r < 4 && nb + r < a.n; ++r) a.d[drow * a.n + nb + r] = v[r];
        }
        continue;
      }
      const int nb = n0 + nl;
      const size_t base = (size_t)m * a.n + nb;
      if (nb + 3 < a.n && (a.n & 3) == 0) {
        if (a.residual) {
          const uint2 r = *(const uint2 *)(a.residual + base);
          v[0] += bf_lo(r.x);
          v[1] += bf_hi(r.x);
          v[2] += bf_lo(r.y);
          v[3] += bf_hi(r.y);
        }
        *(uint2 *)(a.y + base) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (nb + r >= a.n) break;
          float t2 = v[r];
          if (a.residual) t2 += bf_lo(a.residual[base + r]);
          a.y[base + r] = __builtin_bit_cast(uint16_t, (__bf16)t2);
        }
      }
    }
  }
}

template <int FMT, int TM, int WAVES, int MODE>
hipError_t launch_big(const GemmArgs &a, dim3 grid, hipStream_t s) {
  static_assert(MODE == kDense || 32 * TM <= kMoeTileRows,
                "X tiles hold the routing table's tiles of at most kMoeTileRows rows");
  constexpr size_t lds = (size_t)kStages * 32 * TM * kXRow;
  // more than 64 KiB of dynamic LDS must be allowed once per device
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void *)gemm_big_kernel<FMT, TM, WAVES, MODE>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((gemm_big_kernel<FMT, TM, WAVES, MODE>), grid, dim3(64 * WAVES), lds, s, a);
  return hipGetLastError();
}

template <int TM, int WAVES, int MODE>
hipError_t launch_big_mode(int format, const GemmArgs &a, dim3 grid, hipStream_t s) {
  switch (format) {
    case QMM_AFFINE4_G64: return launch_big<QMM_AFFINE4_G64, TM, WAVES, MODE>(a, grid, s);
    case QMM_MXFP4: return launch_big<QMM_MXFP4, TM, WAVES, MODE>(a, grid, s);
    case QMM_NVFP4: return launch_big<QMM_NVFP4, TM, WAVES, MODE>(a, grid, s);
    default: return launch_big<QMM_Q6_K, TM, WAVES, MODE>(a, grid, s);
  }
}

// workgroups' rows of W for a configuration of `waves` waves
constexpr int bn_of(int waves) { return 32 * waves; }

// Small calls (m <= 256 rows): the activation tile height and the number of
// K splits, from a sweep on 17408 x 5120 (MI355X, kernel trace, medians of 24
// cold-weight launches; unsplit 128-row tiles take ~55 us for any m, a
// workgroup walking its 80 slices in series):
//   m <= 16: 32-row tiles, 4 splits  (35.6 us at m = 1, 36.4 at 8, 38.8 at 16)
//   m <= 32: 32-row tiles, 2 splits  (42.6 us)
//   m <= 64: 64-row tiles, unsplit   (46.7 us; splits cost more than they save)
//   else:    128-row tiles, unsplit  (57 us at m = 128; 2 splits 75 us)
// A split writes and reads back m x n float32 partials, so it pays only while
// m is small.
// Up to 256 activation rows: the tile height (tm blocks of 32 rows) and the
// K split (sk ways, float32 partials in the caller's workspace).  From the
// fewest blocks that cover M (split 4 ways up to 16 rows and 2 up to 32),
// lower tiles or more splits where they take less time counted in rounds of
// one workgroup per compute unit, a workgroup costing its slices
// (64 K values) weighted by tile height (1, 0.8 and 0.72 for 128, 64 and 32
// rows: each tile runs its whole K range) plus ~20 slices for a split's
// partials, finish and counter clearing.  Interleaved A/B, NVFP4 (bits equal
// where nothing splits): 17408 x 5120 at M = 160-192 89 -> 72 us (64-row
// tiles), 96, 128 and 256 unchanged (no split pays with 80 slices); 5120 x
// 17408 (40 blocks of weight rows, 272 slices) at M = 96-128 97-99 -> 52-56
// us (128-row tiles split 4 ways), 192 105 -> 72 us (64-row, 2 ways), 256
// 110 -> 87 us (128-row, 2 ways), 40-64 102-106 -> 38-42 us (64-row, 4
// ways), 24 52 -> 32 us (32-row, 4 ways).  `split` false: the caller's
// workspace cannot hold partials.
struct SmallPlan {
  int tm, sk;
};

SmallPlan small_m_plan(const qmm_weight &w, int m, bool split) {
  const int slices = w.k / kBK;
  // partial offsets stay 32-bit; each split keeps the three-stage pipeline busy
  auto split_ok = [&](int sk) {
    return split && w.n % 4 == 0 && (slices + sk - 1) / sk >= 4 &&
           (double)sk * m * w.n * 4 < 4294967296.0;
  };
  // the base plan: the fewest blocks that cover M, and (up to 32 rows) the
  // split measured best on the mid band's 17408 x 5120 calls
  const int tm0 = m <= 32 ? 1 : m <= 64 ? 2 : 4;
  int sk0 = m <= 16 ? 4 : (m <= 32 ? 2 : 1);
  while (sk0 > 1 && !split_ok(sk0)) sk0 /= 2;
  const long nb = (w.n + 127) / 128, cus = compute_units();
  auto cost = [&](int tm, int sk) {
    const long wgs = (m + 32 * tm - 1) / (32 * tm) * nb * sk;
    const double per = (tm == 4 ? 1.0 : tm == 2 ? 0.8 : 0.72) * ((slices + sk - 1) / sk) +
                       (sk > 1 ? 20.0 : 0.0);
    return (double)((wgs + cus - 1) / cus) * per;
  };
  // lower tiles or more splits where the round count says so
  SmallPlan p{tm0, sk0};
  double best = cost(tm0, sk0);
  for (int tm : {4, 2, 1})
    for (int sk : {1, 2, 4}) {
      if (tm > tm0 || sk < sk0 || (sk > 1 && !split_ok(sk))) continue;
      const double c = cost(tm, sk);
      if (c < best) p = {tm, sk}, best = c;
    }
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_GEMM_SPLITS")) p.sk = split ? std::max(1, atoi(e)) : 1;
  if (const char *e = getenv("QMM_SMALL_TM")) p.tm = atoi(e);
#endif
  return p;
}

int small_m_splits(const qmm_weight &w, int m) { return m > 256 ? 1 : small_m_plan(w, m, true).sk; }

size_t split_counters_bytes(const qmm_weight &w, int m) {
  const size_t tiles = (size_t)((m + 31) / 32) * ((w.n + 127) / 128);  // 32-row tiles at most
  return (tiles * 4 + 255) / 256 * 256;
}

struct BigTail {
  long tiles_m, tiles_n, tn_a;  // tiles of the first launch: tiles_m x tn_a
};

GemmArgs big_args(const qmm_weight &w) {
  GemmArgs a{};
  a.splits = 1;
  a.sps = w.k / kBK;
  a.codes = (const uint8_t *)w.codes;
  a.codes_hi = (const uint8_t *)w.codes_hi;
  a.scales = (const uint8_t *)w.scales;
  a.scales2 = (const uint8_t *)w.scales2;
  a.tensor_scale = w.tensor_scale;
  a.n = w.n;
  a.k = w.k;
  a.wrows = w.batch * w.n;
  return a;
}

// The last round of one-per-CU workgroups.  When at least one whole round
// is followed by a last round that holds at most a quarter of the compute
// units, the big tiles cover the whole rounds only (tn_a of the tiles_n
// weight-row blocks) and a second launch takes the remaining weight rows as
// 128 x 128 tiles, several to a compute unit.  Measured on 17408 x 5120
// (interleaved A/B, bit-identical: each output's sum over K runs in the same
// order in either tile): M = 4096 (1024 + 256 small tiles) 7-8% faster,
// M = 3072 9%, M = 1024 7-9% (against 192-row tiles), M = 2048 and 8192
// within 1%; a last round of 3/5 of the compute units (M = 1536) 4% slower,
// and K split two or three ways over the last 128 big tiles of M = 8192
// (partials in a workspace) 2-8% slower: while only part of the chip runs,
// the matrix cores' power-limited clock rises, so a short last round costs
// less than its share of tiles.
bool big_tail_fits(long full, long frac, long cus) { return full >= 1 && frac > 0 && 4 * frac <= cus; }

BigTail big_tail(const qmm_weight &w, int m, int cfg) {
  BigTail t{};
  const int bm = cfg == 0 ? 256 : cfg == 10 ? 320 : 192;
  t.tiles_m = (m + bm - 1) / bm;
  t.tiles_n = (w.n + bn_of(8) - 1) / bn_of(8);
  t.tn_a = t.tiles_n;
  const long cus = compute_units();
  const long full = t.tiles_m * t.tiles_n / cus;         // whole rounds
  const long frac = t.tiles_m * t.tiles_n - full * cus;  // tiles of the last round
  bool tail = big_tail_fits(full, frac, cus);
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_BIG_TAIL")) tail = tail && atoi(e) != 0;
#endif
  if (!tail) return t;
  const long tn_a = full * cus / t.tiles_m;  // weight-row blocks that fill whole rounds
  if (tn_a > 0 && tn_a < t.tiles_n) t.tn_a = tn_a;
  return t;
}

// Activation rows of the tail's tiles, in blocks of 32: 128, halved while the
// halved tiles still fit one round of workgroups (nb blocks of 128 weight
// rows).
int tail_tm(long m, long nb, long cus) {
  int tm = 4;
  while (tm > 1 && (m + 16 * tm - 1) / (16 * tm) * nb <= cus) tm /= 2;
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_TAIL_TM")) tm = atoi(e);
#endif
  return tm;
}

// The big-tile configuration above 256 rows: 8 waves of 32 W rows x 256 X
// rows (0), x 192 rows (4) or x 320 rows (10), whichever takes the least
// time counted in rounds of 256-row workgroups (one per compute unit): a
// 192-row round takes about 0.85 of a 256-row one, a 320-row round 1.25, and
// a small-tile tail about 0.33 per round of 128 x 128 tiles (each of them
// runs the whole K loop, so a short tail still takes that long: 192-row
// tiles plus a tail at M = 768 measured 20% slower than one round of
// 256-row tiles).  (320-row tiles, 244 registers a lane, measured as their
// round count predicts: 2-3% faster at M = 8192 on 17408 rows, 1768 tiles
// in 6.9 rounds against 2176 in 8.5; equal at 16384, 6% slower at 4096.)
int big_cfg(const qmm_weight &w, int m) {
  const long nt = (w.n + bn_of(8) - 1) / bn_of(8), cus = compute_units();
  auto cost = [&](int bm, double per_round) {
    const long tm = (m + bm - 1) / bm, tl = tm * nt, full = tl / cus, frac = tl - full * cus;
    if (big_tail_fits(full, frac, cus)) {
      const long tn_a = std::min(nt, std::max(1L, full * cus / tm));
      const long small = (m + 127) / 128 * ((w.n - tn_a * bn_of(8) + bn_of(4) - 1) / bn_of(4));
      return per_round * (double)((tm * tn_a + cus - 1) / cus) + 0.33 * (double)((small + cus - 1) / cus);
    }
    return per_round * (double)((tl + cus - 1) / cus);
  };
  const double r0 = cost(256, 1.0), r4 = cost(192, 0.85), r10 = cost(320, 1.25);
  int cfg = r4 < r0 ? 4 : 0;
  if (r10 < std::min(r0, r4)) cfg = 10;
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_BIG_CFG")) cfg = atoi(e);
#endif
  return cfg;
}

}  // namespace

long compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int v = cached[dev & 63].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 256;
  cached[dev & 63].store(v, std::memory_order_relaxed);
  return v;
}

size_t gemm_big_workspace(const qmm_weight &w, int m) {
  const int sk = small_m_splits(w, m);
  if (sk == 1) return 0;
  return split_counters_bytes(w, m) + (size_t)sk * m * w.n * 4;
}

// 5 to 8 rows whose activations fit in LDS take the row-streaming GEMV
// (gemv_rows.hip, which holds the measurements) instead of the MFMA tiles.
bool gemm_uses_rows(const qmm_weight &w, int m) {
  bool rows = gemm_rows_fits(w, m);
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_GEMM_ROWS")) rows = rows && atoi(e) != 0;
#endif
  return rows;
}

size_t gemm_workspace_size(const qmm_weight &w, int m) {
  if (!gemm_big_fits(w, (size_t)m) || gemm_uses_rows(w, m)) return 0;
  return gemm_big_workspace(w, m);
}

bool gemm_big_fits(const qmm_weight &w, size_t x_rows) {
  // 32-bit buffer offsets for X and every weight plane
  return x_rows * (size_t)w.k * 2 < (1ull << 32) && (size_t)w.batch * w.n * w.k < (1ull << 32);
}

hipError_t launch_gemm_big(const qmm_weight &w, const void *x, int m, const void *residual, void *y,
                           void *workspace, size_t workspace_bytes, hipStream_t s) {
  if (gemm_uses_rows(w, m)) return launch_gemm_rows(w, x, m, residual, y, s);
  GemmArgs a = big_args(w);
  a.x = (const uint16_t *)x;
  a.residual = (const uint16_t *)residual;
  a.y = (uint16_t *)y;
  a.m = m;
  auto grid = [&](int bm, int bn) {
    return dim3((unsigned)(((m + bm - 1) / bm) * ((w.n + bn - 1) / bn) * a.splits));
  };
  // 8 waves of 32 W rows x 256 X rows: each decoded weight feeds twice the
  // MFMAs of the 4-wave 64 x 128 form (measured 1.3x faster from M = 512 on);
  // or 8 waves of 32 x 192 where that takes fewer rounds of workgroups
  // (big_cfg; 192-row tiles measured 1.2x faster at M = 300 and 512 on 17408
  // rows, and 1.14x at M = 2048 before the tail launch below existed, which
  // now gives 256-row tiles the same time there).  Up to 256 rows of X: 4
  // waves of 32 x 128, whose 128-row W tiles give a 128-row call 136
  // workgroups (1.9x faster than 128 x 128 tiles staged through LDS at
  // M = 128, 1.4x at M = 256).
  const int cfg = m > 256 ? big_cfg(w, m) : 1;
  if (cfg == 0 || cfg == 4 || cfg == 10) {
    const BigTail t = big_tail(w, m, cfg);
    const dim3 ga((unsigned)(t.tiles_m * t.tn_a));
    const hipError_t e = cfg == 0  ? launch_big_mode<8, 8, kDense>(w.format, a, ga, s)
                         : cfg == 4 ? launch_big_mode<6, 8, kDense>(w.format, a, ga, s)
                                    : launch_big_mode<10, 8, kDense>(w.format, a, ga, s);
    if (e != hipSuccess || t.tn_a == t.tiles_n) return e;
    // the remaining weight rows as tiles of 128 weight rows
    a.n_begin = (int)(t.tn_a * bn_of(8));
    const int rest = w.n - a.n_begin;
    const int nb = (rest + bn_of(4) - 1) / bn_of(4);
    const int tm = tail_tm(m, nb, compute_units());
    const dim3 gb((unsigned)(((m + 32 * tm - 1) / (32 * tm)) * nb));
    if (tm == 1) return launch_big_mode<1, 4, kDense>(w.format, a, gb, s);
    if (tm == 2) return launch_big_mode<2, 4, kDense>(w.format, a, gb, s);
    return launch_big_mode<4, 4, kDense>(w.format, a, gb, s);
  }
  // up to 256 rows: split K when the caller's workspace holds the partials
  SmallPlan p = small_m_plan(w, m, true);
  if (p.sk > 1 && !(workspace && workspace_bytes >= gemm_big_workspace(w, m)))
    p = small_m_plan(w, m, false);
  if (p.sk > 1) {
    a.splits = p.sk;
    a.sps = (w.k / kBK + p.sk - 1) / p.sk;
    a.counters = (uint32_t *)workspace;
    a.partials = (float *)((char *)workspace + split_counters_bytes(w, m));
    // the workspace may hold anything: the tile counters start from zero,
    // cleared by a kernel ahead of the split launch on the same stream
    const hipError_t e = launch_zero(workspace, split_counters_bytes(w, m), s);
    if (e != hipSuccess) return e;
  }
  const int tm = p.tm;
  if (tm == 1) return launch_big_mode<1, 4, kDense>(w.format, a, grid(32, bn_of(4)), s);
  if (tm == 2) return launch_big_mode<2, 4, kDense>(w.format, a, grid(64, bn_of(4)), s);
  return launch_big_mode<4, 4, kDense>(w.format, a, grid(128, bn_of(4)), s);
}

// the grouped launches' 1-D grid: routing tiles (rounded up to a multiple
// of 16: 8 XCDs x tile pairs) x column blocks of bn weight rows
static dim3 moe_grid(int max_tiles, int n, int bn) {
  const unsigned ncb = (unsigned)((n + bn - 1) / bn);
  return dim3((unsigned)((max_tiles + 15) / 16 * 16) * ncb);
}

hipError_t launch_moe_big_gate_up(const qmm_weight &gu, const void *x, const MoeTables &t,
                                  int max_tiles, int tile_rows, hipStream_t s) {
  GemmArgs a = big_args(gu);
  a.x = (const uint16_t *)x;
  a.tiles = t.tiles;
  a.n_tiles = t.n_tiles;
  a.token_of_row = t.token_of_row;
  a.h = t.h;
  a.inter = gu.n / 2;
  // each workgroup covers 128 intermediate columns (256 interleaved rows) of
  // one routing tile (tile_rows activation rows); a 32-row tile is four X load
  // instructions a slice, so it takes 4 waves (64 columns)
  const dim3 grid = moe_grid(max_tiles, gu.n, bn_of(8));
  switch (tile_rows) {
    case 32: return launch_big_mode<1, 4, kMoeGateUp>(
        gu.format, a, moe_grid(max_tiles, gu.n, bn_of(4)), s);
    case 64: return launch_big_mode<2, 8, kMoeGateUp>(gu.format, a, grid, s);
    case 128: return launch_big_mode<4, 8, kMoeGateUp>(gu.format, a, grid, s);
    case 192: return launch_big_mode<6, 8, kMoeGateUp>(gu.format, a, grid, s);
    default: return launch_big_mode<8, 8, kMoeGateUp>(gu.format, a, grid, s);
  }
}

hipError_t launch_moe_big_down(const qmm_weight &dn, const MoeTables &t, int max_tiles,
                               int tile_rows, hipStream_t s) {
  GemmArgs a = big_args(dn);
  a.tiles = t.tiles;
  a.n_tiles = t.n_tiles;
  a.h = t.h;
  a.d = t.d;
  a.slot_of_row = t.slot_of_row;
  a.inter = dn.k;
  const dim3 grid = moe_grid(max_tiles, dn.n, bn_of(8));
  switch (tile_rows) {
    case 32: return launch_big_mode<1, 4, kMoeDown>(
        dn.format, a, moe_grid(max_tiles, dn.n, bn_of(4)), s);
    case 64: return launch_big_mode<2, 8, kMoeDown>(dn.format, a, grid, s);
    case 128: return launch_big_mode<4, 8, kMoeDown>(dn.format, a, grid, s);
    case 192: return launch_big_mode<6, 8, kMoeDown>(dn.format, a, grid, s);
    default: return launch_big_mode<8, 8, kMoeDown>(dn.format, a, grid, s);
  }
}

}  // namespace qmm
