// qgemm with 256-row weight tiles, for prefill with many activation rows
// (dense mode).  Same arithmetic as gemm.hip -- each weight decoded once per
// tile into bfloat16 ("TurboEXL3" section 4.1: decode once, multiply many
// times), v_mfma_f32_16x16x32_bf16, float32 sums over K in slice order -- on
// a different data path:
//
//   * the activation tile (TM x 16 rows) goes from memory straight into LDS
//     (buffer_load_dwordx4 ... lds), three 64-wide K slices in flight, with no
//     register staging; its 16-byte chunks are XOR-swizzled by row so that the
//     MFMA operand reads of a lane group fall on distinct LDS bank groups;
//   * the weights never pass through LDS: each wave owns 16 TN rows of the
//     tile, loads their codes and scales itself (registers, three slices
//     ahead) and decodes them straight into its MFMA A operands.  The K order
//     inside a slice is permuted (lane group g of a 16-lane row holds K values
//     16g .. 16g+15, the first 8 for the slice's first MFMA, the rest for the
//     second) and the activation operand is read in the same order, so each
//     lane decodes one contiguous 16-weight run of one row;
//   * a wave computes TN x TM MFMA tiles (16 TN rows of W x 16 TM rows of X).
//     From 257 rows of X on: 8 waves of 32 W rows x 256 X rows (TN = 2,
//     TM = 16), so that each decoded weight feeds 32 MFMAs of its slice, as
//     do the grouped MoE modes (256 rows is the routing table's tile height).
//     Up to 256 rows: 4 waves of 32 x 128 (more workgroups for small calls).
//     A wave holds at most 128 float32 accumulators; two waves share a SIMD.
//     (One wave of 64 x 256, with 256 accumulators, spilled.)
//
// Per slice and wave (dense): 64 MFMAs, 32 decoded weights per lane, 32 KB of
// LDS operand reads; per workgroup 32 KB of activations and 9-14 KB of
// weight codes from memory, about half of what the 128 x 128 tiles of gemm.hip
// move per flop.
#include <atomic>
#include <cstdlib>

#include "gemm_common.h"

namespace qmm {
namespace {

using namespace gemm;

constexpr int kStages = 3;      // LDS stages of X = slices in flight
constexpr int kXRow = kBK * 2;  // bytes of one X row in a slice

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 bytes per lane from buffer `r` (lane's byte offset voff + soff) to LDS at
// dst + 16 * lane (an ordinary function, so that host passes over the kernel
// templates never see the LDS address space)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void *dst, uint32_t voff,
                                                  uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, voff, soff, 0, 0);
}

// A 16-weight run of one row: codes and what scales them.
struct Run {
  uint2 q;     // 16 codes (Q6_K: low nibbles), value 2i in the low nibble of byte i
  uint32_t h;  // Q6_K: 2 high bits per value
  uint32_t s;  // affine (scale, bias) / E8M0 / E4M3 / Q6_K int8 sub-block scale
  uint32_t d;  // Q6_K super-block scale
};

// Buffer descriptors and the per-lane constant parts of the weight offsets
// (the lane's row and run); the slice's part goes in the scalar offset.
struct WSrc {
  __amdgpu_buffer_rsrc_t rc, rh, rs, rs2;
  uint32_t v_code[4], v_hi[4], v_s[4], v_d[4];  // per W tile (TN <= 4)
};

template <int FMT>
__device__ __forceinline__ Run load_run(const WSrc &w, int i, int s) {
  Run p;
  p.q = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(w.rc, w.v_code[i], s * (kBK / 2), 0));
  if constexpr (FMT == QMM_AFFINE4_G64) {
    p.s = __builtin_amdgcn_raw_buffer_load_b32(w.rs, w.v_s[i], s * 4, 0);
  } else if constexpr (FMT == QMM_MXFP4) {
    p.s = __builtin_amdgcn_raw_buffer_load_b8(w.rs, w.v_s[i], s * 2, 0);
  } else if constexpr (FMT == QMM_NVFP4) {
    p.s = __builtin_amdgcn_raw_buffer_load_b8(w.rs, w.v_s[i], s * 4, 0);
  } else {
    p.h = __builtin_amdgcn_raw_buffer_load_b32(w.rh, w.v_hi[i], s * (kBK / 4), 0);
    p.s = __builtin_amdgcn_raw_buffer_load_b8(w.rs, w.v_s[i], s * 4, 0);
    p.d = __builtin_amdgcn_raw_buffer_load_b16(w.rs2, w.v_d[i], (s / 4) * 2, 0);
  }
  return p;
}

// The run's 16 weights as bfloat16: values 0-7 -> lo, 8-15 -> hi.
template <int FMT>
__device__ __forceinline__ void decode_run(const Run &p, bf16x8_t &lo, bf16x8_t &hi) {
  const uint32_t w[2] = {p.q.x, p.q.y};
  uint32_t o[8];
  if constexpr (FMT == QMM_AFFINE4_G64) {
    const float s = half_to_float(p.s & 0xFFFFu), b = half_to_float(p.s >> 16);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // even codes to the bytes of one word, odd codes to another, so that
      // each code becomes a float with one v_cvt_f32_ubyteN
      uint32_t ev = w[j] & 0x0F0F0F0Fu, od = (w[j] >> 4) & 0x0F0F0F0Fu;
      asm volatile("" : "+v"(ev));
      asm volatile("" : "+v"(od));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[4 * j + i] = pack_bf16(__builtin_fmaf(s, (float)((ev >> (8 * i)) & 0xFFu), b),
                                 __builtin_fmaf(s, (float)((od >> (8 * i)) & 0xFFu), b));
    }
  } else if constexpr (FMT == QMM_MXFP4) {
    const float sc = e8m0_to_float(p.s);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      o[4 * j + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 0));
      o[4 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 1));
      o[4 * j + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 2));
      o[4 * j + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[j], sc, 3));
    }
  } else if constexpr (FMT == QMM_NVFP4) {
    float sc, unused;
    e4m3x2_to_float(p.s, sc, unused);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // E2M1 pair -> two float32 (unit scale), times the E4M3 block scale
      // (exact), -> bfloat16 pair (exact)
      const f32x2_t e[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 0),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 1),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 2),
                            __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 3)};
#pragma unroll
      for (int i = 0; i < 4; ++i) o[4 * j + i] = pack_bf16(e[i][0] * sc, e[i][1] * sc);
    }
  } else {  // Q6_K: (d * sc) * (q - 32), exact in float32
    const float dsc = half_to_float(p.d) * (float)(int8_t)(p.s & 0xFFu);
#pragma unroll
    for (int v = 0; v < 16; v += 2) {
      const uint32_t q0 = ((w[v / 8] >> (4 * (v % 8))) & 15u) | (((p.h >> (2 * v)) & 3u) << 4);
      const uint32_t q1 = ((w[v / 8] >> (4 * (v % 8) + 4)) & 15u) | (((p.h >> (2 * v + 2)) & 3u) << 4);
      o[v / 2] = pack_bf16(dsc * (float)((int)q0 - 32), dsc * (float)((int)q1 - 32));
    }
  }
  lo = __builtin_bit_cast(bf16x8_t, u32x4_t{o[0], o[1], o[2], o[3]});
  hi = __builtin_bit_cast(bf16x8_t, u32x4_t{o[4], o[5], o[6], o[7]});
}

// Physical 16-byte chunk offset of X row `row` in LDS: logical chunk c sits at
// c ^ swz(row).  The 16 rows read by one ds_read_b128 lane group (same logical
// chunk) then land on distinct bank groups; measured on gfx950 at 119 TB/s of
// LDS reads against 71 TB/s for a plain (row / 2) swizzle.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// s_waitcnt with vmcnt <= n and the other counters left free (gfx9 encoding)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int FMT>
constexpr int w_loads_per_run() { return FMT == QMM_Q6_K ? 4 : 2; }

// A wave computes TN x TM MFMA tiles: 16 TN rows of W x 16 TM rows of X;
// the workgroup's WAVES waves cover BN = 16 TN WAVES rows of W, all sharing
// the BM = 16 TM rows of X.  MODE as in gemm.hip: dense, or the grouped MoE
// gate/up (rows of x gathered by token, gate and up weight rows interleaved,
// SwiGLU epilogue) and down products over the routing tile table (tiles of BM
// grouped rows, one expert each).
template <int FMT, int TN, int TM, int WAVES, int MODE>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_big_kernel(GemmArgs a) {
  constexpr int kTN = TN;
  constexpr int WROWS = 16 * TN;  // W rows per wave
  constexpr int kBN = WROWS * WAVES;
  constexpr int BM = 16 * TM;
  constexpr int kXStage = BM * kXRow;  // bytes per LDS stage
  constexpr int XI = BM / (8 * WAVES);  // X load instructions per wave and slice (8 rows each)
  extern __shared__ __align__(16) uint8_t lds[];  // kStages x [BM rows][128 bytes]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int m0, n0, mrows, wrow0 = 0, expert = 0;
  if constexpr (MODE == kDense) {
    const int tiles_m = (a.m + BM - 1) / BM;
    m0 = (blockIdx.x % tiles_m) * BM;
    n0 = (blockIdx.x / tiles_m) * kBN;
    mrows = a.m - m0;
  } else {
    if (blockIdx.x >= *a.n_tiles) return;  // beyond this call's tiles (whole workgroup)
    const uint32_t *t = a.tiles + 3 * blockIdx.x;
    expert = (int)t[0];
    m0 = (int)t[1];
    mrows = (int)t[2];
    n0 = blockIdx.y * kBN;
    wrow0 = expert * a.n;  // first row of the expert's matrix
  }
  const int slices = a.k / kBK;
  const uint32_t k = (uint32_t)a.k;
  const int lr = lane & 15, g = lane >> 4;

  // activations: wave w fills rows (BM/4) w .. of a stage, 8 rows per
  // instruction; lane l of instruction i writes LDS chunk l % 8 of row
  // (BM/4) w + 8i + l / 8, which holds the row's logical chunk (l % 8) ^ swz(row)
  // (grouped modes: the routing tables index valid rows of x or h, whose
  // extent the call does not pass; their descriptor spans the 32-bit range)
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

  // weights: lane (lr, g) of tile i holds tile row j = 64w + 16i + lr, run g;
  // tile row j is weight row n0 + j, or in the gate/up mode gate or up row
  // n0/2 + j/2 of the expert (even j gate, odd j up)
  WSrc ws;
  {
    const size_t rows = (size_t)a.wrows;
    ws.rc = make_rsrc(a.codes, (uint32_t)(rows * (k / 2)));
    ws.rh = make_rsrc(a.codes_hi, a.codes_hi ? (uint32_t)(rows * (k / 4)) : 0u);
    ws.rs = make_rsrc(a.scales, (uint32_t)(rows * (k / (FMT == QMM_AFFINE4_G64 ? 16 : (FMT == QMM_MXFP4 ? 32 : 16)))));
    ws.rs2 = make_rsrc(a.scales2, a.scales2 ? (uint32_t)(rows * (k / 256) * 2) : 0u);
#pragma unroll
    for (int i = 0; i < kTN; ++i) {
      const int j = WROWS * wave + 16 * i + lr;
      uint32_t r;
      if constexpr (MODE == kMoeGateUp)
        r = (uint32_t)(wrow0 + ((j & 1) ? a.inter : 0) + min(n0 / 2 + j / 2, a.inter - 1));
      else
        r = (uint32_t)(wrow0 + min(n0 + j, a.n - 1));
      ws.v_code[i] = r * (k / 2) + 8 * g;
      ws.v_hi[i] = r * (k / 4) + 4 * g;
      ws.v_s[i] = FMT == QMM_AFFINE4_G64 ? r * (k / 64) * 4
                : FMT == QMM_MXFP4       ? r * (k / 32) + (g >> 1)
                                         : r * (k / 16) + g;
      ws.v_d[i] = r * (k / 256) * 2;
    }
  }
  Run wr[kStages][kTN];
  auto load_w = [&](int s, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kTN; ++i) wr[st][i] = load_run<FMT>(ws, i, s);
  };

  f32x4_t acc[kTN][TM];
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // operand reads of the activation tile: row 16j + lr, logical chunk 2g + kk
  // at physical chunk (2g + kk) ^ swz(lr) (swz of 16j + lr is swz(lr))
  const uint32_t xo0 = (uint32_t)lr * kXRow + (uint32_t)(((2 * g) ^ swz(lr)) * 16);
  const uint32_t xo1 = (uint32_t)lr * kXRow + (uint32_t)(((2 * g + 1) ^ swz(lr)) * 16);

  // slices 0 .. kStages-2 in flight; every iteration then issues one more
  // (the last slice again past the end, so that every wave issues the same
  // loads and the counts below hold)
  constexpr int kLoadsPerSlice = XI + kTN * w_loads_per_run<FMT>();
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p) {
    const int sp = min(p, slices - 1);
    load_x(sp);
    load_w(sp, p);
  }

  for (int s0 = 0; s0 < slices; s0 += kStages) {
#pragma unroll
    for (int u = 0; u < kStages; ++u) {
      const int s = s0 + u;
      if (s >= slices) break;  // uniform
      // this wave's share of slice s is in LDS once at most the loads issued
      // after it (kStages - 2 slices) are outstanding; the barrier then makes
      // every wave's share visible and frees the stage read in iteration s - 1
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((kStages - 2) * kLoadsPerSlice));
      __syncthreads();
      const int sn = min(s + kStages - 1, slices - 1);
      load_x(sn);
      load_w(sn, (u + kStages - 1) % kStages);

      bf16x8_t af[kTN][2];
#pragma unroll
      for (int i = 0; i < kTN; ++i) decode_run<FMT>(wr[u][i], af[i][0], af[i][1]);

      const uint8_t *st = lds + (s % kStages) * kXStage;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // all of this half-slice's activation operands first, so that the
        // MFMAs below do not wait on LDS after every four
        bf16x8_t bfr[TM];
#pragma unroll
        for (int j = 0; j < TM; ++j) bfr[j] = *(const bf16x8_t *)(st + j * 16 * kXRow + (kk ? xo1 : xo0));
        // (Q6_K's longer decode leaves no registers for that)
        if constexpr (FMT != QMM_Q6_K) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < TM; ++j)
#pragma unroll
          for (int i = 0; i < kTN; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i][kk], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // epilogue: lane holds D[n = 4*(lane/16) + r][m = lane % 16] of each tile
  const float gs = (FMT == QMM_NVFP4 && a.tensor_scale) ? a.tensor_scale[expert] : 1.0f;
#pragma unroll
  for (int i = 0; i < kTN; ++i) {
    const int nl = WROWS * wave + 16 * i + 4 * g;  // tile row of v[0]
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int ml = 16 * j + lr;
      if (ml >= mrows) continue;
      const int m = m0 + ml;
      float v[4] = {acc[i][j][0] * gs, acc[i][j][1] * gs, acc[i][j][2] * gs, acc[i][j][3] * gs};
      if constexpr (MODE == kMoeGateUp) {
        // (gate, up, gate, up) of two consecutive intermediate columns; SwiGLU
        // in float32: h = silu(g) * u, silu(g) = g / (1 + e^-g)
        const int col = n0 / 2 + nl / 2;  // even, and I is even
        if (col < a.inter) {
          const float h0 = v[0] / (1.0f + expf(-v[0])) * v[1];
          const float h1 = v[2] / (1.0f + expf(-v[2])) * v[3];
          *(uint32_t *)(a.h + (size_t)m * a.inter + col) = pack_bf16(h0, h1);
        }
        continue;
      } else if constexpr (MODE == kMoeDown) {
        const int nb = n0 + nl;
        if (nb + 3 < a.n) {
          *(float4 *)(a.d + (size_t)m * a.n + nb) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          for (int r = 0; r < 4 && nb + r < a.n; ++r) a.d[(size_t)m * a.n + nb + r] = v[r];
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
          float t = v[r];
          if (a.residual) t += bf_lo(a.residual[base + r]);
          a.y[base + r] = __builtin_bit_cast(uint16_t, (__bf16)t);
        }
      }
    }
  }
}

template <int FMT, int TN, int TM, int WAVES, int MODE>
hipError_t launch_big(const GemmArgs &a, dim3 grid, hipStream_t s) {
  static_assert(MODE == kDense || 16 * TM == kMoeTileRows,
                "X tiles are the routing table's tiles of kMoeTileRows rows");
  constexpr size_t lds = (size_t)kStages * 16 * TM * kXRow;
  // more than 64 KiB of dynamic LDS must be allowed once per device
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void *)gemm_big_kernel<FMT, TN, TM, WAVES, MODE>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((gemm_big_kernel<FMT, TN, TM, WAVES, MODE>), grid, dim3(64 * WAVES), lds, s, a);
  return hipGetLastError();
}

template <int TN, int TM, int WAVES, int MODE>
hipError_t launch_big_mode(int format, const GemmArgs &a, dim3 grid, hipStream_t s) {
  switch (format) {
    case QMM_AFFINE4_G64: return launch_big<QMM_AFFINE4_G64, TN, TM, WAVES, MODE>(a, grid, s);
    case QMM_MXFP4: return launch_big<QMM_MXFP4, TN, TM, WAVES, MODE>(a, grid, s);
    case QMM_NVFP4: return launch_big<QMM_NVFP4, TN, TM, WAVES, MODE>(a, grid, s);
    default: return launch_big<QMM_Q6_K, TN, TM, WAVES, MODE>(a, grid, s);
  }
}

// workgroups' rows of W for a TN x WAVES configuration
constexpr int bn_of(int tn, int waves) { return 16 * tn * waves; }

// compute units of the current device (cached per device)
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

GemmArgs big_args(const qmm_weight &w) {
  GemmArgs a{};
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

}  // namespace

bool gemm_big_fits(const qmm_weight &w, size_t x_rows) {
  // 32-bit buffer offsets for X and every weight plane
  return x_rows * (size_t)w.k * 2 < (1ull << 32) && (size_t)w.batch * w.n * w.k < (1ull << 32);
}

hipError_t launch_gemm_big(const qmm_weight &w, const void *x, int m, const void *residual, void *y,
                           hipStream_t s) {
  GemmArgs a = big_args(w);
  a.x = (const uint16_t *)x;
  a.residual = (const uint16_t *)residual;
  a.y = (uint16_t *)y;
  a.m = m;
  auto grid = [&](int bm, int bn) {
    return dim3((unsigned)(((m + bm - 1) / bm) * ((w.n + bn - 1) / bn)));
  };
  // 8 waves of 32 W rows x 256 X rows: each decoded weight feeds twice the
  // MFMAs of the 4-wave 64 x 128 form (measured 1.3x faster from M = 512 on);
  // or 8 waves of 32 x 192 where that leaves fewer idle compute units in the
  // last round of workgroups (one workgroup per compute unit; a 192-row round
  // takes about 0.85 of a 256-row one): M = 2048 at 17408 rows is 544
  // workgroups of 256 (2.1 rounds) or 748 of 192 (2.9 rounds), measured 1.14x
  // faster; M = 300 and 512 1.2x, M >= 3072 no gain.  Up to 256 rows of X: 4 waves of 32 x 128, whose 128-row W tiles
  // give a 128-row call 136 workgroups (1.9x faster than the LDS-staged kernel
  // at M = 128, 1.4x at M = 256).
  int cfg = 1;
  if (m > 256) {
    const long nt = (w.n + bn_of(2, 8) - 1) / bn_of(2, 8), cus = compute_units();
    auto rounds = [&](int bm) { return ((m + bm - 1) / bm * nt + cus - 1) / cus; };
    cfg = 17 * rounds(192) < 20 * rounds(256) ? 4 : 0;
  }
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_BIG_CFG")) cfg = atoi(e);
  if (cfg == 2) return launch_big_mode<4, 8, 4, kDense>(w.format, a, grid(128, bn_of(4, 4)), s);
#endif
  if (cfg == 0) return launch_big_mode<2, 16, 8, kDense>(w.format, a, grid(256, bn_of(2, 8)), s);
  if (cfg == 4) return launch_big_mode<2, 12, 8, kDense>(w.format, a, grid(192, bn_of(2, 8)), s);
  return launch_big_mode<2, 8, 4, kDense>(w.format, a, grid(128, bn_of(2, 4)), s);
}

hipError_t launch_moe_big_gate_up(const qmm_weight &gu, const void *x, const MoeTables &t,
                                  int max_tiles, hipStream_t s) {
  GemmArgs a = big_args(gu);
  a.x = (const uint16_t *)x;
  a.tiles = t.tiles;
  a.n_tiles = t.n_tiles;
  a.token_of_row = t.token_of_row;
  a.h = t.h;
  a.inter = gu.n / 2;
  // each workgroup covers 128 intermediate columns (256 interleaved rows)
  constexpr int bn = bn_of(2, 8);
  return launch_big_mode<2, 16, 8, kMoeGateUp>(gu.format, a, dim3(max_tiles, (gu.n + bn - 1) / bn), s);
}

hipError_t launch_moe_big_down(const qmm_weight &dn, const MoeTables &t, int max_tiles,
                               hipStream_t s) {
  GemmArgs a = big_args(dn);
  a.tiles = t.tiles;
  a.n_tiles = t.n_tiles;
  a.h = t.h;
  a.d = t.d;
  a.inter = dn.k;
  constexpr int bn = bn_of(2, 8);
  return launch_big_mode<2, 16, 8, kMoeDown>(dn.format, a, dim3(max_tiles, (dn.n + bn - 1) / bn), s);
}

}  // namespace qmm
