// qgemm: prefill matrix multiply Y[m][n] = g * sum_k x[m][k] w[n][k] (+ r[m][n]),
// bf16 out, for many activation rows.  "Decode once, multiply many times"
// ("TurboEXL3" section 4.1): per K-slice of 64, a workgroup decodes its BN x 64
// tile of weights once into LDS as bfloat16 -- the decoded weights never reach
// device memory -- and multiplies it against its BM x 64 tile of activations on
// the matrix cores (v_mfma_f32_16x16x32_bf16, float32 accumulation).
//
// Tiles: a workgroup of 4 waves (2 along n x 2 along m) owns BN rows of W and
// BM rows of X; each wave computes (BN/2) x (BM/2) outputs as 16 x 16 MFMA
// tiles.  The MFMA's A operand is the weight tile (rows n) and its B operand the
// activation tile (columns m), so each lane's four accumulators are four
// consecutive n of one m: one 8-byte store per tile in the epilogue.
//
// Pipeline: two LDS stages.  While the MFMAs of slice s run, the global loads of
// slice s+1 (activations as 16-byte pieces, codes and block scales) are in
// flight in registers; afterwards the weights are decoded and both tiles are
// written to the other stage.  One barrier per slice.
//
// Decode to bfloat16 per format (the weight is rounded once more, to bf16, as
// any 16-bit-operand multiply must; E2M1 x E8M0 and E2M1 x E4M3 are exact in
// bf16, affine and Q6_K values are rounded to nearest even):
//   affine: fma(s, q, b) in float32 -> bf16
//   MXFP4:  v_cvt_scalef32_pk_bf16_fp4 with the power-of-two scale (exact)
//   NVFP4:  E2M1 -> float32, times the E4M3 block scale (exact), -> bf16; the
//           tensor multiplier g is applied to the float32 sums in the epilogue
//   Q6_K:   (d * sc) * (q - 32) in float32 (exact) -> bf16
#include <algorithm>
#include <atomic>
#include <cstdlib>

#include "gemm_common.h"

namespace qmm {
namespace {

using namespace gemm;

template <int FMT, int BM, int BN, int MODE, int PD>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  constexpr int TN = BN / 32, TM = BM / 32;      // 16x16 tiles per wave along n and m
  constexpr int XP = BM * (kBK / 8) / 256;       // 16-byte activation pieces per thread
  constexpr int WP = BN * (kBK / 32) / 256;      // 32-weight pieces per thread
  static_assert(XP >= 1 && WP >= 1, "tile too small for 256 threads");
  constexpr int STAGE = (BM + BN) * kRowH;       // bf16 per LDS stage
  extern __shared__ __align__(16) uint16_t lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  int m0, n0, mrows, wrow0 = 0, expert = 0;
  if constexpr (MODE == kDense) {
    const int tiles_m = (a.m + BM - 1) / BM;
    m0 = (blockIdx.x % tiles_m) * BM;
    n0 = (blockIdx.x / tiles_m) * BN;
    mrows = a.m - m0;
  } else {
    if (blockIdx.x >= *a.n_tiles) return;            // beyond this call's tiles
    const uint32_t *t = a.tiles + 3 * blockIdx.x;
    expert = (int)t[0];
    m0 = (int)t[1];
    mrows = (int)t[2];
    n0 = blockIdx.y * BN;
    wrow0 = expert * a.n;                              // first row of the expert's matrix
  }
  const int slices = a.k / kBK;
  // weight row of tile row j (gate/up interleaved in the gate/up mode)
  auto wrow = [&](int j) __attribute__((always_inline)) {
    if constexpr (MODE == kMoeGateUp) {
      const int i = n0 / 2 + j / 2;
      return wrow0 + ((j & 1) ? a.inter + i : i);
    } else {
      return wrow0 + min(n0 + j, a.n - 1);
    }
  };

  // global -> register loads of one slice, into register stage `r`
  u32x4_t xr[PD][XP];
  Piece wr[PD][WP];
  auto load_slice = [&](int s, int r) __attribute__((always_inline)) {
    const int k0 = s * kBK;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = tid + 256 * i, row = p / (kBK / 8), col = p % (kBK / 8);
      const int rr = m0 + min(row, mrows - 1);
      const uint16_t *src;
      if constexpr (MODE == kDense) src = a.x + (size_t)rr * a.k;
      else if constexpr (MODE == kMoeGateUp) src = a.x + (size_t)a.token_of_row[rr] * a.k;
      else src = a.h + (size_t)rr * a.k;
      xr[r][i] = *(const u32x4_t *)(src + k0 + col * 8);
    }
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int p = tid + 256 * i, row = p / 2, half = p % 2;
      wr[r][i] = load_piece<FMT>(a, wrow(row), k0 + half * 32);
    }
  };
  // decode register stage `r` and write it into LDS stage `st`
  auto store_slice = [&](int r, int st) __attribute__((always_inline)) {
    uint16_t *xs = lds + st * STAGE;
    uint16_t *ws = xs + BM * kRowH;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int p = tid + 256 * i, row = p / (kBK / 8), col = p % (kBK / 8);
      *(u32x4_t *)(xs + row * kRowH + col * 8) = xr[r][i];
    }
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int p = tid + 256 * i, row = p / 2, half = p % 2;
      uint32_t o[16];
      decode_piece<FMT>(wr[r][i], o);
      u32x4_t *dst = (u32x4_t *)(ws + row * kRowH + half * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = u32x4_t{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    }
  };

  f32x4_t acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // slices 0 .. PD-1 in flight, slice 0 decoded into LDS stage 0
#pragma unroll
  for (int r = 0; r < PD; ++r)
    if (r < slices) load_slice(r, r);
  store_slice(0, 0);
  __syncthreads();

  // Slice q lives in register stage q % PD and LDS stage q % 2.  Iteration q:
  // the loads of slice q + PD go to register stage q % PD (slice q is already
  // in LDS), the MFMAs run on LDS stage q % 2, then slice q + 1 is decoded
  // into the other LDS stage; one barrier per slice.
  const int lr = lane & 15, lk = (lane >> 4) * 8;  // operand row within a 16-tile, k offset
  for (int s0 = 0; s0 < slices; s0 += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int s = s0 + u;
      if (s >= slices) break;  // uniform
      if (s + PD < slices) load_slice(s + PD, u);
      const uint16_t *xs = lds + (s & 1) * STAGE;
      const uint16_t *ws = xs + BM * kRowH;
#pragma unroll
      for (int kk = 0; kk < kBK; kk += 32) {
        bf16x8_t af[TN], bfr[TM];
#pragma unroll
        for (int i = 0; i < TN; ++i)
          af[i] = *(const bf16x8_t *)(ws + (wn * (BN / 2) + i * 16 + lr) * kRowH + kk + lk);
#pragma unroll
        for (int j = 0; j < TM; ++j)
          bfr[j] = *(const bf16x8_t *)(xs + (wm * (BM / 2) + j * 16 + lr) * kRowH + kk + lk);
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int j = 0; j < TM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (s + 1 < slices) store_slice((u + 1) % PD, (s + 1) & 1);
      __syncthreads();
    }
  }

  // epilogue: lane holds D[n = 4*(lane/16) + r][m = lane % 16] of each tile
  const float g = (FMT == QMM_NVFP4 && a.tensor_scale) ? a.tensor_scale[expert] : 1.0f;
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int ml = wm * (BM / 2) + j * 16 + lr;
      const int nl = wn * (BN / 2) + i * 16 + (lane >> 4) * 4;
      if (ml >= mrows) continue;
      const int m = m0 + ml;
      float v[4] = {acc[i][j][0] * g, acc[i][j][1] * g, acc[i][j][2] * g, acc[i][j][3] * g};
      if constexpr (MODE == kMoeGateUp) {
        // (gate, up, gate, up) of two consecutive intermediate columns; SwiGLU
        // in float32: h = silu(g) * u, silu(g) = g / (1 + e^-g)
        const int col = n0 / 2 + nl / 2;
        const float h0 = v[0] / (1.0f + expf(-v[0])) * v[1];
        const float h1 = v[2] / (1.0f + expf(-v[2])) * v[3];
        *(uint32_t *)(a.h + (size_t)m * a.inter + col) = pack_bf16(h0, h1);
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

template <int FMT, int BM, int BN, int MODE, int PD>
hipError_t launch_tile(const GemmArgs &a, dim3 grid, hipStream_t s) {
  constexpr size_t lds = 2 * (size_t)(BM + BN) * kRowH * 2;
  // more than 64 KiB of dynamic LDS must be allowed once per device
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void *)gemm_kernel<FMT, BM, BN, MODE, PD>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((gemm_kernel<FMT, BM, BN, MODE, PD>), grid, dim3(256), lds, s, a);
  return hipGetLastError();
}

// slices of global loads in flight (register stages)
int gemm_depth() {
  int pd = 1;  // deeper register prefetch measured slower (it costs occupancy)
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_GEMM_PD")) pd = atoi(e);
#endif
  return pd;
}

// activation rows per tile: kGemmBM dense, the routing table's tiles grouped
template <int MODE>
constexpr int kTileM = MODE == kDense ? kGemmBM : kMoeTileRows;

template <int FMT, int MODE>
hipError_t launch_fd(const GemmArgs &a, dim3 grid, hipStream_t s) {
  switch (gemm_depth()) {
#ifdef QMM_TUNE
    case 2: return launch_tile<FMT, kTileM<MODE>, 128, MODE, 2>(a, grid, s);
    case 3: return launch_tile<FMT, kTileM<MODE>, 128, MODE, 3>(a, grid, s);
#endif
    default: return launch_tile<FMT, kTileM<MODE>, 128, MODE, 1>(a, grid, s);
  }
}

template <int MODE>
hipError_t launch_mode(int format, const GemmArgs &a, dim3 grid, hipStream_t s) {
  switch (format) {
    case QMM_AFFINE4_G64: return launch_fd<QMM_AFFINE4_G64, MODE>(a, grid, s);
    case QMM_MXFP4: return launch_fd<QMM_MXFP4, MODE>(a, grid, s);
    case QMM_NVFP4: return launch_fd<QMM_NVFP4, MODE>(a, grid, s);
    default: return launch_fd<QMM_Q6_K, MODE>(a, grid, s);
  }
}

GemmArgs weight_args(const qmm_weight &w) {
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

size_t gemm_workspace_size(const qmm_weight &w, int m) {
  return gemm_big_fits(w, (size_t)m) ? gemm_big_workspace(w, m) : 0;
}

hipError_t launch_gemm(const qmm_weight &w, const void *x, int m, const void *residual, void *y,
                       void *workspace, size_t workspace_bytes, hipStream_t s) {
  // weights decoded straight into MFMA operands (gemm_big.hip) wherever its
  // 32-bit offsets reach; this LDS-staged kernel otherwise
  bool big = true;
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_GEMM_BIG")) big = atoi(e) != 0;
#endif
  if (big && gemm_big_fits(w, (size_t)m))
    return launch_gemm_big(w, x, m, residual, y, workspace, workspace_bytes, s);
  GemmArgs a = weight_args(w);
  a.x = (const uint16_t *)x;
  a.residual = (const uint16_t *)residual;
  a.y = (uint16_t *)y;
  a.m = m;
  const unsigned blocks = (unsigned)(((m + kGemmBM - 1) / kGemmBM) * ((w.n + 127) / 128));
  return launch_mode<kDense>(w.format, a, dim3(blocks), s);
}

hipError_t launch_moe_gemm_gate_up(const qmm_weight &gu, const void *x, const MoeTables &t,
                                   int max_tiles, hipStream_t s) {
  GemmArgs a = weight_args(gu);
  a.x = (const uint16_t *)x;
  a.tiles = t.tiles;
  a.n_tiles = t.n_tiles;
  a.token_of_row = t.token_of_row;
  a.h = t.h;
  a.inter = gu.n / 2;
  // each workgroup covers 64 intermediate columns (128 interleaved rows)
  return launch_mode<kMoeGateUp>(gu.format, a, dim3(max_tiles, (gu.n + 127) / 128), s);
}

hipError_t launch_moe_gemm_down(const qmm_weight &dn, const MoeTables &t, int max_tiles,
                                hipStream_t s) {
  GemmArgs a = weight_args(dn);
  a.tiles = t.tiles;
  a.n_tiles = t.n_tiles;
  a.h = t.h;
  a.d = t.d;
  a.inter = dn.k;
  return launch_mode<kMoeDown>(dn.format, a, dim3(max_tiles, (dn.n + 127) / 128), s);
}

}  // namespace qmm
