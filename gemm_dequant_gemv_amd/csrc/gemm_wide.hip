// qgemm for many activation rows: the same "decode once, multiply many times"
// scheme as gemm.hip ("TurboEXL3" section 4.1) with 256 x 256 output tiles.
//
// A workgroup of 8 waves (2 along n x 4 along m) owns 256 weight rows and 256
// activation rows; each wave computes a 128 x 64 block as 8 x 4 MFMA tiles
// (v_mfma_f32_16x16x32_bf16), two waves per SIMD.
// Per 64-wide K slice the workgroup decodes its 256 x 64 weight tile once into
// LDS as bfloat16 (the decoded weights never reach device memory).
//
// Pipeline: two LDS stages and two register stages.  While the MFMAs of slice
// s run from LDS stage s % 2, the global loads of slice s + 2 are in flight
// and slice s + 1 (loaded one slice earlier) is decoded and written to the
// other LDS stage afterwards; one barrier per slice.  Global loads thus have
// two slices of MFMA time to arrive.
//
// Tile order: workgroups are dealt to the 8 XCDs round-robin by id, so ids are
// remapped to give each XCD a contiguous run of tiles, m fastest: the ~32
// workgroups one XCD runs at a time share one weight tile in that XCD's L2.
#include <algorithm>
#include <atomic>

#include "gemm_common.h"

namespace qmm {
namespace {

using namespace gemm;

constexpr int kBM = 256, kBN = 256;
constexpr int kWavesN = 2, kWavesM = 4, kThreads = 64 * kWavesN * kWavesM;
constexpr int kWaveN = kBN / kWavesN, kWaveM = kBM / kWavesM;  // 128 x 64 per wave
constexpr int kTN = kWaveN / 16, kTM = kWaveM / 16;  // 16x16 tiles per wave along n and m
constexpr int kXP = kBM * (kBK / 8) / kThreads;       // 16-byte activation pieces per thread
constexpr int kWP = kBN * (kBK / 32) / kThreads;      // 32-weight pieces per thread
constexpr int kStage = (kBM + kBN) * kRowH;        // bf16 per LDS stage
constexpr size_t kLds = 2 * (size_t)kStage * 2;
constexpr int kXcds = 8;

template <int FMT>
__global__ __launch_bounds__(kThreads) void gemm_wide_kernel(GemmArgs a) {
  extern __shared__ __align__(16) uint16_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % kWavesN, wm = wave / kWavesN;

  const int tiles_m = (a.m + kBM - 1) / kBM;
  const int ntiles = tiles_m * ((a.n + kBN - 1) / kBN);
  const int per = (ntiles + kXcds - 1) / kXcds;
  const int t = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (t >= ntiles) return;
  const int m0 = (t % tiles_m) * kBM, n0 = (t / tiles_m) * kBN;
  const int mrows = a.m - m0;
  const int slices = a.k / kBK;

  u32x4_t xr[2][kXP];
  Piece wr[2][kWP];
  auto load_slice = [&](int s, u32x4_t (&x)[kXP], Piece (&w)[kWP]) {
    const int k0 = s * kBK;
#pragma unroll
    for (int i = 0; i < kXP; ++i) {
      const int p = tid + kThreads * i, row = p / (kBK / 8), col = p % (kBK / 8);
      const int r = m0 + min(row, mrows - 1);
      x[i] = *(const u32x4_t *)(a.x + (size_t)r * a.k + k0 + col * 8);
    }
#pragma unroll
    for (int i = 0; i < kWP; ++i) {
      const int p = tid + kThreads * i, row = p / 2, half = p % 2;
      w[i] = load_piece<FMT>(a, min(n0 + row, a.n - 1), k0 + half * 32);
    }
  };
  auto store_slice = [&](int st, const u32x4_t (&x)[kXP], const Piece (&w)[kWP]) {
    uint16_t *xs = lds + st * kStage;
    uint16_t *ws = xs + kBM * kRowH;
#pragma unroll
    for (int i = 0; i < kXP; ++i) {
      const int p = tid + kThreads * i, row = p / (kBK / 8), col = p % (kBK / 8);
      *(u32x4_t *)(xs + row * kRowH + col * 8) = x[i];
    }
#pragma unroll
    for (int i = 0; i < kWP; ++i) {
      const int p = tid + kThreads * i, row = p / 2, half = p % 2;
      uint32_t o[16];
      decode_piece<FMT>(w[i], o);
      u32x4_t *dst = (u32x4_t *)(ws + row * kRowH + half * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q) dst[q] = u32x4_t{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    }
  };

  f32x4_t acc[kTN][kTM];
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15, lk = (lane >> 4) * 8;  // operand row within a 16-tile, k offset
  auto mfma_slice = [&](int st) __attribute__((always_inline)) {
    const uint16_t *xs = lds + st * kStage;
    const uint16_t *ws = xs + kBM * kRowH;
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      // the wave's activation fragments stay in registers; weight fragments
      // are read one at a time, each feeding kTM MFMAs
      bf16x8_t bfr[kTM];
#pragma unroll
      for (int j = 0; j < kTM; ++j)
        bfr[j] = *(const bf16x8_t *)(xs + (wm * kWaveM + j * 16 + lr) * kRowH + kk + lk);
#pragma unroll
      for (int i = 0; i < kTN; ++i) {
        const bf16x8_t af = *(const bf16x8_t *)(ws + (wn * kWaveN + i * 16 + lr) * kRowH + kk + lk);
#pragma unroll
        for (int j = 0; j < kTM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // slices 0 and 1 in flight, slice 0 decoded into stage 0
  load_slice(0, xr[0], wr[0]);
  if (slices > 1) load_slice(1, xr[1], wr[1]);
  store_slice(0, xr[0], wr[0]);
  __syncthreads();

  // iteration s: MFMAs on stage s % 2; loads of slice s + 2 go to register
  // stage s % 2 (its slice s is already in LDS); slice s + 1 is decoded from
  // register stage (s + 1) % 2 into LDS stage (s + 1) % 2 after the MFMAs
  for (int s = 0; s < slices; s += 2) {
    if (s + 2 < slices) load_slice(s + 2, xr[0], wr[0]);
    mfma_slice(0);
    if (s + 1 < slices) store_slice(1, xr[1], wr[1]);
    __syncthreads();
    if (s + 1 >= slices) break;
    if (s + 3 < slices) load_slice(s + 3, xr[1], wr[1]);
    mfma_slice(1);
    if (s + 2 < slices) store_slice(0, xr[0], wr[0]);
    __syncthreads();
  }

  // epilogue: lane holds D[n = 4*(lane/16) + r][m = lane % 16] of each tile
  const float g = (FMT == QMM_NVFP4 && a.tensor_scale) ? a.tensor_scale[0] : 1.0f;
#pragma unroll
  for (int i = 0; i < kTN; ++i)
#pragma unroll
    for (int j = 0; j < kTM; ++j) {
      const int ml = wm * kWaveM + j * 16 + lr;
      const int nl = wn * kWaveN + i * 16 + (lane >> 4) * 4;
      if (ml >= mrows) continue;
      const int m = m0 + ml, nb = n0 + nl;
      float v[4] = {acc[i][j][0] * g, acc[i][j][1] * g, acc[i][j][2] * g, acc[i][j][3] * g};
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
          float tv = v[r];
          if (a.residual) tv += bf_lo(a.residual[base + r]);
          a.y[base + r] = __builtin_bit_cast(uint16_t, (__bf16)tv);
        }
      }
    }
}

template <int FMT>
hipError_t launch_wide(const GemmArgs &a, hipStream_t s) {
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void *)gemm_wide_kernel<FMT>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int ntiles = ((a.m + kBM - 1) / kBM) * ((a.n + kBN - 1) / kBN);
  const int grid = (ntiles + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((gemm_wide_kernel<FMT>), dim3(grid), dim3(kThreads), kLds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_wide(const qmm_weight &w, const void *x, int m, const void *residual,
                            void *y, hipStream_t s) {
  GemmArgs a{};
  a.codes = (const uint8_t *)w.codes;
  a.codes_hi = (const uint8_t *)w.codes_hi;
  a.scales = (const uint8_t *)w.scales;
  a.scales2 = (const uint8_t *)w.scales2;
  a.tensor_scale = w.tensor_scale;
  a.n = w.n;
  a.k = w.k;
  a.x = (const uint16_t *)x;
  a.residual = (const uint16_t *)residual;
  a.y = (uint16_t *)y;
  a.m = m;
  switch (w.format) {
    case QMM_AFFINE4_G64: return launch_wide<QMM_AFFINE4_G64>(a, s);
    case QMM_MXFP4: return launch_wide<QMM_MXFP4>(a, s);
    case QMM_NVFP4: return launch_wide<QMM_NVFP4>(a, s);
    default: return launch_wide<QMM_Q6_K>(a, s);
  }
}

}  // namespace qmm
