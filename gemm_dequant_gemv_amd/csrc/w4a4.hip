// W4A4: both operands of the multiply in MXFP4 ("TurboEXL3" section 2.2, the
// W4A4 bullet: the activations are quantized to a 4-bit block format on the
// fly, so both operands are FP4; section 2.1: MXFP4 is E2M1 values with one
// E8M0 power-of-two scale per 32).  gfx950's block-scaled matrix cores take
// exactly this pair: v_mfma_scale_f32_32x32x64_f8f6f4 multiplies E2M1 codes
// of both operands, each lane's 32 values scaled by its own E8M0 byte.
//
//   quant_mxfp4_kernel: x bf16 [m][k] -> codes u8 [m][k/2] and E8M0 u8
//     [m][k/32].  One thread per block of 32: amax, the shared exponent
//     E = floor(log2 amax) - 2 (E8M0 = max(E + 127, 0); an all-zero block
//     gets 0 and zero codes), then every value times 2^-E compared with the
//     E2M1 decision points (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; a value on a
//     point goes to the neighbour with the even index; past 6 saturates),
//     sign in bit 3, a value that rounds to zero coded 0.
//   gemm_w4a4_kernel: the product of the MXFP4 weights and the quantized
//     activations, float32 sums, bf16 y (+ residual).  A workgroup of 8 waves
//     owns 256 weight rows x 32 TM activation rows; per 256-wide K slice the
//     activation codes and scales go from memory straight into LDS (three
//     slices in flight) and each wave loads its own 32 weight rows' codes and
//     scales into registers (three slices ahead, through the caches: the 32
//     activation tiles of a weight tile read it again, and the non-temporal
//     loads of the streaming GEMV measured 28-39% slower here).  The codes are
//     the MFMA operands as they are: there is no decode step.  Inside a slice,
//     lane half h multiplies K blocks 4h .. 4h + 3 (k-steps 0 .. 3) for both
//     operands, so a lane reads 64 contiguous code bytes of its weight row.
//     (128-wide slices, one barrier per two k-steps instead of four, were
//     7-12% slower.)
//   The products of E2M1 values and powers of two are exact; only the float32
//   sums round, in a fixed order (slices in order, k-steps in order, the two
//   lane halves inside the matrix core).
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <type_traits>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float f32x16_w __attribute__((ext_vector_type(16)));

constexpr int kW4Stages = 3;         // slices in flight (128-wide: 4 and 6 measured 2-6% slower)
constexpr int kW4Waves = 8;
constexpr int kW4BN = 32 * kW4Waves; // weight rows per workgroup

// ---------------------------------------------------------------- quantizer

__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const uint16_t *__restrict__ x,
                                                          uint8_t *__restrict__ codes,
                                                          uint8_t *__restrict__ scales,
                                                          uint32_t blocks) {
  const uint32_t b = blockIdx.x * 256u + threadIdx.x;
  if (b >= blocks) return;
  const uint4 *src = (const uint4 *)(x + (size_t)b * 32);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = src[i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  // largest magnitude, as bfloat16 bits (finite values order as integers)
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  uint32_t e8 = 0;
  int sh = 0;  // the values are multiplied by 2^sh = 2^(127 - E8M0)
  if (amax != 0) {
    const int ex = (int)(amax >> 7);
    // floor(log2 amax): the exponent field, or for a subnormal mantissa m
    // (value m * 2^-133) the position of its top bit
    const int fl = ex > 0 ? ex - 127 : (31 - __builtin_clz(amax & 0x7Fu)) - 133;
    const int e8i = max(fl - 2 + 127, 0);
    e8 = (uint32_t)e8i;
    sh = 127 - e8i;
  }
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t hbits = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    const float a = __builtin_ldexpf(__uint_as_float((hbits & 0x7FFFu) << 16), sh);
    const uint32_t idx = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                         (uint32_t)(a > 5.0f);
    const uint32_t code = idx ? (idx | ((hbits >> 12) & 8u)) : 0u;
    out[j >> 3] |= code << (4 * (j & 7));
  }
  *(uint4 *)(codes + (size_t)b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  scales[b] = (uint8_t)e8;
}

// ---------------------------------------------------------------- GEMM

struct W4A4Args {
  const uint8_t *wcodes, *wscales;  // MXFP4 weight [n][k/2], [n][k/32]
  const uint8_t *xcodes, *xscales;  // quantized activations [m][k/2], [m][k/32]
  const uint16_t *residual;         // bf16 [m][n] or null
  uint16_t *y;                      // bf16 [m][n]
  int m, n, k;
  int n_begin;                      // first weight row of the launch's tiles
};

// Slices of KS k-steps of 64 values (KS = 4 where K is a multiple of 256,
// else 2): per row KS * 32 code bytes in 2 KS chunks of 16, and KS / 2 words
// of four E8M0 scales.
template <int KS>
struct W4Slice {
  static constexpr int kK = 64 * KS;          // K values per slice
  static constexpr int kRowBytes = 32 * KS;   // code bytes of one row per slice
  static constexpr int kChunks = 2 * KS;      // 16-byte chunks of one row
  static constexpr int kScaleWords = KS / 2;  // E8M0 words of one row per slice
  // Physical 16-byte chunk of logical chunk c of activation row r in a
  // slice's LDS image: the 16 rows one ds_read_b128 lane group reads at one
  // logical chunk land on 16 distinct bank groups (16 / kChunks rows share
  // a 256-byte bank row; the row's next bits pick the XOR).
  static __device__ __forceinline__ int xchunk(int r, int c) {
    return c ^ ((r / (16 / kChunks)) & (kChunks - 1));
  }
};

// The workgroup's 8 waves as kWN x kWM: wave w owns weight rows
// 32 TN (w % kWN) .. (TN groups of 32) and activation rows 32 TM (w / kWN) ..
// (TM groups of 32) of the 256 x 256 tile, so every activation operand read
// from LDS feeds TN products and every weight operand TM.
template <int TN, int TM, int KS>
__global__ __launch_bounds__(64 * kW4Waves) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_w4a4_kernel(W4A4Args a) {
  using SL = W4Slice<KS>;
  constexpr int kSliceK = SL::kK, kRowBytes = SL::kRowBytes, kKSteps = KS;
  constexpr int kScaleWords = SL::kScaleWords;
  constexpr int kWN = kW4BN / (32 * TN);       // wave columns over the weight rows
  constexpr int kWM = kW4Waves / kWN;          // wave rows over the activation rows
  constexpr int BM = 32 * TM * kWM;
  static_assert(kWN * 32 * TN == kW4BN && kWN * kWM == kW4Waves, "wave grid");
  constexpr int kCodeStage = BM * kRowBytes;  // activation codes of one slice
  constexpr int kStage = kCodeStage + BM * 4 * kScaleWords; // + their scales
  constexpr int XI = BM * kRowBytes / 1024 / kW4Waves;  // code-load instructions per wave and slice
  constexpr int SI = BM * kScaleWords / 64;             // scale-load instructions per slice
  static_assert(XI >= 1 && XI * 1024 * kW4Waves == BM * kRowBytes && SI >= 1 && SI <= kW4Waves, "tiles");
  constexpr int kLoads = XI + 1 + (kKSteps + 1) * TN;  // X codes, X scales, W codes + scales
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % kWN, wm = wave / kWN;
  const int lr = lane & 31, h = lane >> 5;
  const int tiles_m = (a.m + BM - 1) / BM;
  const int m0 = ((int)blockIdx.x % tiles_m) * BM;
  const int n0 = a.n_begin + ((int)blockIdx.x / tiles_m) * kW4BN;
  const int mrows = a.m - m0;
  const int slices = a.k / kSliceK;
  const uint32_t kb = (uint32_t)a.k / 2, kq = (uint32_t)a.k / 32;

  // activation codes: lane L of this wave's instruction i writes LDS piece
  // P = (wave + 8 i) 64 + L of the stage, i.e. row P / 2KS, physical chunk
  // P % 2KS, which holds the row's logical chunk xchunk(row, P % 2KS)
  const __amdgpu_buffer_rsrc_t rxc = make_rsrc(a.xcodes, (uint32_t)((size_t)a.m * kb));
  const __amdgpu_buffer_rsrc_t rxs = make_rsrc(a.xscales, (uint32_t)((size_t)a.m * kq));
  uint32_t v_x[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int P = (wave + kW4Waves * i) * 64 + lane;
    const int r = P / SL::kChunks;
    v_x[i] = (uint32_t)(m0 + min(r, mrows - 1)) * kb + (uint32_t)SL::xchunk(r, P % SL::kChunks) * 16u;
  }
  // activation scales: instruction wave % SI covers rows 64 (wave % SI) ..;
  // waves past SI repeat one (the same bytes to the same place)
  const int si = wave % SI;
  const int srow = (si * 64 + lane) / kScaleWords, sword = (si * 64 + lane) % kScaleWords;
  const uint32_t v_xs = (uint32_t)(m0 + min(srow, mrows - 1)) * kq + (uint32_t)sword * 4u;
  auto load_x = [&](int s) __attribute__((always_inline)) {
    uint8_t *st = lds + (s % kW4Stages) * kStage;
#pragma unroll
    for (int i = 0; i < XI; ++i)
      buffer_load_lds16(rxc, st + (wave + kW4Waves * i) * 1024, v_x[i], (uint32_t)s * kRowBytes);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rxs, (lds_void_t *)(st + kCodeStage + si * 256), 4,
                                             v_xs, (uint32_t)s * (kSliceK / 32), 0, 0);
  };

  // weights: lane (lr, h) holds weight rows n0 + 32 (TN wn + tn) + lr; per
  // slice their code bytes 16 KS h .. (K blocks KS h .. KS h + KS - 1) and the
  // row's 2 KS scales of the slice
  const __amdgpu_buffer_rsrc_t rwc = make_rsrc(a.wcodes, (uint32_t)((size_t)a.n * kb));
  const __amdgpu_buffer_rsrc_t rws = make_rsrc(a.wscales, (uint32_t)((size_t)a.n * kq));
  uint32_t v_wc[TN], v_ws[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const uint32_t wrow = (uint32_t)min(n0 + 32 * (TN * wn + tn) + lr, a.n - 1);
    v_wc[tn] = wrow * kb + 16u * KS * (uint32_t)h;
    v_ws[tn] = wrow * kq;
  }
  struct WPiece {
    u32x4_t q[kKSteps][TN];       // K blocks KS h + ks
    uint32_t s[TN][kScaleWords];  // each row's 2 KS E8M0 scales of the slice
  };
  auto load_w = [&](int s) __attribute__((always_inline)) {
    WPiece p;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        p.q[ks][tn] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
            rwc, v_wc[tn], (uint32_t)s * kRowBytes + 16u * ks, 0));
      if constexpr (kScaleWords == 2) {
        const uint2 w2 = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
            rws, v_ws[tn], (uint32_t)s * (kSliceK / 32), 0));
        p.s[tn][0] = w2.x;
        p.s[tn][kScaleWords - 1] = w2.y;
      } else {
        p.s[tn][0] = __builtin_amdgcn_raw_buffer_load_b32(rws, v_ws[tn], (uint32_t)s * (kSliceK / 32), 0);
      }
    }
    return p;
  };
  WPiece wr[kW4Stages];

  f32x16_w acc[TN][TM];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[tn][t][e] = 0.f;

  // this lane's activation operand reads: row 32 (TM wm + t) + lr, logical
  // chunk KS h + ks at its physical place (the XOR takes row bits below 32,
  // so it is that of lr)
  uint32_t xo[kKSteps];
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks)
    xo[ks] = (uint32_t)(32 * TM * wm + lr) * kRowBytes + (uint32_t)SL::xchunk(lr, KS * h + ks) * 16u;
  // the lane's scale bytes KS h .. KS h + KS - 1 of the row: word (KS h) / 4
  // from byte (KS h) % 4 on
  const uint32_t xso = (uint32_t)kCodeStage + (uint32_t)(32 * TM * wm + lr) * 4u * kScaleWords +
                       (uint32_t)(KS * h / 4) * 4u;
  const int sbyte0 = (KS * h) % 4;

  // The waits below count loads, so the loads must issue slice by slice (the
  // scheduler is kept from regrouping the first slices' loads).
#pragma unroll
  for (int p = 0; p < kW4Stages - 1; ++p) {
    const int sp = min(p, slices - 1);
    load_x(sp);
    wr[p] = load_w(sp);
    __builtin_amdgcn_sched_barrier(0);
  }

  // One slice: s is the slice, u its weight slot s % kW4Stages.
  auto slice = [&](const int s, auto uc) __attribute__((always_inline)) {
    constexpr int u = decltype(uc)::value;
    // slice s is in LDS (this wave's share) once at most the loads of the
    // kW4Stages - 2 slices issued after it are outstanding; the barrier
    // makes every wave's share visible and frees the stage of slice s - 1
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kW4Stages - 2) * kLoads));
    __builtin_amdgcn_s_barrier();
    const int sn = min(s + kW4Stages - 1, slices - 1);
    load_x(sn);
    wr[(u + kW4Stages - 1) % kW4Stages] = load_w(sn);

    const uint8_t *stg = lds + (s % kW4Stages) * kStage;
    const WPiece &wp = wr[u];
    // k-step 0's activation operands and the scale words first; k-step
    // ks + 1's operands are read from LDS during k-step ks's MFMAs (one read
    // after each of the last TM MFMAs, the order pinned)
    u32x4_t bk[2][TM];
    uint32_t xsc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const uint8_t *row = stg + t * 32 * kRowBytes;
      bk[0][t] = *(const u32x4_t *)(row + xo[0]);
      xsc[t] = *(const uint32_t *)(stg + xso + t * 32 * 4 * kScaleWords);
    }
    uint32_t wsc[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) wsc[tn] = h ? wp.s[tn][kScaleWords - 1] : wp.s[tn][0];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const u32x4_t q = wp.q[ks][tn];
        const v8i_t av = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
        const int sa = (int)((wsc[tn] >> (8 * (sbyte0 + ks))) & 0xFFu);
#pragma unroll
        for (int t = 0; t < TM; ++t) {
          const u32x4_t b = bk[ks & 1][t];
          const v8i_t bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
          acc[tn][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              av, bv, acc[tn][t], 4, 4, 0, sa, 0, (int)((xsc[t] >> (8 * (sbyte0 + ks))) & 0xFFu));
          if (tn == TN - 1 && ks + 1 < kKSteps)
            bk[(ks + 1) & 1][t] = *(const u32x4_t *)(stg + t * 32 * kRowBytes + xo[ks + 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  // Whole groups of kW4Stages slices, then the rest: the loop body has no exit
  // of its own, so that the compiler's wait analysis keeps track of the
  // weight loads' age across the back edge (with an exit per slice it waited
  // for the loads issued one slice earlier).
  static_assert(kW4Stages == 3, "the slice loop is written out for three stages");
  int s = 0;
  for (; s + kW4Stages <= slices; s += kW4Stages) {
    slice(s, std::integral_constant<int, 0>{});
    slice(s + 1, std::integral_constant<int, 1>{});
    slice(s + 2, std::integral_constant<int, 2>{});
  }
  if (s < slices) slice(s, std::integral_constant<int, 0>{});
  if (s + 1 < slices) slice(s + 1, std::integral_constant<int, 1>{});
  // the re-reads issued past the last slice: no LDS write may be pending when
  // the workgroup ends
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // epilogue: lane (lr, h) holds D[n = 8b + 4h + r][m = lr] of each tile as
  // value 4b + r: four consecutive weight rows per b
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    const int ml = 32 * (TM * wm + t) + lr;
    if (ml >= mrows) continue;
    const int m = m0 + ml;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int nb = n0 + 32 * (TN * wn + tn) + 8 * b + 4 * h;
        float v[4] = {acc[tn][t][4 * b], acc[tn][t][4 * b + 1], acc[tn][t][4 * b + 2],
                      acc[tn][t][4 * b + 3]};
        const size_t base = (size_t)m * a.n + nb;
        if (nb + 3 < a.n && (a.n & 3) == 0) {  // 8-byte aligned: 4 bf16 at once
          if (a.residual) {
            const uint2 r = *(const uint2 *)(a.residual + base);
            v[0] += bf_lo(r.x);
            v[1] += bf_hi(r.x);
            v[2] += bf_lo(r.y);
            v[3] += bf_hi(r.y);
          }
          *(uint2 *)(a.y + base) = make_uint2(float_to_bf16(v[0]) | (float_to_bf16(v[1]) << 16),
                                              float_to_bf16(v[2]) | (float_to_bf16(v[3]) << 16));
          continue;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (nb + r >= a.n) break;
          float o = v[r];
          if (a.residual) o += bf_lo(a.residual[base + r]);
          a.y[base + r] = (uint16_t)float_to_bf16(o);
        }
      }
    }
  }
}

constexpr size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t w4a4_workspace_size(int m, int k) {
  return align256((size_t)m * (size_t)(k / 2)) + align256((size_t)m * (size_t)(k / 32));
}

bool w4a4_fits(const qmm_weight &w, int m) {
  // 32-bit buffer offsets for both operands' planes
  return (size_t)m * (size_t)(w.k / 2) < (1ull << 32) && (size_t)w.n * (size_t)(w.k / 2) < (1ull << 32);
}

hipError_t launch_quant_mxfp4(const void *x, int m, int k, void *codes, void *scales,
                              hipStream_t s) {
  const uint32_t blocks = (uint32_t)((size_t)m * (size_t)(k / 32));
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_mxfp4_kernel, dim3((blocks + 255) / 256), dim3(256), 0, s,
                     (const uint16_t *)x, (uint8_t *)codes, (uint8_t *)scales, blocks);
  return hipGetLastError();
}

namespace {

// Dynamic LDS above the default 64 KB: raised once per device and kernel.
template <int TN, int TM, int KS>
hipError_t allow_w4_lds(size_t lds) {
  if (lds <= 65536) return hipSuccess;
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (raised.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute((const void *)gemm_w4a4_kernel<TN, TM, KS>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) raised.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// The GEMM launches: tiles_m x tn_a tiles of 256 x 256, then (tn_a <
// tiles_n) the remaining weight rows as tiles of 128 activation rows, or of
// 64 with 256-wide slices where those still fit one round of workgroups.
template <int KS>
hipError_t launch_w4_tiles(W4A4Args a, int m, long tiles_m, long tn_a, long tiles_n, hipStream_t s) {
  using SL = W4Slice<KS>;
  constexpr int BM = 256;
  constexpr size_t lds = (size_t)kW4Stages * (BM * SL::kRowBytes + BM * 4 * SL::kScaleWords);
  hipError_t e = allow_w4_lds<1, 8, KS>(lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_w4a4_kernel<1, 8, KS>), dim3((unsigned)(tiles_m * tn_a)), dim3(64 * kW4Waves),
                     lds, s, a);
  if (tn_a == tiles_n) return hipGetLastError();
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  a.n_begin = (int)(tn_a * kW4BN);
  auto tail = [&](auto tm_c) {
    constexpr int TM = decltype(tm_c)::value, BMT = 32 * TM;
    constexpr size_t lds_t = (size_t)kW4Stages * (BMT * SL::kRowBytes + BMT * 4 * SL::kScaleWords);
    hipError_t e2 = allow_w4_lds<1, TM, KS>(lds_t);
    if (e2 != hipSuccess) return e2;
    const unsigned grid_t = (unsigned)(((m + BMT - 1) / BMT) * (tiles_n - tn_a));
    hipLaunchKernelGGL((gemm_w4a4_kernel<1, TM, KS>), dim3(grid_t), dim3(64 * kW4Waves), lds_t, s, a);
    return hipGetLastError();
  };
  if constexpr (KS == 4) {
    bool half = (m + 63) / 64 * (tiles_n - tn_a) <= compute_units();
#ifdef QMM_TUNE
    if (const char *v = getenv("QMM_W4_TAIL_TM")) half = atoi(v) == 2;
#endif
    if (half) return tail(std::integral_constant<int, 2>());
  }
  return tail(std::integral_constant<int, 4>());
}

}  // namespace

hipError_t launch_gemm_w4a4(const qmm_weight &w, const void *x, int m, const void *residual,
                            void *y, void *workspace, hipStream_t s) {
  uint8_t *xc = (uint8_t *)workspace;
  uint8_t *xs = xc + align256((size_t)m * (size_t)(w.k / 2));
  hipError_t e = launch_quant_mxfp4(x, m, w.k, xc, xs, s);
  if (e != hipSuccess) return e;
  W4A4Args a;
  a.wcodes = (const uint8_t *)w.codes;
  a.wscales = (const uint8_t *)w.scales;
  a.xcodes = xc;
  a.xscales = xs;
  a.residual = (const uint16_t *)residual;
  a.y = (uint16_t *)y;
  a.m = m;
  a.n = w.n;
  a.k = w.k;
  // one weight-row group per wave: 2 and 4 groups (activation operands
  // shared by 2 or 4 products, but every weight row loaded by 2 or 4 waves)
  // measured 17-24% and 46-50% slower on 17408 x 5120 at M = 512-8192
  constexpr int BM = 256;
  a.n_begin = 0;
  // The last round of one-per-CU workgroups: after at least one whole round,
  // a last round of at most a quarter of the compute units runs as a second
  // launch over the remaining weight rows with 128 activation rows per tile
  // (twice as many workgroups, each half the work)
  const long tiles_m = (m + BM - 1) / BM, tiles_n = (w.n + kW4BN - 1) / kW4BN;
  const long cus = compute_units(), full = tiles_m * tiles_n / cus;
  const long frac = tiles_m * tiles_n - full * cus;
  long tn_a = tiles_n;
  if (full >= 1 && frac > 0 && 4 * frac <= cus) {
    const long ta = full * cus / tiles_m;  // weight-row blocks that fill whole rounds
    if (ta >= 1 && ta < tiles_n) tn_a = ta;
  }
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_W4_TAIL"); e && !atoi(e)) tn_a = tiles_n;
#endif
  // 256-wide K slices where K allows (a multiple of 256), else 128-wide
  return w.k % 256 == 0 ? launch_w4_tiles<4>(a, m, tiles_m, tn_a, tiles_n, s)
                        : launch_w4_tiles<2>(a, m, tiles_m, tn_a, tiles_n, s);
}

}  // namespace qmm
