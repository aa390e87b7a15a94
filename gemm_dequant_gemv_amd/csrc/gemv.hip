// qgemv: decode matrix-vector product for 1-4 activation rows, weights
// dequantized in registers ("TurboEXL3" section 2.2, W4A16: each weight is
// expanded to 16 bits inside the kernel and multiplied at 16-bit precision with
// 32-bit accumulation; section 4.3: 1-4 rows take one GEMV launch whose output
// blocks are finished by the workgroup that arrives last).
//
// Mapping: a workgroup of 4 waves owns 32 R rows and a range of K steps of 256.
// In a wave, lane = 8*g + c: the 8 lanes c = 0..7 of a group read 8 x 16
// contiguous bytes of a row per step (whole 128-byte lines), and each lane
// carries R rows, so every activation value it loads from LDS feeds R rows x M
// lanes of multiply-adds.  D steps of codes are kept in flight per lane.
//
// Everything small is staged once per workgroup in LDS with a few wide loads,
// because scattered 2-16 byte loads per row and step cost as much memory-pipe
// time as the code stream itself:
//   * the workgroup's activations, already in the pair order the weight
//     unpacking produces, with per-block sums of x that fold the zero points
//     out of the per-weight work:
//       affine: sum (s q + b) x = s * sum q x + b * sum x, where the weight
//               operand is the bfloat16 128 + q (the nibble OR-ed into the
//               mantissa of 128) and the chain is seeded with -128 * sum x;
//       Q6_K:   sum (q - 32) x, operand 128 + q (q < 64 fits the 7 mantissa
//               bits), chain seeded with -160 * sum x over the 16-weight
//               sub-block.  This is the zero-point-in-the-seed form of splash
//               PR #19 ("128 + code", seed -160 x the sum of 16 inputs) carried
//               to bfloat16 operands;
//       E2M1:   hardware FP4 -> bfloat16 pair conversion, block scale applied
//               to the block's partial dot product;
//   * the block scales of the workgroup's rows and K range.
// The code stream uses buffer loads (scalar base, 32-bit offsets) with the
// non-temporal hint, issued unconditionally so that the compiler can count
// outstanding loads and wait only for the oldest step.
//
// Products are v_dot2_f32_bf16 (two bf16 products + fp32 accumulate).  The 8
// lanes of a row are reduced with cross-lane shuffles at the end; with K split
// over several workgroups each writes float32 partial sums and the last one to
// arrive adds them in split order, so results do not depend on timing.  The
// per-tile arrival counters live at the head of the caller's workspace and
// are cleared by a small kernel ahead of each split launch, so the workspace
// needs no particular contents on entry.
#include <algorithm>
#include <cstdlib>

#include "gemv_step.h"

namespace qmm {
namespace {

constexpr int kLK = 8;         // lanes sharing a row
constexpr int kGroups = 64 / kLK;

struct GemvArgs {
  const uint8_t *codes;
  const uint8_t *codes_hi;
  const uint8_t *scales;
  const uint8_t *scales2;
  const float *tensor_scale;
  const uint16_t *x;
  const uint16_t *residual;
  void *y;
  float *partials;     // [splits][M][tiles * rows per workgroup]
  uint32_t *counters;  // [tiles]
  uint32_t codes_bytes, hi_bytes, scales_bytes, scales2_bytes;
  int n, k, steps, splits, y_bf16;
};

// Row stride (in u32) of the staged scales: room for kMaxSplitK values and a
// pad that puts the 8 rows one ds_read touches on distinct banks.
template <int FMT, int R>
constexpr int scale_stride() {
  constexpr int words = kMaxSplitK / FmtTraits<FMT>::kKPerScaleByte / 4;
  int p = words + 1;
  while ((R * p) % 32 != 4 && p < words + 64) ++p;
  return p;
}

template <int FMT, int M, int R, int D, bool EARLY>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(GemvArgs a) {
  using T = FmtTraits<FMT>;
  constexpr int kNS = T::kSums;
  constexpr int ROWS = 4 * kGroups * R;      // rows per workgroup
  constexpr int XSTRIDE = 16 * M + 4;        // u32 per staged chunk; +16 B keeps the 8
                                             // chunks one instruction reads on distinct banks
  constexpr int SSTRIDE = scale_stride<FMT, R>();  // u32 per staged scale row
  constexpr int MAXCH = kMaxSplitK / 32;
  extern __shared__ __align__(16) uint32_t smem[];
  uint32_t *xs = smem;                                         // [MAXCH][XSTRIDE]
  float *xsum = (float *)(xs + MAXCH * XSTRIDE);               // [MAXCH][M][kNS]
  uint32_t *ssc = (uint32_t *)(xsum + MAXCH * M * (kNS > 0 ? kNS : 1));  // [ROWS][SSTRIDE]
  uint16_t *sd = (uint16_t *)(ssc + ROWS * SSTRIDE);           // Q6_K: [ROWS][MAXCH/8]

  const int tid = threadIdx.x;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int t0 = (int)((long)split * a.steps / a.splits);
  const int t1 = (int)((long)(split + 1) * a.steps / a.splits);
  const int kbase = t0 * kGemvStep;
  const int krange = min(a.k, t1 * kGemvStep) - kbase;
  const int row_wg = tile * ROWS;

  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane % kLK, g = lane / kLK;
  const int lrow0 = wave * (kGroups * R) + g * R;  // first row of this lane in the workgroup
  uint32_t offc[R], offh[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = (uint32_t)min(row_wg + lrow0 + r, a.n - 1);
    offc[r] = row * (uint32_t)(a.k / 2);
    offh[r] = row * (uint32_t)(a.k / 4);
  }
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes, a.codes_bytes);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.codes_hi, a.hi_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales, a.scales_bytes);
  const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(a.scales2, a.scales2_bytes);

  const UnpackK K = unpack_consts();
  float acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;

  // Every global load below is issued unconditionally (out-of-range steps and
  // lanes re-read a clamped, already-requested address), so the compiler can
  // count outstanding loads exactly and wait only for the oldest ones.
  //
  // 1. activations: at most kMaxSplitK values of x, a fixed number of 16-byte
  //    pieces per thread
  constexpr int XP = (MAXCH * M * 4 + kGemvThreads - 1) / kGemvThreads;
  const int valid_ch = krange / 32;
  const int items = valid_ch * M * 4;
  // (a load with no piece to fetch points past the end of the buffer and
  // returns zeros without a memory access: clamped copies of the last piece
  // from every workgroup of a split would queue on one L2 channel)
  const uint32_t x_bytes = (uint32_t)(M * a.k * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, x_bytes);
  uint4 xv[XP];
#pragma unroll
  for (int j = 0; j < XP; ++j) {
    const int i = j * kGemvThreads + tid;
    const int ch = i / (4 * M), m = (i >> 2) % M, part = i & 3;
    const uint32_t off =
        i < items ? ((uint32_t)m * a.k + kbase + ch * 32 + part * 8) * 2u : x_bytes;
    xv[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
  }

  // 2. block scales of the workgroup's rows and K range, as 32-bit words (the
  //    row stride of every scale plane is a multiple of 4 bytes)
  const uint32_t srow = (uint32_t)(a.k / T::kKPerScaleByte);       // bytes per row
  const uint32_t soff = (uint32_t)(kbase / T::kKPerScaleByte);
  const int sdpr = (krange / T::kKPerScaleByte + 3) / 4;            // words per row
  constexpr int SP = (ROWS * (kMaxSplitK / T::kKPerScaleByte / 4) + kGemvThreads - 1) / kGemvThreads;
  uint32_t sv[SP];
#pragma unroll
  for (int j = 0; j < SP; ++j) {
    const int i = min(j * kGemvThreads + tid, ROWS * sdpr - 1);
    const int rr = i / sdpr, w = i - rr * sdpr;
    const uint32_t row = (uint32_t)min(row_wg + rr, a.n - 1);
    sv[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, row * srow + soff + 4 * w, 0, 0);
  }
  // Q6_K super-block scales: 2 bytes per 256 values
  constexpr int DP = FMT == QMM_Q6_K ? (ROWS * (MAXCH / 8) + kGemvThreads - 1) / kGemvThreads : 0;
  const int dpr = krange / 256;
  uint32_t dv[DP > 0 ? DP : 1];
  if constexpr (FMT == QMM_Q6_K) {
#pragma unroll
    for (int j = 0; j < DP; ++j) {
      const int i = min(j * kGemvThreads + tid, ROWS * dpr - 1);
      const int rr = i / dpr, w = i - rr * dpr;
      const uint32_t row = (uint32_t)min(row_wg + rr, a.n - 1);
      dv[j] = __builtin_amdgcn_raw_buffer_load_b16(
          rs2, (row * (uint32_t)(a.k / 256) + (uint32_t)(kbase / 256) + w) * 2, 0, 0);
    }
  }

  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!EARLY) {
    // Wait for the small loads before the code stream starts.
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // 3. the codes of the first D steps; afterwards every consumed step is
  //    refilled with the step D ahead, keeping D steps in flight (when D covers
  //    a whole split there is nothing to refill)
  constexpr bool kRefill = D < kMaxSplitK / kGemvStep;
  const int tlast = t1 - 1;
  const int klast = a.k - 32;
  RowData buf[D][R];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const uint32_t kc = (uint32_t)min(min(t0 + d, tlast) * kGemvStep + c * 32, klast);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      buf[d][r].q = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, offc[r] + kc / 2, 0, 2));
      if constexpr (FMT == QMM_Q6_K)
        buf[d][r].h = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rh, offh[r] + kc / 4, 0, 2));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // 4. stage x (pair order + per-block sums) and the scales in LDS
#pragma unroll
  for (int j = 0; j < XP; ++j) {
    if (j * kGemvThreads >= items) break;  // uniform
    const int i = j * kGemvThreads + tid;
    const bool ok = i < items;
    const int ch = i / (4 * M), m = (i >> 2) % M, part = i & 3;
    const uint4 v = xv[j];
    if constexpr (kNS > 0) {
      float sm = ((bf_lo(v.x) + bf_hi(v.x)) + (bf_lo(v.y) + bf_hi(v.y))) +
                 ((bf_lo(v.z) + bf_hi(v.z)) + (bf_lo(v.w) + bf_hi(v.w)));
      sm += __shfl_xor(sm, 1);
      if constexpr (kNS == 1) {
        sm += __shfl_xor(sm, 2);
        if (ok && part == 0) xsum[ch * M + m] = sm;
      } else {
        if (ok && (part & 1) == 0) xsum[(ch * M + m) * 2 + (part >> 1)] = sm;
      }
    }
    if (ok) {
      uint4 o = v;
      if constexpr (T::kPermute) {
        o.x = (v.x & 0xFFFFu) | (v.z << 16);
        o.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
        o.z = (v.y & 0xFFFFu) | (v.w << 16);
        o.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
      }
      *(uint4 *)(xs + ch * XSTRIDE + m * 16 + part * 4) = o;
    }
  }
#pragma unroll
  for (int j = 0; j < SP; ++j) {
    const int i = j * kGemvThreads + tid;
    if (i < ROWS * sdpr) {
      const int rr = i / sdpr, w = i - rr * sdpr;
      ssc[rr * SSTRIDE + w] = sv[j];
    }
  }
  if constexpr (FMT == QMM_Q6_K) {
#pragma unroll
    for (int j = 0; j < DP; ++j) {
      const int i = j * kGemvThreads + tid;
      if (i < ROWS * dpr) {
        const int rr = i / dpr, w = i - rr * dpr;
        sd[rr * (MAXCH / 8) + w] = (uint16_t)dv[j];
      }
    }
  }
  __syncthreads();

  const uint8_t *ssb = (const uint8_t *)ssc;
  for (int tb = t0; tb < t1; tb += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int t = tb + d;
      const int kc = t * kGemvStep + c * 32;
      if (t < t1 && kc < a.k) {
        const int lc = (t - t0) * kLK + c;   // chunk index within the workgroup's range
        uint32_t X[M][16];
        float S[M][2];
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const uint4 *src = (const uint4 *)(xs + lc * XSTRIDE + m * 16);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 v = src[q];
            X[m][4 * q + 0] = v.x;
            X[m][4 * q + 1] = v.y;
            X[m][4 * q + 2] = v.z;
            X[m][4 * q + 3] = v.w;
          }
          S[m][0] = kNS > 0 ? xsum[(lc * M + m) * (kNS > 0 ? kNS : 1)] : 0.0f;
          S[m][1] = kNS > 1 ? xsum[(lc * M + m) * 2 + 1] : 0.0f;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int lr = lrow0 + r;
          RowData rd = buf[d][r];
          if constexpr (FMT == QMM_AFFINE4_G64) {
            rd.s = ssc[lr * SSTRIDE + lc / 2];
          } else if constexpr (FMT == QMM_MXFP4) {
            rd.s = ssb[(lr * SSTRIDE) * 4 + lc];
          } else {  // NVFP4 and Q6_K: two bytes per 32-value chunk
            rd.s = *(const uint16_t *)(ssb + (lr * SSTRIDE) * 4 + 2 * lc);
            if constexpr (FMT == QMM_Q6_K) rd.d = sd[lr * (MAXCH / 8) + lc / 8];
          }
          row_step<FMT, M>(rd, X, S, acc[r], K);
        }
      }
      if constexpr (kRefill) {
        const uint32_t kn = (uint32_t)min(min(t + D, tlast) * kGemvStep + c * 32, klast);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          buf[d][r].q = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, offc[r] + kn / 2, 0, 2));
          if constexpr (FMT == QMM_Q6_K)
            buf[d][r].h = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rh, offh[r] + kn / 4, 0, 2));
        }
      }
    }
  }

  // ---- reduce the 8 lanes of each row
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = acc[r][m];
#pragma unroll
      for (int o = 1; o < kLK; o <<= 1) v += __shfl_xor(v, o);
      acc[r][m] = v;
    }

  const float gscale = (FMT == QMM_NVFP4 && a.tensor_scale) ? a.tensor_scale[0] : 1.0f;
  const int npad = gridDim.x * ROWS;

  // each of the 8 lanes of a group stores some of its rows x M results
#pragma unroll
  for (int i = 0; i < R * M; ++i) {
    if ((i % kLK) != c) continue;
    const int r = i / M, m = i % M;
    const int row = row_wg + lrow0 + r;
    if (row >= a.n) continue;
    if (a.splits == 1) {
      float v = acc[r][m] * gscale;
      if (a.residual) v += bf_lo(a.residual[(size_t)m * a.n + row]);
      if (a.y_bf16)
        ((uint16_t *)a.y)[(size_t)m * a.n + row] = (uint16_t)float_to_bf16(v);
      else
        ((float *)a.y)[(size_t)m * a.n + row] = v;
    } else {
      // agent-scope store: written through to the point where every XCD sees it
      __hip_atomic_store(&a.partials[((size_t)split * M + m) * npad + row], acc[r][m],
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (a.splits == 1) return;

  // ---- split-K finish by the last workgroup of this row tile.  The partial
  // sums travel only through agent-scope atomic stores and loads (coherent
  // across XCDs without flushing or invalidating the L2s); every wave waits
  // for its stores to complete before the barrier that precedes the counter
  // increment, so a workgroup that sees the count reach splits-1 also sees
  // every split's partials.
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(a.splits - 1);
  __syncthreads();
  if (!s_last) return;
  for (int i = tid; i < ROWS * M; i += kGemvThreads) {
    const int m = i / ROWS;
    const int row = row_wg + (i % ROWS);
    if (row >= a.n) continue;
    float v = 0.0f;
    for (int sp = 0; sp < a.splits; ++sp)
      v += __hip_atomic_load(&a.partials[((size_t)sp * M + m) * npad + row], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    v *= gscale;
    if (a.residual) v += bf_lo(a.residual[(size_t)m * a.n + row]);
    if (a.y_bf16)
      ((uint16_t *)a.y)[(size_t)m * a.n + row] = (uint16_t)float_to_bf16(v);
    else
      ((float *)a.y)[(size_t)m * a.n + row] = v;
  }
}

template <int FMT, int M, int R>
constexpr size_t lds_bytes_cfg() {
  constexpr int kNS = FmtTraits<FMT>::kSums;
  constexpr int MAXCH = kMaxSplitK / 32;
  constexpr int ROWS = 4 * kGroups * R;
  return (size_t)MAXCH * (16 * M + 4) * 4 + (size_t)MAXCH * M * (kNS > 0 ? kNS : 1) * 4 +
         (size_t)ROWS * scale_stride<FMT, R>() * 4 +
         (FMT == QMM_Q6_K ? (size_t)ROWS * (MAXCH / 8) * 2 : 0);
}

template <int FMT, int M, int R, int D, bool EARLY>
hipError_t launch_cfg(const GemvArgs &a, const GemvPlan &p, hipStream_t s) {
  constexpr size_t lds = lds_bytes_cfg<FMT, M, R>();
  static_assert(lds <= 65536, "GEMV LDS budget");
  hipLaunchKernelGGL((gemv_kernel<FMT, M, R, D, EARLY>), dim3(p.tiles, p.splits), dim3(kGemvThreads),
                     lds, s, a);
  return hipGetLastError();
}

// (rows per lane, steps in flight) configurations compiled in
#ifdef QMM_TUNE
#define QMM_GEMV_CONFIGS(X) X(1, 2, 0) X(1, 2, 1) X(1, 4, 1) X(1, 8, 1) X(1, 4, 0) X(2, 4, 1) X(2, 2, 1)
#else
#define QMM_GEMV_CONFIGS(X) X(1, 2, 0)
#endif

template <int FMT, int M>
hipError_t launch_fm(const GemvArgs &a, const GemvPlan &p, hipStream_t s) {
#define QMM_CASE(RR, DD, EE) \
  if (p.rows_per_lane == RR && p.depth == DD && p.early == EE) \
    return launch_cfg<FMT, M, RR, DD, EE>(a, p, s);
  QMM_GEMV_CONFIGS(QMM_CASE)
#undef QMM_CASE
  return hipErrorInvalidConfiguration;
}

template <int FMT>
hipError_t launch_f(const GemvArgs &a, int m, const GemvPlan &p, hipStream_t s) {
  switch (m) {
    case 1: return launch_fm<FMT, 1>(a, p, s);
    case 2: return launch_fm<FMT, 2>(a, p, s);
    case 3: return launch_fm<FMT, 3>(a, p, s);
    default: return launch_fm<FMT, 4>(a, p, s);
  }
}

}  // namespace

GemvPlan plan_gemv(int format, int n, int k, int m) {
  GemvPlan p{};
  // the row-streaming kernel whenever the activations fit in LDS
  bool streaming = true;
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_GEMV_KIND")) streaming = atoi(e) == 1;
#endif
  if (streaming && plan_gemv_rows(format, n, k, m, p)) return p;
  p = GemvPlan{};
  // One row per lane and two steps in flight: measured best on MI355X for the
  // decode shapes.  Deeper prefetch oversubscribes the memory system, and the
  // activation and scale loads of workgroups that start later then queue behind
  // the whole machine's code requests.
  p.rows_per_lane = 1;
  p.depth = 2;
  p.lanes_k = kLK;
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_GEMV_R")) p.rows_per_lane = atoi(e);
  if (const char *e = getenv("QMM_GEMV_D")) p.depth = atoi(e);
  if (const char *e = getenv("QMM_GEMV_EARLY")) p.early = atoi(e);
#endif
  const int rows = 4 * kGroups * p.rows_per_lane;
  p.steps = (k + kGemvStep - 1) / kGemvStep;
  p.tiles = (n + rows - 1) / rows;
  const int max_steps = kMaxSplitK / kGemvStep;
  const int s_min = (p.steps + max_steps - 1) / max_steps;  // staging bound
  int s_par = (512 + p.tiles - 1) / p.tiles;                 // aim for >= 512 workgroups
  s_par = std::min(s_par, std::max(1, p.steps / 2));         // keep >= 2 steps per split
  int S = std::max(1, std::max(s_min, s_par));
  // prefer an even division of the steps when one is close
  for (int c = S; c <= S + S / 2 && c <= p.steps; ++c)
    if (p.steps % c == 0) { S = c; break; }
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_GEMV_SPLITS")) S = std::max(s_min, atoi(e));
#endif
  S = std::min(S, p.steps);
  p.splits = S;
  p.max_steps = (p.steps + S - 1) / S;
  if (S > 1) {
    p.counters_bytes = ((size_t)p.tiles * 4 + 255) / 256 * 256;
    p.ws_bytes = p.counters_bytes + (size_t)S * m * p.tiles * rows * 4;
  }
  return p;
}

hipError_t launch_gemv(const qmm_weight &w, const void *x, int m, const void *residual,
                       void *y, int y_dtype, void *workspace, const GemvPlan &p,
                       hipStream_t s) {
  if (p.kind == 1) return launch_gemv_rows(w, x, m, residual, y, y_dtype, p, s);
  GemvArgs a;
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
  a.x = (const uint16_t *)x;
  a.residual = (const uint16_t *)residual;
  a.y = y;
  a.counters = (uint32_t *)workspace;
  a.partials = workspace ? (float *)((char *)workspace + p.counters_bytes) : nullptr;
  if (p.splits > 1) {
    // the workspace may hold anything: the tile counters start from zero,
    // cleared by a kernel ahead of the split launch on the same stream
    const hipError_t e = launch_zero(workspace, p.counters_bytes, s);
    if (e != hipSuccess) return e;
  }
  a.n = w.n;
  a.k = w.k;
  a.steps = p.steps;
  a.splits = p.splits;
  a.y_bf16 = y_dtype == QMM_BF16;
  switch (w.format) {
    case QMM_AFFINE4_G64: return launch_f<QMM_AFFINE4_G64>(a, m, p, s);
    case QMM_MXFP4: return launch_f<QMM_MXFP4>(a, m, p, s);
    case QMM_NVFP4: return launch_f<QMM_NVFP4>(a, m, p, s);
    default: return launch_f<QMM_Q6_K>(a, m, p, s);
  }
}

}  // namespace qmm
