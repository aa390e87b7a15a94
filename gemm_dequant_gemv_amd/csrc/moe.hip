// qmoe_grouped: one mixture-of-experts layer (routed experts plus optional
// shared experts).  Up to 16 tokens with at most 128 token slots take the
// decode form (two grouped GEMV launches over the token slots, moe_gemv.hip,
// the second also running the combine); more tokens take the grouped-GEMM form
// ("TurboEXL3" section 4.1):
//   1. route:    count each expert's tokens, group the token slots by expert
//                and build the table of row tiles, instead of sorting first
//                and tabulating afterwards: one launch for calls with few
//                slots, three (per-workgroup counts, one scan, placement)
//                for calls with many;
//   2. gate/up:  one grouped GEMM over the tile table, activations gathered by
//                token, weights decoded once per K-slice per workgroup; SwiGLU
//                in float32 in its epilogue -> bf16 h;
//   3. down:     one grouped GEMM over the same tiles -> float32 d per slot;
//   4. combine:  the score-weighted sum of each token's expert outputs, in a
//                fixed order (routed slots in list order, then shared experts).
// Grouped rows are the token slots sorted by expert; the order of slots inside
// one expert's group comes from LDS atomics and is not fixed, but every row is
// computed independently of its neighbours and the combine reads rows by slot,
// so the layer's output is the same on every run.
#include <algorithm>
#include <cstdlib>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace {

constexpr uint32_t kInvalidRow = 0xFFFFFFFFu;
constexpr int kRouteThreads = 1024;
constexpr int kRun = 16;  // slots per thread and pass in the route kernel

struct RouteArgs {
  const int32_t *topk_ids;
  int t, topk, num_routed, num_shared;
  int tile_rows;  // rows per routing tile
  MoeTables tb;
};

// Block-wide exclusive scan of one value per thread (1024 threads); returns the
// prefix and writes the total to *total.  Each wave scans its 64 values in
// registers (six shuffle steps), then every thread adds the totals of the
// waves before its own from LDS: two barriers in all.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *buf, uint32_t *total) {
  constexpr int kWaves = kRouteThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) buf[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t s = buf[w];
    before += w < wave ? s : 0u;
    all += s;
  }
  if (tid == 0) *total = all;
  __syncthreads();
  return before + incl - v;
}

// Steps 2 to 4 of the route, given each expert's row count in s_count:
// group offsets (exclusive scan over experts), the shared experts' rows (every
// token, in token order), the experts with rows and their tiles of tile_rows
// rows.  s_off receives the offsets.
__device__ void group_and_tile(const RouteArgs &a, uint32_t *s_count, uint32_t *s_off,
                               uint32_t *s_scan, uint32_t *s_total) {
  const int tid = threadIdx.x;
  const int ne = a.num_routed + a.num_shared;
  const MoeTables &tb = a.tb;
  // 2. group offsets (exclusive scan over experts, kMoeMaxExperts / 1024 per thread)
  constexpr int PER = kMoeMaxExperts / kRouteThreads;
  uint32_t local = 0;
  for (int j = 0; j < PER; ++j) {
    const int e = tid * PER + j;
    local += e < ne ? s_count[e] : 0u;
  }
  uint32_t base = block_exclusive_scan(local, s_scan, s_total);
  for (int j = 0; j < PER; ++j) {
    const int e = tid * PER + j;
    if (e < ne) {
      s_off[e] = base;
      tb.counts[e] = s_count[e];
      tb.offsets[e] = base;
      base += s_count[e];
    }
  }
  if (tid == 0) tb.offsets[ne] = *s_total;
  __syncthreads();

  // 3. (shared experts) every token, in token order
  for (int s = 0; s < a.num_shared; ++s)
    for (int t = tid; t < a.t; t += kRouteThreads) {
      const uint32_t row = s_off[a.num_routed + s] + t;
      tb.row_of_shared[(size_t)s * a.t + t] = row;
      tb.token_of_row[row] = (uint32_t)t;
      tb.slot_of_row[row] = (uint32_t)a.t * (uint32_t)a.topk + (uint32_t)(s * a.t + t);
    }

  // 4. experts with rows (in expert order) and their tiles of tile_rows rows
  uint32_t nact = 0, ntile = 0;
  for (int j = 0; j < PER; ++j) {
    const int e = tid * PER + j;
    if (e < ne && s_count[e]) {
      nact += 1;
      ntile += (s_count[e] + a.tile_rows - 1) / a.tile_rows;
    }
  }
  uint32_t act_base = block_exclusive_scan(nact, s_scan, s_total);
  if (tid == 0) *tb.n_active = *s_total;
  uint32_t tile_base = block_exclusive_scan(ntile, s_scan, s_total);
  if (tid == 0) *tb.n_tiles = *s_total;
  for (int j = 0; j < PER; ++j) {
    const int e = tid * PER + j;
    if (e >= ne || !s_count[e]) continue;
    tb.active[act_base++] = (uint32_t)e;
    const uint32_t cnt = s_count[e];
    for (uint32_t r = 0; r < cnt; r += a.tile_rows) {
      uint32_t *tl = tb.tiles + 3 * (size_t)tile_base++;
      tl[0] = (uint32_t)e;
      tl[1] = s_off[e] + r;
      tl[2] = min(cnt - r, (uint32_t)a.tile_rows);
    }
  }
}

// Positions of the routed slots [i0, i1) inside their experts' groups, by
// LDS atomics on s_count (the order inside a group is not fixed); a dropped
// id gets kInvalidRow and sets *bad.  A pass covers kRun x 1024 slots (slot
// b + 1024 j for thread j-th of the pass: consecutive threads, consecutive
// slots); a thread loads all its ids of the pass before its atomics, so that
// it waits on memory once per pass rather than once per slot.
__device__ void count_slots(const RouteArgs &a, int i0, int i1, uint32_t *s_count, int *bad) {
  const int tid = threadIdx.x;
  constexpr int kStride = kRouteThreads;
  for (int b0 = i0; b0 < i1; b0 += kRouteThreads * kRun) {
    const int b = b0 + tid;
    int32_t id[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) id[j] = b + kStride * j < i1 ? a.topk_ids[b + kStride * j] : 0;
    uint32_t pos[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      const int e = id[j];
      pos[j] = kInvalidRow;
      if (b + kStride * j >= i1) continue;
      if (e < 0 || e >= a.num_routed) {
        *bad = 1;  // contributes nothing; reported in err
        continue;
      }
      pos[j] = atomicAdd(&s_count[e], 1u);
    }
#pragma unroll
    for (int j = 0; j < kRun; ++j)
      if (b + kStride * j < i1) a.tb.row_of_slot[b + kStride * j] = pos[j];
  }
}

// Grouped rows of the routed slots [i0, i1): base(expert) (the expert's
// offset, plus the workgroup's first position in the parallel route) plus the
// slot's position; the token each grouped row reads.  The passes are those of
// count_slots, so each thread reads back the positions it wrote.
template <typename Base>
__device__ void place_slots(const RouteArgs &a, int i0, int i1, Base base) {
  const int tid = threadIdx.x;
  constexpr int kStride = kRouteThreads;
  for (int b0 = i0; b0 < i1; b0 += kRouteThreads * kRun) {
    const int b = b0 + tid;
    uint32_t pos[kRun];
    int32_t id[kRun];
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      const int i = b + kStride * j;
      pos[j] = i < i1 ? a.tb.row_of_slot[i] : kInvalidRow;
      id[j] = i < i1 ? a.topk_ids[i] : 0;
    }
#pragma unroll
    for (int j = 0; j < kRun; ++j) {
      if (pos[j] == kInvalidRow) continue;
      const int i = b + kStride * j;
      const uint32_t row = base(id[j]) + pos[j];
      a.tb.row_of_slot[i] = row;
      a.tb.token_of_row[row] = (uint32_t)(i / a.topk);
      a.tb.slot_of_row[row] = (uint32_t)i;
    }
  }
}

// One workgroup: the whole route in one launch (calls with few slots).
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(RouteArgs a) {
  __shared__ uint32_t s_count[kMoeMaxExperts];
  __shared__ uint32_t s_off[kMoeMaxExperts];
  __shared__ uint32_t s_scan[kRouteThreads];
  __shared__ uint32_t s_total;
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int ne = a.num_routed + a.num_shared;
  const int slots = a.t * a.topk;

  for (int e = tid; e < ne; e += kRouteThreads) s_count[e] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  // 1. position of every routed slot inside its expert's group
  count_slots(a, 0, slots, s_count, &s_bad);
  // shared experts see every token
  for (int e = a.num_routed + tid; e < ne; e += kRouteThreads) s_count[e] = (uint32_t)a.t;
  __syncthreads();
  if (tid == 0) *a.tb.err = s_bad ? 1u : 0u;
  group_and_tile(a, s_count, s_off, s_scan, &s_total);
  // 5. grouped row of every routed slot
  place_slots(a, 0, slots, [&](int e) { return s_off[e]; });
}

// The parallel route (calls with many slots): workgroup g counts the routed
// slots of its chunk [g c, (g+1) c) in LDS and writes its counts; one
// workgroup then turns each expert's counts into per-workgroup first
// positions (workgroup order) and runs steps 2 to 4; every workgroup then
// places its chunk's slots.  Rows are grouped by expert as in the one-
// workgroup route; their order inside a group is workgroup order, then the
// order of the LDS atomics.
struct RouteParArgs {
  RouteArgs r;
  int chunk;  // routed slots per workgroup
};

__global__ __launch_bounds__(kRouteThreads) void moe_route_count_kernel(RouteParArgs p) {
  __shared__ uint32_t s_count[kMoeMaxExperts];
  __shared__ int s_bad;
  const RouteArgs &a = p.r;
  const int tid = threadIdx.x, g = blockIdx.x;
  const int ne = a.num_routed + a.num_shared;
  const int slots = a.t * a.topk;
  const int i0 = min(g * p.chunk, slots), i1 = min(i0 + p.chunk, slots);
  for (int e = tid; e < ne; e += kRouteThreads) s_count[e] = 0;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  count_slots(a, i0, i1, s_count, &s_bad);
  __syncthreads();
  for (int e = tid; e < a.num_routed; e += kRouteThreads)
    a.tb.wg_counts[(size_t)g * ne + e] = s_count[e];
  if (tid == 0) a.tb.wg_err[g] = s_bad ? 1u : 0u;
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_scan_kernel(RouteParArgs p) {
  __shared__ uint32_t s_count[kMoeMaxExperts];
  __shared__ uint32_t s_off[kMoeMaxExperts];
  __shared__ uint32_t s_scan[kRouteThreads];
  __shared__ uint32_t s_total;
  const RouteArgs &a = p.r;
  const int tid = threadIdx.x;
  const int ne = a.num_routed + a.num_shared;
  const int groups = a.tb.route_groups;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.tb.wg_counts, (uint32_t)groups * (uint32_t)ne * 4u);
  // each expert's total, and each workgroup's first position in its group
  for (int e = tid; e < ne; e += kRouteThreads) {
    if (e < a.num_routed) {
      const uint32_t col = (uint32_t)e * 4u;
      // batches of 64 loads before their stores: one wait on memory per batch
      // (one batch up to 64 route workgroups); buffer loads and stores at the
      // column's lane offset plus a uniform row offset, so the batch holds no
      // addresses in registers
      uint32_t run = 0;
      for (int g0 = 0; g0 < groups; g0 += 64) {
        uint32_t v[64];
#pragma unroll
        for (int j = 0; j < 64; ++j)
          v[j] = g0 + j < groups ? __builtin_amdgcn_raw_buffer_load_b32(rw, col, (g0 + j) * ne * 4, 0)
                                 : 0u;
#pragma unroll
        for (int j = 0; j < 64; ++j)
          if (g0 + j < groups) {
            __builtin_amdgcn_raw_buffer_store_b32(run, rw, col, (g0 + j) * ne * 4, 0);
            run += v[j];
          }
      }
      s_count[e] = run;
    } else {
      s_count[e] = (uint32_t)a.t;  // shared experts see every token
    }
  }
  int bad = 0;
  for (int g = tid; g < groups; g += kRouteThreads) bad |= a.tb.wg_err[g] != 0u;
  bad = __syncthreads_or(bad);
  if (tid == 0) *a.tb.err = bad ? 1u : 0u;
  group_and_tile(a, s_count, s_off, s_scan, &s_total);
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_place_kernel(RouteParArgs p) {
  const RouteArgs &a = p.r;
  const int g = blockIdx.x;
  const int ne = a.num_routed + a.num_shared;
  const int slots = a.t * a.topk;
  const int i0 = min(g * p.chunk, slots), i1 = min(i0 + p.chunk, slots);
  const uint32_t *offsets = a.tb.offsets;
  const uint32_t *wgb = a.tb.wg_counts + (size_t)g * ne;
  place_slots(a, i0, i1, [&](int e) { return offsets[e] + wgb[e]; });
}

struct CombineArgs {
  const float *topk_w;
  const float *shared_w;
  int t, topk, num_routed, num_shared, h;
  MoeTables tb;
  void *y;
  int y_bf16;
};

// y[t][n] = sum_j w[t][j] d[t topk + j][n] + sum_s ws[t] d[T topk + s T + t][n],
// fixed order (one fma per term; the decode form runs the same chain in its
// down launch).  d holds one row per token slot (the down launch writes each
// grouped row to its slot's row), so a token's routed rows are consecutive
// and every row's address follows from the token alone.  A block serves VEC x
// 256 columns of one token (the blocks of one token are adjacent in launch
// order, so the token's rows are read front to back).  Each thread issues its
// d loads 16 rows at a time together with the wave's scalar loads of those
// slots' weights and drop marks, so nothing waits on a table before the d
// traffic starts (a dropped slot's row is read and left out of the sum).
// VEC columns per thread (4: 16-byte loads of d when H is a multiple of 4;
// the kernel reads every row of d once, 738 MB at T = 8192 on the 512-expert
// layer, with non-temporal loads).  Measured on that layer (bench, ms per
// layer): table staged in LDS before the loads 1.143, this form with normal
// loads 1.119, with non-temporal loads 1.091; 8 columns per thread (one
// block per token) 1.14.
template <int VEC>
__global__ __launch_bounds__(256) void moe_combine_kernel(CombineArgs a) {
  constexpr int kBatch = 16;
  typedef __attribute__((ext_vector_type(VEC))) float fv_t;
  const int t = blockIdx.y;
  const int n = (blockIdx.x * 256 + threadIdx.x) * VEC;  // first of this thread's columns
  const int total = a.topk + a.num_shared;
  const int nn = min(n, a.h - VEC);
  const size_t slot0 = (size_t)t * a.topk;
  fv_t acc = {};
  for (int j0 = 0; j0 < total; j0 += kBatch) {
    // every loop below runs all kBatch iterations (rows past the token's
    // last are not loaded and not added), so the arrays stay in registers;
    // the sum is a select, not a branch, so that no load is sunk into a
    // conditional use and all of the batch's loads are in flight together
    fv_t v[kBatch];
    float w[kBatch];
    bool ok[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + u;
      const size_t row = j < a.topk ? slot0 + j
                                    : (size_t)a.t * a.topk + (size_t)(j - a.topk) * a.t + t;
      if (j < total)  // uniform
        v[u] = __builtin_nontemporal_load((const fv_t *)(a.tb.d + row * a.h + nn));
      else
        v[u] = fv_t{};
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + u;
      ok[u] = false;
      w[u] = 0.0f;
      if (j < a.topk) {
        ok[u] = a.tb.row_of_slot[slot0 + j] != kInvalidRow;
        w[u] = a.topk_w[slot0 + j];
      } else if (j < total) {
        ok[u] = true;
        w[u] = a.shared_w ? a.shared_w[t] : 1.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float f = __builtin_fmaf(w[u], v[u][e], acc[e]);
        acc[e] = ok[u] ? f : acc[e];
      }
    }
  }
  if (n >= a.h) return;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    if (a.y_bf16)
      ((uint16_t *)a.y)[(size_t)t * a.h + n + e] = (uint16_t)float_to_bf16(acc[e]);
    else
      ((float *)a.y)[(size_t)t * a.h + n + e] = acc[e];
  }
}

size_t align_up(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

// Routing tiles: the smallest of 32, 64, 128, 192 and 256 rows that holds 1.2
// times an average routed expert's rows (t x topk / E).  A tile much taller
// than most experts' rows is mostly padding (the MFMAs of its empty rows
// still run); one much shorter splits most experts in two.  Measured on the
// 512-expert layer, NVFP4, time per layer for tiles of 32 / 64 / 128 / 192 /
// 256 rows: T = 1024 (20 rows per expert) 0.48 / 0.50 / 0.52 / 0.63 / 0.76 ms;
// T = 2048 0.81 / 0.55 / 0.59 / 0.68 / 0.80; T = 4096 1.28 / 0.97 / 0.73 /
// 0.81 / 0.92; T = 8192 2.22 / 1.65 / 1.38 / 1.09 / 1.17.
int moe_tile_rows(const qmm_weight &gu, const qmm_weight &dn, int t, int topk, int num_routed) {
  (void)gu;
  (void)dn;
  const double need = 1.2 * (double)t * topk / num_routed;
  int tr = 256;
  for (int c : {192, 128, 64, 32})
    if (c >= need) tr = c;
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_MOE_TILE")) tr = atoi(e);
#endif
  return tr;
}

// Workgroups of the route pass: one up to kRouteParallelSlots routed slots
// (its single pass is cheaper than three launches there); above, one per
// kRouteSlotsPerGroup slots, at most kRouteMaxGroups.
constexpr size_t kRouteParallelSlots = 16384;
constexpr size_t kRouteSlotsPerGroup = 2048;
constexpr int kRouteMaxGroups = 128;

int route_groups(size_t slots) {
  if (slots <= kRouteParallelSlots) return 1;
  return (int)std::min<size_t>((slots + kRouteSlotsPerGroup - 1) / kRouteSlotsPerGroup, kRouteMaxGroups);
}

MoeLayout moe_layout(int num_experts, int t, int topk, int num_shared, int inter, int hidden,
                     int tile_rows) {
  MoeLayout L{};
  const size_t rows = (size_t)t * topk + (size_t)t * num_shared;
  L.max_rows = rows;
  L.tile_rows = (size_t)tile_rows;
  L.max_tiles = (rows + tile_rows - 1) / tile_rows + (size_t)num_experts;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  L.counts = take((size_t)num_experts * 4);
  L.offsets = take(((size_t)num_experts + 1) * 4);
  L.row_of_slot = take((size_t)t * topk * 4);
  L.row_of_shared = take((size_t)t * num_shared * 4 + 4);
  L.token_of_row = take(rows * 4 + 4);
  L.slot_of_row = take(rows * 4 + 4);
  L.active = take((size_t)num_experts * 4);
  L.scalars = take(16);  // n_active, n_tiles, err
  L.tiles = take(L.max_tiles * 12);
  L.h = take(rows * (size_t)inter * 2);
  L.d = take(rows * (size_t)hidden * 4);
  L.route_groups = (size_t)route_groups((size_t)t * topk);
  L.wg_counts = take(L.route_groups > 1 ? L.route_groups * num_experts * 4 : 0);
  L.wg_err = take(L.route_groups > 1 ? L.route_groups * 4 : 0);
  L.bytes = o;
  return L;
}

MoeTables moe_tables(const MoeLayout &L, void *ws) {
  char *b = (char *)ws;
  MoeTables t;
  t.counts = (uint32_t *)(b + L.counts);
  t.offsets = (uint32_t *)(b + L.offsets);
  t.row_of_slot = (uint32_t *)(b + L.row_of_slot);
  t.row_of_shared = (uint32_t *)(b + L.row_of_shared);
  t.token_of_row = (uint32_t *)(b + L.token_of_row);
  t.slot_of_row = (uint32_t *)(b + L.slot_of_row);
  t.active = (uint32_t *)(b + L.active);
  t.n_active = (uint32_t *)(b + L.scalars);
  t.n_tiles = t.n_active + 1;
  t.err = t.n_active + 2;
  t.tiles = (uint32_t *)(b + L.tiles);
  t.h = (uint16_t *)(b + L.h);
  t.d = (float *)(b + L.d);
  t.wg_counts = (uint32_t *)(b + L.wg_counts);
  t.wg_err = (uint32_t *)(b + L.wg_err);
  t.route_groups = (int)L.route_groups;
  return t;
}

bool moe_uses_gemv(const qmm_weight &gu, const qmm_weight &dn, int t, int topk, int num_shared) {
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_MOE_GEMV")) return atoi(e) != 0 && moe_gemv_fits(gu, dn, t, topk, num_shared);
#endif
  return moe_gemv_fits(gu, dn, t, topk, num_shared);
}

hipError_t launch_moe(const qmm_weight &gu, const qmm_weight &dn, int num_routed, int num_shared,
                      const void *x, int t, const int32_t *topk_ids, const float *topk_w,
                      int topk, const float *shared_w, void *y, int y_dtype, void *workspace,
                      hipStream_t s) {
  const MoeLayout L = moe_layout(num_routed + num_shared, t, topk, num_shared, gu.n / 2, dn.n,
                                moe_tile_rows(gu, dn, t, topk, num_routed));
  const MoeTables tb = moe_tables(L, workspace);
  hipError_t e;
  if (moe_uses_gemv(gu, dn, t, topk, num_shared)) {
    // the decode form's down launch also runs the combine
    return launch_moe_gemv(gu, dn, num_routed, num_shared, x, t, topk_ids, topk_w, topk, shared_w,
                           y, y_dtype == QMM_BF16, tb, s);
  } else {
    RouteArgs ra{topk_ids, t, topk, num_routed, num_shared, (int)L.tile_rows, tb};
    if (tb.route_groups <= 1) {
      hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(kRouteThreads), 0, s, ra);
    } else {
      const int slots = t * topk;
      RouteParArgs rp{ra, (slots + tb.route_groups - 1) / tb.route_groups};
      hipLaunchKernelGGL(moe_route_count_kernel, dim3(tb.route_groups), dim3(kRouteThreads), 0, s, rp);
      hipLaunchKernelGGL(moe_route_scan_kernel, dim3(1), dim3(kRouteThreads), 0, s, rp);
      hipLaunchKernelGGL(moe_route_place_kernel, dim3(tb.route_groups), dim3(kRouteThreads), 0, s, rp);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // weight tiles decoded straight into MFMA operands (gemm_big.hip; the host
    // checks reject calls whose 32-bit offsets it would not reach)
    e = launch_moe_big_gate_up(gu, x, tb, (int)L.max_tiles, (int)L.tile_rows, s);
    if (e != hipSuccess) return e;
    e = launch_moe_big_down(dn, tb, (int)L.max_tiles, (int)L.tile_rows, s);
    if (e != hipSuccess) return e;
  }

  CombineArgs ca{topk_w, shared_w, t, topk, num_routed, num_shared, dn.n, tb, y,
                 y_dtype == QMM_BF16};
  if (dn.n % 4 == 0)
    hipLaunchKernelGGL(moe_combine_kernel<4>, dim3((dn.n + 1023) / 1024, t), dim3(256), 0, s, ca);
  else
    hipLaunchKernelGGL(moe_combine_kernel<1>, dim3((dn.n + 255) / 256, t), dim3(256), 0, s, ca);
  return hipGetLastError();
}

hipError_t launch_moe_logits(const qmm_weight &gu, const qmm_weight &dn, int num_routed,
                             int num_shared, const void *x, int t, const float *logits,
                             int32_t *topk_ids, float *topk_w, int topk, const float *shared_w,
                             void *y, int y_dtype, void *workspace, hipStream_t s) {
  if (moe_uses_gemv(gu, dn, t, topk, num_shared) && moe_router_folds(num_routed)) {
    const MoeLayout L = moe_layout(num_routed + num_shared, t, topk, num_shared, gu.n / 2, dn.n,
                                  moe_tile_rows(gu, dn, t, topk, num_routed));
    return launch_moe_gemv(gu, dn, num_routed, num_shared, x, t, nullptr, nullptr, topk, shared_w,
                           y, y_dtype == QMM_BF16, moe_tables(L, workspace), s, logits, topk_ids,
                           topk_w);
  }
  hipError_t e = launch_router(logits, t, num_routed, topk, topk_ids, topk_w, s);
  if (e != hipSuccess) return e;
  return launch_moe(gu, dn, num_routed, num_shared, x, t, topk_ids, topk_w, topk, shared_w, y,
                    y_dtype, workspace, s);
}

}  // namespace qmm
