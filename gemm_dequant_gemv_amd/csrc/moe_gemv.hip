// qmoe_grouped for decode (up to 16 tokens and 128 token slots, when the
// staged vectors fit in LDS): the expert multiplies as one grouped GEMV
// launch per projection ("TurboEXL3" section 3.1: decode passes 1 to 4
// tokens, and a layer's work must not split into many small dependent
// launches; section 4.2: 1 to 16 rows take the GEMV chain).
//
// With so few tokens nearly every active expert serves one row, so row tiles
// of an MFMA GEMM would be almost empty.  Instead every token slot (routed
// slots in list order, then the shared experts' slots) is its own matrix-
// vector product, streamed like the row-streaming qgemv kernel:
//   * gate/up: a unit is one 1024-value step of the row pair (gate i, up I+i)
//     of the slot's expert, one row per half-wave, against the slot's token;
//     after the pair's last step the two half-wave sums are g and u, and one
//     lane writes h = silu(g) * u (float32, then bfloat16);
//   * down and combine, one launch: an item is (token t, output quad 4p ..
//     4p+3) and a job is one of the item's terms j: the token's slots in
//     combine order (routed slots in list order, then the shared experts).
//     Workgroup g owns a contiguous block of items and splits its jobs evenly
//     over its waves (at 4 tokens there are half as many items as waves).  A
//     unit is one step of a job: the quad's rows of the slot's down matrix,
//     one row per quarter-wave (a quarter-wave covers 512 values, the whole
//     intermediate width at I = 512), against the slot's h; after the job's
//     last step the four sums are d, written to d [slot][H] in float32 and to
//     an LDS slot of the item.  After a barrier one wave per item runs, in
//     lanes 0-3, the chain y = fma(w_j, d_j, y) over the item's terms in
//     order from 0, the chain the grouped form's combine kernel runs.
// The grouped rows are the slots themselves (no routing pass): h and d row s
// belong to slot s, a shared expert's rows follow all routed slots.  Slots
// whose expert id is outside [0, E) are skipped (their rows are never read
// and they add nothing).
#include <algorithm>
#include <atomic>
#include <cstdlib>

#include "gemv_step.h"
#include "router_device.h"
#include "swiglu_device.h"

namespace qmm {
namespace {

constexpr size_t kLdsLimit = 160 * 1024 - 8192;  // dynamic part; the static tables take <= 6.5 KB

struct MoeGemvArgs {
  const uint8_t *codes, *codes_hi, *scales, *scales2;
  const float *tensor_scale;
  uint32_t codes_bytes, hi_bytes, scales_bytes, scales2_bytes;
  int k;            // reduction length: H (gate/up) or I (down)
  int rows;         // rows of one expert's matrix: 2I or H
  int pairs;        // row groups per slot: I (gate/up pairs) or H / 4 (down quads)
  int half_rows;    // rows between the lane groups of a row group: I or 1
  int pair_step;    // rows between consecutive row groups: 1 or 4
  int steps;        // ceil(k / step values)
  const int32_t *topk_ids;
  int t, topk, num_routed, num_shared;
  const uint16_t *src;  // vectors staged in LDS: x [t][H] or h [slots][I]
  int nsrc;
  uint16_t *h;      // gate/up output [slots][I]
  float *d;         // down output [slots][H]
  // down and combine
  const float *topk_w;    // [t][topk]
  const float *shared_w;  // [t] or null (weight 1)
  void *y;                // [t][H] float32, or bfloat16 when y_bf16
  int y_bf16;
  uint32_t *err;          // 1 when an id was outside [0, E)
  // gate/up with the router folded in: logits [t][num_routed] in; the routing
  // out (written by workgroup 0, read by the down launch)
  const float *logits;
  int32_t *ids_out;
  float *w_out;
};

// The router folded into the gate/up launch takes up to 64 x 8 routed experts.
constexpr int kRouterFoldPer = 8;

// LDS layout of the staged vectors: chunk ch (32 values) of vector l at u32
// offset ch * stride + 16 l, stride = 16 nsrc + 4 (the pad spreads the chunks
// of one ds_read over the banks); then the sums of x per chunk (affine) or
// per 16 values (Q6_K), [l][sub][nch].
__host__ __device__ inline size_t moe_gemv_stride(int nsrc) { return 16 * (size_t)nsrc + 4; }

template <bool DOWN>
struct MoeShape {
  static constexpr int kGroups = DOWN ? 4 : 2;      // rows per unit, one per lane group
  static constexpr int kLanes = 64 / kGroups;       // lanes per row
  static constexpr int kStepK = 32 * kLanes;        // values per row per step
};

template <int FMT, bool DOWN, int U, int WAVES, bool ROUTER>
__global__ __launch_bounds__(64 * WAVES) void moe_gemv_kernel(MoeGemvArgs a) {
  static_assert(!(ROUTER && DOWN), "the router folds into the gate/up launch");
  constexpr int kThreads = 64 * WAVES;
  using SH = MoeShape<DOWN>;
  constexpr int kStepK = SH::kStepK;
  using T = FmtTraits<FMT>;
  constexpr int kNS = T::kSums;
  extern __shared__ __align__(16) uint32_t smem[];
  __shared__ float s_w[DOWN ? kMoeGemvMaxSlots : 1];  // combine weight of each slot
  const int nch = a.k / 32;
  const int stride = (int)moe_gemv_stride(a.nsrc);
  uint32_t *xs = smem;
  float *xsum = (float *)(xs + (size_t)nch * stride);

  const int tid = threadIdx.x;
  const int lane = tid & 63, hf = lane / SH::kLanes, c = lane % SH::kLanes;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.steps;
  const uint32_t k = (uint32_t)a.k;
  const int routed = a.t * a.topk;
  const int slots = routed + a.t * a.num_shared;
  // gate/up: items (slot, pair), one pass of S steps each; down: items
  // (token, quad), one pass of S steps for each of the token's J slots
  const int J = DOWN ? a.topk + a.num_shared : 1;
  const int items = (DOWN ? a.t : slots) * a.pairs;
  const int W = gridDim.x * WAVES;
  const int gw = blockIdx.x * WAVES + wave;
  // the wave's jobs: gate/up items gw, gw + W, ... for the rfull whole rounds
  // of W items, then in the last, partial round item rfull W + w G + g
  // (wave-major, so that every workgroup gets its share of that round: with
  // gw there, half the workgroups took one item per wave more than the
  // rest); down jobs [q0, q1) of the workgroup's items [ib0, ib1), item-major
  int ib0 = 0, ib1 = 0, q0 = 0, myjobs, rfull = 0, ilast = 0;
  if constexpr (DOWN) {
    ib0 = (int)((long long)blockIdx.x * items / gridDim.x);
    ib1 = (int)((long long)(blockIdx.x + 1) * items / gridDim.x);
    const int nq = (ib1 - ib0) * J;
    q0 = wave * nq / WAVES;
    myjobs = (wave + 1) * nq / WAVES - q0;
  } else {
    rfull = items / W;
    ilast = rfull * W + wave * (int)gridDim.x + (int)blockIdx.x;
    myjobs = rfull + (ilast < items ? 1 : 0);
  }
  const int units = myjobs * S;
  // the wave's first and last job: (slot or token, pair or quad, term)
  int s_first, p_first, term_first, s_last, p_last, term_last;
  {
    int i0, i1;
    if constexpr (DOWN) {
      const int qa = q0, qb = q0 + max(myjobs, 1) - 1;
      i0 = ib0 + qa / J;
      term_first = qa % J;
      i1 = ib0 + qb / J;
      term_last = qb % J;
    } else {
      i0 = rfull > 0 ? gw : ilast;
      i1 = myjobs > rfull ? ilast : (rfull > 0 ? gw + (rfull - 1) * W : ilast);
      term_first = term_last = 0;
    }
    s_first = i0 / a.pairs;
    p_first = i0 - s_first * a.pairs;
    s_last = i1 / a.pairs;
    p_last = i1 - s_last * a.pairs;
  }
  float *dq = (float *)(xs + (size_t)nch * stride) + (size_t)a.nsrc * kNS * nch;  // down: [items][J][4]

  const __amdgpu_buffer_rsrc_t rc = make_rsrc(a.codes, a.codes_bytes);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.codes_hi, a.hi_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.scales, a.scales_bytes);
  const __amdgpu_buffer_rsrc_t rs2 = make_rsrc(a.scales2, a.scales2_bytes);
  const uint32_t hr = (uint32_t)(hf * a.half_rows);
  const uint32_t v_code = hr * (k / 2) + 16 * c;
  const uint32_t v_scale = FMT == QMM_AFFINE4_G64 ? hr * (k / 16) + (c / 2) * 4
                         : FMT == QMM_MXFP4 ? hr * (k / 32) + c
                         : hr * (k / 16) + 2 * c;
  const uint32_t v_hi = hr * (k / 4) + 8 * c;
  const uint32_t v_d = (hr * (k / 256) + c / 8) * 2;

  // 0. (router folded in) every workgroup routes the call's tokens itself,
  //    one wave per token ("TurboEXL3" section 4.2: the router's top-k and
  //    softmax run inside the chain's first launch), into LDS; workgroup 0
  //    also writes the routing out for the down launch and the caller
  __shared__ int32_t s_rid[ROUTER ? kMoeGemvMaxSlots : 1];
  if constexpr (ROUTER) {
    for (int tk = wave; tk < a.t; tk += WAVES) {
      int id;
      float w;
      router::topk_softmax_wave<kRouterFoldPer>(a.logits + (size_t)tk * a.num_routed,
                                                a.num_routed, a.topk, id, w);
      if (lane < a.topk) {
        s_rid[tk * a.topk + lane] = id;
        if (blockIdx.x == 0) {
          a.ids_out[tk * a.topk + lane] = id;
          a.w_out[tk * a.topk + lane] = w;
        }
      }
    }
    __syncthreads();
  }

  // slot -> expert (-1 for an id outside [0, E)) and staged vector
  auto slot_expert = [&](int s) {
    if (s < routed) {
      const int e = ROUTER ? s_rid[s] : a.topk_ids[s];
      return (e < 0 || e >= a.num_routed) ? -1 : e;
    }
    return a.num_routed + (s - routed) / a.t;
  };
  auto slot_vector = [&](int s) {
    return DOWN ? s : (s < routed ? s / a.topk : (s - routed) % a.t);
  };
  // down: slot of the token's j-th term (routed slots in list order, then the
  // shared experts), and its combine weight
  auto slot_of = [&](int t, int j) {
    return j < a.topk ? t * a.topk + j : routed + (j - a.topk) * a.t + t;
  };
  auto slot_weight = [&](int sl) {
    if (sl < routed) return a.topk_w[sl];
    return a.shared_w ? a.shared_w[(sl - routed) % a.t] : 1.0f;
  };

  // 1. the first units' weights, then the staged vectors.  The expert of a
  //    unit comes from global memory for these first units and from the LDS
  //    table afterwards, so that no later weight load waits for a scalar
  //    load of the routing ids.
  // Gate/up items advance by W: (slot, pair) moves by (W / pairs, W %
  //    pairs), so the walk needs no division per unit, except into the last
  //    round (job rfull); down items advance by one (token, quad).
  const int sW = DOWN ? 0 : W / a.pairs, pW = DOWN ? 1 : W - (W / a.pairs) * a.pairs;
  auto advance = [&](int &s, int &p, int &jn) {
    if (!DOWN && ++jn >= rfull) {
      s = ilast / a.pairs;
      p = ilast - s * a.pairs;
      return;
    }
    s += sW;
    p += pW;
    if (p >= a.pairs) { p -= a.pairs; ++s; }
  };
  // Slot table in registers: lane l holds slot l (tab0, gsc0) and slot
  // 64 + l (tab1, gsc1): valid << 31 | expert << 16 | staged vector (an
  // invalid slot reads expert 0's rows), and the expert's NVFP4 tensor scale;
  // read back with v_readlane at a uniform lane, so every lookup lands in
  // scalar registers.  (An LDS table, or a global load of the tensor scale
  // per item, made the compiler wait for every weight load in flight before
  // each lookup, which undid the load pipeline.)
  uint32_t tab0 = 0, tab1 = 0;
  float gsc0 = 1.0f, gsc1 = 1.0f;
  auto table_entry = [&](int sl, float &gs) {
    const int e = slot_expert(sl);
    gs = (FMT == QMM_NVFP4 && a.tensor_scale && e >= 0) ? a.tensor_scale[e] : 1.0f;
    return (e >= 0 ? 0x80000000u : 0u) | ((uint32_t)max(e, 0) << 16) | (uint32_t)slot_vector(sl);
  };
  auto lookup = [&](int sl) {
    const uint32_t v0 = (uint32_t)__builtin_amdgcn_readlane((int)tab0, sl & 63);
    const uint32_t v1 = (uint32_t)__builtin_amdgcn_readlane((int)tab1, sl & 63);
    return sl < 64 ? v0 : v1;
  };
  auto tensor_scale_of = [&](int sl) {
    const float v0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gsc0), sl & 63));
    const float v1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gsc1), sl & 63));
    return sl < 64 ? v0 : v1;
  };
  auto load_unit = [&](int u, int s, int p, int term, int s_step, RowData &rd, bool from_lds) {
    if (u >= units) {  // uniform: re-read the wave's last unit (or its first job)
      s = s_last;
      p = p_last;
      term = term_last;
      s_step = S - 1;
    }
    if constexpr (DOWN) s = slot_of(min(s, a.t - 1), term);
    s = min(s, slots - 1);
    const int e = from_lds ? (int)((lookup(s) >> 16) & 0x7FFFu) : max(slot_expert(s), 0);
    const uint32_t row0 = (uint32_t)(e * a.rows + p * a.pair_step);
    rd.q = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
        rc, v_code, row0 * (k / 2) + (uint32_t)s_step * (kStepK / 2), 2));
    if constexpr (FMT == QMM_AFFINE4_G64) {
      rd.s = __builtin_amdgcn_raw_buffer_load_b32(
          rs, v_scale, row0 * (k / 16) + (uint32_t)s_step * (kStepK / 16), 0);
    } else if constexpr (FMT == QMM_MXFP4) {
      rd.s = __builtin_amdgcn_raw_buffer_load_b8(
          rs, v_scale, row0 * (k / 32) + (uint32_t)s_step * (kStepK / 32), 0);
    } else {
      rd.s = __builtin_amdgcn_raw_buffer_load_b16(
          rs, v_scale, row0 * (k / 16) + (uint32_t)s_step * (kStepK / 16), 0);
    }
    if constexpr (FMT == QMM_Q6_K) {
      rd.h = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
          rh, v_hi, row0 * (k / 4) + (uint32_t)s_step * (kStepK / 4), 2));
      rd.d = __builtin_amdgcn_raw_buffer_load_b16(
          rs2, v_d, (row0 * (k / 256) + (uint32_t)s_step * (kStepK / 256)) * 2, 0);
    }
  };
  RowData buf[U];
  int ls = 0, lt = term_first, l_s = s_first, l_p = p_first, l_j = 0;  // next unit to load
  auto advance_unit = [&](int &st, int &term, int &s, int &p, int &jn) {
    if (++st == S) {
      st = 0;
      if (++term == J) { term = 0; advance(s, p, jn); }
    }
  };
#pragma unroll
  for (int j = 0; j < U; ++j) {
    load_unit(j, l_s, l_p, lt, ls, buf[j], false);
    advance_unit(ls, lt, l_s, l_p, l_j);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (lane < slots) tab0 = table_entry(lane, gsc0);
  if (lane + 64 < slots) tab1 = table_entry(lane + 64, gsc1);
  if constexpr (DOWN) {
    for (int i = tid; i < slots; i += kThreads) s_w[i] = slot_weight(i);
  }
  if constexpr (DOWN) {
    // the decode form has no routing pass: report dropped ids here
    if (blockIdx.x == 0) {
      int bad = 0;
      for (int i = tid; i < routed; i += kThreads)
        bad |= (a.topk_ids[i] < 0 || a.topk_ids[i] >= a.num_routed) ? 1 : 0;
      bad = __syncthreads_or(bad);
      if (tid == 0) *a.err = bad ? 1u : 0u;
    }
  }

  const int pieces = a.nsrc * nch * 4;  // 16-byte pieces, [vector][chunk][part]
  constexpr int XP = 4;                  // pieces per thread in flight
  // a load with no piece to fetch points past the end of the buffer and
  // returns zeros without a memory access (clamped copies of the last piece
  // from every wave would all queue on the one L2 channel holding it)
  const uint32_t src_bytes = (uint32_t)pieces * 16u;
  const __amdgpu_buffer_rsrc_t rsrc_x = make_rsrc(a.src, src_bytes);
  for (int i0 = 0; i0 < pieces; i0 += XP * kThreads) {  // uniform trip count
    uint4 xv[XP];
#pragma unroll
    for (int u = 0; u < XP; ++u) {
      const int i = i0 + u * kThreads + tid;
      const int l = i / (nch * 4), ch = (i / 4) % nch, part = i & 3;
      const uint32_t off = i < pieces ? ((uint32_t)l * a.k + ch * 32 + part * 8) * 2u : src_bytes;
      xv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc_x, off, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < XP; ++u) {
      const bool ok = i0 + u * kThreads + tid < pieces;
      const int i = min(i0 + u * kThreads + tid, pieces - 1);
      const int l = i / (nch * 4), ch = (i / 4) % nch, part = i & 3;
      const uint4 v = xv[u];
      if constexpr (kNS > 0) {
        float sm = ((bf_lo(v.x) + bf_hi(v.x)) + (bf_lo(v.y) + bf_hi(v.y))) +
                   ((bf_lo(v.z) + bf_hi(v.z)) + (bf_lo(v.w) + bf_hi(v.w)));
        sm += __shfl_xor(sm, 1);
        if constexpr (kNS == 1) {
          sm += __shfl_xor(sm, 2);
          if (ok && part == 0) xsum[l * nch + ch] = sm;
        } else {
          if (ok && (part & 1) == 0) xsum[(l * 2 + (part >> 1)) * nch + ch] = sm;
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
        *(uint4 *)(xs + ch * stride + l * 16 + part * 4) = o;
      }
    }
  }
  __syncthreads();

  // The table's loads were waited for at the barrier above (loads complete
  // in order and the staged vectors were loaded after them); passing the
  // values through an empty asm tells the compiler so, which keeps it from
  // waiting for every load in flight at each lookup in the loop below.
  asm volatile("" : "+v"(tab0), "+v"(tab1), "+v"(gsc0), "+v"(gsc1));
  // 2. the units: unit (item, term, step) of this wave
  const UnpackK K = unpack_consts();
  float acc[1] = {0.0f};
  int cs = 0, ct = term_first, c_s = s_first, c_p = p_first, c_j = 0;  // unit being computed
  for (int t0 = 0; t0 < units; t0 += U) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (t0 + j < units) {  // uniform
        const int s = DOWN ? slot_of(c_s, ct) : c_s, p = c_p;
        const uint32_t ent = lookup(s);
        const bool valid = (ent >> 31) != 0;
        const int l = (int)(ent & 0xFFFFu);
        const int ch = cs * SH::kLanes + c;
        if (ch < nch) {
          uint32_t X[1][16];
          float Sx[1][2];
          const uint4 *src = (const uint4 *)(xs + ch * stride + l * 16);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint4 v = src[q];
            X[0][4 * q + 0] = v.x;
            X[0][4 * q + 1] = v.y;
            X[0][4 * q + 2] = v.z;
            X[0][4 * q + 3] = v.w;
          }
          Sx[0][0] = kNS > 0 ? xsum[(l * (kNS > 0 ? kNS : 1)) * nch + ch] : 0.0f;
          Sx[0][1] = kNS > 1 ? xsum[(l * 2 + 1) * nch + ch] : 0.0f;
          row_step<FMT, 1>(buf[j], X, Sx, acc, K);
        }
        if (cs == S - 1) {  // the item's rows are complete
          const float g = tensor_scale_of(s);
          if constexpr (!DOWN) {
            float s0, s1;
            half_sums(acc[0], s0, s1);
            if (valid && lane == 0) {
              const float gv = s0 * g, uv = s1 * g;
              const float hv = silu_f32(gv) * uv;
              a.h[(size_t)s * a.pairs + p] = (uint16_t)float_to_bf16(hv);
            }
          } else {
            float q4[4];
            quarter_sums(acc[0], q4);
            const float v = lane == 0 ? q4[0] : lane == 1 ? q4[1] : lane == 2 ? q4[2] : q4[3];
            const float dv = v * g;
            if (lane < 4) {
              if (valid) a.d[(size_t)s * a.rows + 4 * p + lane] = dv;
              dq[((size_t)(c_s * a.pairs + p - ib0) * J + ct) * 4 + lane] = dv;
            }
          }
          acc[0] = 0.0f;
        }
        advance_unit(cs, ct, c_s, c_p, c_j);
      }
      load_unit(t0 + j + U, l_s, l_p, lt, ls, buf[j], true);
      advance_unit(ls, lt, l_s, l_p, l_j);
    }
  }

  if constexpr (DOWN) {
    // the combine: one wave per item, lanes 0-3 its four outputs, the terms
    // in order, dropped slots skipped
    __syncthreads();
    for (int il = wave; il < ib1 - ib0; il += WAVES) {
      const int item = ib0 + il, tok = item / a.pairs, p = item - tok * a.pairs;
      if (lane < 4) {
        float y = 0.0f;
        for (int j = 0; j < J; ++j) {
          const int sl = slot_of(tok, j);
          if (lookup(sl) >> 31) y = __builtin_fmaf(s_w[sl], dq[((size_t)il * J + j) * 4 + lane], y);
        }
        const size_t o = (size_t)tok * a.rows + 4 * p + lane;
        if (a.y_bf16)
          ((uint16_t *)a.y)[o] = (uint16_t)float_to_bf16(y);
        else
          ((float *)a.y)[o] = y;
      }
    }
  }
}

int cu_count_moe() {
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

// (units in flight, waves per workgroup, workgroups per compute unit)
struct MoeGemvCfg {
  int u, waves, wpc;
};

MoeGemvCfg moe_gemv_cfg(bool down) {
  // measured best on the 512-expert decode layer (the down launch: 2 units in
  // flight 14.4 us, 4 15.1 us, 8 16.4 us)
  (void)down;
  MoeGemvCfg c{2, 16, 1};
#ifdef QMM_TUNE
  if (const char *e = getenv("QMM_MOE_U")) c.u = atoi(e);
  if (const char *e = getenv("QMM_MOE_WAVES")) c.waves = atoi(e);
  if (const char *e = getenv("QMM_MOE_WPC")) c.wpc = atoi(e);
#endif
  return c;
}

template <int FMT, bool DOWN, int U, int WAVES, bool ROUTER>
hipError_t launch_one(const MoeGemvArgs &a, size_t lds, int grid, hipStream_t s) {
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(raised.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void *)moe_gemv_kernel<FMT, DOWN, U, WAVES, ROUTER>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsLimit);
    if (e != hipSuccess) return e;
    raised.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL((moe_gemv_kernel<FMT, DOWN, U, WAVES, ROUTER>), dim3(grid), dim3(64 * WAVES), lds, s, a);
  return hipGetLastError();
}

#ifdef QMM_TUNE
#define QMM_MOE_GEMV_CONFIGS(X) X(2, 16) X(4, 16) X(2, 8) X(4, 8) X(8, 8) X(4, 4) X(8, 4)
#else
#define QMM_MOE_GEMV_CONFIGS(X) X(2, 16)
#endif

template <int FMT, bool DOWN, bool ROUTER>
hipError_t launch_cfg(const MoeGemvCfg &c, const MoeGemvArgs &a, size_t lds, int grid, hipStream_t s) {
#define QMM_CASE(UU, WW) \
  if (c.u == UU && c.waves == WW) return launch_one<FMT, DOWN, UU, WW, ROUTER>(a, lds, grid, s);
  QMM_MOE_GEMV_CONFIGS(QMM_CASE)
#undef QMM_CASE
  return hipErrorInvalidConfiguration;
}

template <bool DOWN, bool ROUTER = false>
hipError_t launch_fmt(int format, const MoeGemvArgs &a, size_t lds, int grid, hipStream_t s) {
  const MoeGemvCfg c = moe_gemv_cfg(DOWN);
  switch (format) {
    case QMM_AFFINE4_G64: return launch_cfg<QMM_AFFINE4_G64, DOWN, ROUTER>(c, a, lds, grid, s);
    case QMM_MXFP4: return launch_cfg<QMM_MXFP4, DOWN, ROUTER>(c, a, lds, grid, s);
    case QMM_NVFP4: return launch_cfg<QMM_NVFP4, DOWN, ROUTER>(c, a, lds, grid, s);
    default: return launch_cfg<QMM_Q6_K, DOWN, ROUTER>(c, a, lds, grid, s);
  }
}

size_t stage_lds(int format, int k, int nsrc) {
  const int sums = format == QMM_AFFINE4_G64 ? 1 : (format == QMM_Q6_K ? 2 : 0);
  const size_t nch = (size_t)k / 32;
  return nch * moe_gemv_stride(nsrc) * 4 + (size_t)nsrc * sums * nch * 4;
}

int moe_grid() { return cu_count_moe() * moe_gemv_cfg(true).wpc; }

// the down launch: staged h, then the d quads of the workgroup's items
size_t down_lds(const qmm_weight &dn, int t, int topk, int num_shared, int grid) {
  const int slots = t * (topk + num_shared);
  const size_t items = (size_t)t * (dn.n / 4);
  const size_t per_wg = (items + grid - 1) / grid;
  return stage_lds(dn.format, dn.k, slots) + per_wg * (topk + num_shared) * 16;
}

MoeGemvArgs weight_args(const qmm_weight &w) {
  MoeGemvArgs a{};
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
  a.k = w.k;
  a.rows = w.n;
  return a;
}

}  // namespace

bool moe_gemv_fits(const qmm_weight &gu, const qmm_weight &dn, int t, int topk, int num_shared) {
  if (t > kMoeGemvMaxTokens) return false;
  const int slots = t * (topk + num_shared);
  if (slots > kMoeGemvMaxSlots || dn.n % 4 != 0) return false;
  if (cu_count_moe() <= 0) return false;
  return stage_lds(gu.format, gu.k, t) <= kLdsLimit &&
         down_lds(dn, t, topk, num_shared, moe_grid()) <= kLdsLimit;
}

bool moe_router_folds(int num_routed) { return num_routed <= 64 * kRouterFoldPer; }

hipError_t launch_moe_gemv(const qmm_weight &gu, const qmm_weight &dn, int num_routed,
                           int num_shared, const void *x, int t, const int32_t *topk_ids,
                           const float *topk_w, int topk, const float *shared_w, void *y,
                           int y_bf16, const MoeTables &tb, hipStream_t s, const float *logits,
                           int32_t *ids_out, float *w_out) {
  if (logits) {  // the router folded into the gate/up launch writes the routing
    topk_ids = ids_out;
    topk_w = w_out;
  }
  const int slots = t * (topk + num_shared);
  const int inter = gu.n / 2;

  MoeGemvArgs g = weight_args(gu);
  g.steps = (gu.k + MoeShape<false>::kStepK - 1) / MoeShape<false>::kStepK;
  g.pairs = inter;
  g.half_rows = inter;
  g.pair_step = 1;
  g.topk_ids = topk_ids;
  g.t = t;
  g.topk = topk;
  g.num_routed = num_routed;
  g.num_shared = num_shared;
  g.src = (const uint16_t *)x;
  g.nsrc = t;
  g.h = tb.h;
  const int grid = moe_grid();
  g.logits = logits;
  g.ids_out = ids_out;
  g.w_out = w_out;
  hipError_t e = logits ? launch_fmt<false, true>(gu.format, g, stage_lds(gu.format, gu.k, t), grid, s)
                        : launch_fmt<false>(gu.format, g, stage_lds(gu.format, gu.k, t), grid, s);
  if (e != hipSuccess) return e;

  MoeGemvArgs d = weight_args(dn);
  d.steps = (dn.k + MoeShape<true>::kStepK - 1) / MoeShape<true>::kStepK;
  d.pairs = dn.n / 4;
  d.half_rows = 1;
  d.pair_step = 4;
  d.topk_ids = topk_ids;
  d.t = t;
  d.topk = topk;
  d.num_routed = num_routed;
  d.num_shared = num_shared;
  d.src = tb.h;
  d.nsrc = slots;
  d.d = tb.d;
  d.topk_w = topk_w;
  d.shared_w = shared_w;
  d.y = y;
  d.y_bf16 = y_bf16;
  d.err = tb.err;
  return launch_fmt<true>(dn.format, d, down_lds(dn, t, topk, num_shared, grid), grid, s);
}

}  // namespace qmm
