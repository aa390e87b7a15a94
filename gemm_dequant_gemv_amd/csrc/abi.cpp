// The C ABI of libqmm: argument validation on the host, workspace sizing, and
// dispatch to the kernels on the caller's stream.  Nothing here allocates,
// frees or synchronizes.
#include <algorithm>
#include <stdint.h>

#include "qmm.h"
#include "qmm_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return QMM_OK;
  g_last_hip_error = (int)e;
  return QMM_ERR_HIP;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
  uintptr_t lo, hi;
};
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }
Range range(const void *p, size_t bytes) { return Range{(uintptr_t)p, (uintptr_t)p + bytes}; }

size_t codes_bytes(const qmm_weight &w) { return (size_t)w.batch * w.n * (size_t)(w.k / 2); }
size_t hi_bytes(const qmm_weight &w) { return (size_t)w.batch * w.n * (size_t)(w.k / 4); }
size_t scales_bytes(const qmm_weight &w) {
  const size_t rows = (size_t)w.batch * w.n;
  switch (w.format) {
    case QMM_AFFINE4_G64: return rows * (w.k / 64) * 4;
    case QMM_MXFP4: return rows * (w.k / 32);
    case QMM_NVFP4: return rows * (w.k / 16);
    default: return rows * (w.k / 16);
  }
}
size_t scales2_bytes(const qmm_weight &w) { return (size_t)w.batch * w.n * (size_t)(w.k / 256) * 2; }

// Every byte range the weight occupies (for aliasing checks).
int weight_ranges(const qmm_weight &w, Range out[5]) {
  int n = 0;
  out[n++] = range(w.codes, codes_bytes(w));
  out[n++] = range(w.scales, scales_bytes(w));
  if (w.codes_hi) out[n++] = range(w.codes_hi, hi_bytes(w));
  if (w.scales2) out[n++] = range(w.scales2, scales2_bytes(w));
  if (w.tensor_scale) out[n++] = range(w.tensor_scale, (size_t)w.batch * 4);
  return n;
}

int check_weight(const qmm_weight *w) {
  if (!w) return QMM_ERR_NULL;
  if (w->format < QMM_AFFINE4_G64 || w->format > QMM_Q6_K) return QMM_ERR_FORMAT;
  if (!w->codes || !w->scales) return QMM_ERR_NULL;
  const bool q6 = w->format == QMM_Q6_K;
  if (q6 && (!w->codes_hi || !w->scales2)) return QMM_ERR_NULL;
  if (!q6 && (w->codes_hi || w->scales2)) return QMM_ERR_FORMAT;
  if (w->tensor_scale && w->format != QMM_NVFP4) return QMM_ERR_FORMAT;
  if (w->n < 1 || w->k < 32 || w->batch < 1) return QMM_ERR_SHAPE;
  if (w->k % 32 != 0) return QMM_ERR_SHAPE;
  // every row of every scale plane starts on a 4-byte boundary
  if (w->format == QMM_AFFINE4_G64 && w->k % 64 != 0) return QMM_ERR_SHAPE;
  if (w->format == QMM_NVFP4 && w->k % 64 != 0) return QMM_ERR_SHAPE;
  if (w->format == QMM_MXFP4 && w->k % 128 != 0) return QMM_ERR_SHAPE;
  if (q6 && w->k % 256 != 0) return QMM_ERR_SHAPE;
  // every plane is addressed with 32-bit byte offsets
  if ((uint64_t)w->batch * (uint64_t)w->n * (uint64_t)(w->k / 2) >= (1ull << 32)) return QMM_ERR_SHAPE;
  if (!aligned(w->codes, 16) || !aligned(w->scales, 4)) return QMM_ERR_ALIGN;
  if (q6 && (!aligned(w->codes_hi, 8) || !aligned(w->scales2, 2))) return QMM_ERR_ALIGN;
  if (w->tensor_scale && !aligned(w->tensor_scale, 4)) return QMM_ERR_ALIGN;
  return QMM_OK;
}

}  // namespace

extern "C" {

const char *qstatus_string(int status) {
  switch (status) {
    case QMM_OK: return "ok";
    case QMM_ERR_NULL: return "a required pointer is NULL";
    case QMM_ERR_FORMAT: return "unknown format, or a plane the format does not have";
    case QMM_ERR_SHAPE: return "shape out of range, or k not a multiple of 32 and of the format's k granule (64 affine and NVFP4, 128 MXFP4, 256 Q6_K)";
    case QMM_ERR_ALIGN: return "pointer not aligned as required";
    case QMM_ERR_M_RANGE: return "m (activation rows) out of range for this call";
    case QMM_ERR_WORKSPACE: return "workspace missing or too small";
    case QMM_ERR_ALIAS: return "an output overlaps an input";
    case QMM_ERR_HIP: return "a HIP runtime call failed";
    case QMM_ERR_DTYPE: return "unknown output dtype";
    case QMM_ERR_ARG: return "argument out of range";
    case QMM_ERR_SCRATCH: return "the call needs more scratch than the static 16 MiB buffer of the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int qlast_hip_error(void) { return g_last_hip_error; }

int qworkspace_init(void *workspace, size_t workspace_bytes, void *stream) {
  if (workspace_bytes == 0) return QMM_OK;
  if (!workspace) return QMM_ERR_NULL;
  if (!aligned(workspace, 4)) return QMM_ERR_ALIGN;
  return hip_status(qmm::launch_zero(workspace, workspace_bytes, (hipStream_t)stream));
}

int qdequant(const qmm_weight *w, int32_t out_dtype, void *out, void *stream) {
  int st = check_weight(w);
  if (st) return st;
  if (out_dtype != QMM_F32 && out_dtype != QMM_BF16) return QMM_ERR_DTYPE;
  if (!out) return QMM_ERR_NULL;
  if (!aligned(out, 16)) return QMM_ERR_ALIGN;
  const size_t ob = (size_t)w->batch * w->n * (size_t)w->k * (out_dtype == QMM_F32 ? 4 : 2);
  Range rs[5];
  const int nr = weight_ranges(*w, rs);
  for (int i = 0; i < nr; ++i)
    if (overlap(range(out, ob), rs[i])) return QMM_ERR_ALIAS;
  return hip_status(qmm::launch_dequant(*w, out_dtype, out, (hipStream_t)stream));
}

int qbench_stream_read(const void *buf, size_t bytes, void *sink, int32_t blocks, void *stream) {
  if (!buf || !sink) return QMM_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return QMM_ERR_ALIGN;
  if (bytes == 0 || bytes % 16 != 0) return QMM_ERR_SHAPE;
  if (blocks < 1 || blocks > (1 << 20)) return QMM_ERR_ARG;
  if (overlap(range(sink, 4), range(buf, bytes))) return QMM_ERR_ALIAS;
  return hip_status(
      qmm::launch_stream_read(buf, bytes, (uint32_t *)sink, blocks, (hipStream_t)stream));
}

int qbench_mfma_peak(int32_t iters, int32_t blocks, void *sink, double *flops, void *stream) {
  if (!sink) return QMM_ERR_NULL;
  if (!aligned(sink, 4)) return QMM_ERR_ALIGN;
  if (iters < 1 || iters > (1 << 24) || blocks < 1 || blocks > (1 << 20)) return QMM_ERR_ARG;
  if (flops) *flops = qmm::mfma_peak_flops(iters, blocks);
  return hip_status(qmm::launch_mfma_peak(iters, (float *)sink, blocks, (hipStream_t)stream));
}

size_t qgemv_workspace_size(const qmm_weight *w, int32_t m) {
  if (check_weight(w) || m < 1 || m > 4) return 0;
  return qmm::plan_gemv(w->format, w->n, w->k, m).ws_bytes;
}

int qgemv(const qmm_weight *w, const void *x, int32_t m, const void *residual, void *y,
          int32_t y_dtype, void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_weight(w);
  if (st) return st;
  if (w->batch != 1) return QMM_ERR_SHAPE;
  if (m < 1 || m > 4) return QMM_ERR_M_RANGE;
  if (y_dtype != QMM_F32 && y_dtype != QMM_BF16) return QMM_ERR_DTYPE;
  if (!x || !y) return QMM_ERR_NULL;
  const size_t esz = y_dtype == QMM_F32 ? 4 : 2;
  if (!aligned(x, 16) || !aligned(y, esz) || (residual && !aligned(residual, 2)))
    return QMM_ERR_ALIGN;
  const qmm::GemvPlan p = qmm::plan_gemv(w->format, w->n, w->k, m);
  if (p.ws_bytes) {
    if (!workspace) return QMM_ERR_WORKSPACE;
    if (workspace_bytes < p.ws_bytes) return QMM_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QMM_ERR_ALIGN;
  }
  const Range ry = range(y, (size_t)m * w->n * esz);
  Range ins[8];
  int ni = weight_ranges(*w, ins);
  ins[ni++] = range(x, (size_t)m * w->k * 2);
  if (residual) ins[ni++] = range(residual, (size_t)m * w->n * 2);
  if (p.ws_bytes) ins[ni++] = range(workspace, p.ws_bytes);
  for (int i = 0; i < ni; ++i)
    if (overlap(ry, ins[i])) return QMM_ERR_ALIAS;
  if (p.ws_bytes) {
    const Range rw = range(workspace, p.ws_bytes);
    for (int i = 0; i < ni - 1; ++i)
      if (overlap(rw, ins[i])) return QMM_ERR_ALIAS;
  }
  return hip_status(qmm::launch_gemv(*w, x, m, residual, y, y_dtype, workspace, p,
                                     (hipStream_t)stream));
}

size_t qgemm_workspace_size(const qmm_weight *w, int32_t m) {
  if (check_weight(w) || w->batch != 1 || w->k % 64 != 0 || m < 1) return 0;
  return qmm::gemm_workspace_size(*w, m);
}

int qgemm(const qmm_weight *w, const void *x, int32_t m, const void *residual, void *y,
          void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_weight(w);
  if (st) return st;
  if (w->batch != 1) return QMM_ERR_SHAPE;
  if (w->k % 64 != 0) return QMM_ERR_SHAPE;
  if (workspace && !aligned(workspace, 256)) return QMM_ERR_ALIGN;
  if (m < 1) return QMM_ERR_M_RANGE;
  // the kernel addresses x and the weight planes with 32-bit offsets
  if (!qmm::gemm_big_fits(*w, (size_t)m)) return QMM_ERR_SHAPE;
  if (!x || !y) return QMM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16) || (residual && !aligned(residual, 16)))
    return QMM_ERR_ALIGN;
  const Range ry = range(y, (size_t)m * w->n * 2);
  Range ins[8];
  int ni = weight_ranges(*w, ins);
  ins[ni++] = range(x, (size_t)m * w->k * 2);
  if (residual) ins[ni++] = range(residual, (size_t)m * w->n * 2);
  for (int i = 0; i < ni; ++i)
    if (overlap(ry, ins[i])) return QMM_ERR_ALIAS;
  if (workspace) {
    const Range rw = range(workspace, workspace_bytes);
    if (overlap(rw, ry)) return QMM_ERR_ALIAS;
    for (int i = 0; i < ni; ++i)
      if (overlap(rw, ins[i])) return QMM_ERR_ALIAS;
  }
  return hip_status(
      qmm::launch_gemm_big(*w, x, m, residual, y, workspace, workspace_bytes, (hipStream_t)stream));
}

namespace {

int hadamard_check(const void *in, int32_t m, int32_t len, size_t in_esz, const void *scale,
                   const void *out, size_t out_esz) {
  if (!in || !out) return QMM_ERR_NULL;
  if (m < 1) return QMM_ERR_M_RANGE;
  if (len < 128 || len % 128 != 0 || (uint64_t)m * (uint64_t)len >= (1ull << 31))
    return QMM_ERR_SHAPE;
  if (!aligned(in, in_esz) || !aligned(out, out_esz) || (scale && !aligned(scale, 2)))
    return QMM_ERR_ALIGN;
  const Range ro = range(out, (size_t)m * len * out_esz);
  if (overlap(ro, range(in, (size_t)m * len * in_esz))) return QMM_ERR_ALIAS;
  if (scale && overlap(ro, range(scale, (size_t)len * 2))) return QMM_ERR_ALIAS;
  return QMM_OK;
}

}  // namespace

int qhadamard_prepare(const void *x, int32_t m, int32_t k, const void *in_scale, void *out,
                      void *stream) {
  const int st = hadamard_check(x, m, k, 2, in_scale, out, 2);
  if (st) return st;
  return hip_status(qmm::launch_hadamard(true, x, m, k, in_scale, out, 1, (hipStream_t)stream));
}

int qhadamard_finish(const float *y, int32_t m, int32_t n, const void *out_scale, void *out,
                     int32_t out_dtype, void *stream) {
  if (out_dtype != QMM_F32 && out_dtype != QMM_BF16) return QMM_ERR_DTYPE;
  const int st = hadamard_check(y, m, n, 4, out_scale, out, out_dtype == QMM_F32 ? 4 : 2);
  if (st) return st;
  return hip_status(qmm::launch_hadamard(false, y, m, n, out_scale, out, out_dtype == QMM_BF16,
                                         (hipStream_t)stream));
}

namespace {

// qgemv_hadamard's workspace: the prepared activations, the float32 product
// when y is bf16, then qgemv's own split-K workspace
struct HadWs {
  size_t xp, ylin, gemv, total;
};

HadWs had_ws(const qmm_weight &w, int m, int y_dtype) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  HadWs h;
  h.xp = up((size_t)m * w.k * 2);
  h.ylin = y_dtype == QMM_BF16 ? up((size_t)m * w.n * 4) : 0;
  h.gemv = qmm::plan_gemv(w.format, w.n, w.k, m).ws_bytes;
  h.total = h.xp + h.ylin + h.gemv;
  return h;
}

}  // namespace

size_t qgemv_hadamard_workspace_size(const qmm_weight *w, int32_t m, int32_t y_dtype) {
  if (check_weight(w) || m < 1 || m > 4) return 0;
  if (y_dtype != QMM_F32 && y_dtype != QMM_BF16) return 0;
  return had_ws(*w, m, y_dtype).total;
}

int qgemv_hadamard(const qmm_weight *w, const void *x, int32_t m, const void *in_scale,
                   const void *out_scale, void *y, int32_t y_dtype, void *workspace,
                   size_t workspace_bytes, void *stream) {
  int st = check_weight(w);
  if (st) return st;
  if (w->batch != 1) return QMM_ERR_SHAPE;
  if (m < 1 || m > 4) return QMM_ERR_M_RANGE;
  if (y_dtype != QMM_F32 && y_dtype != QMM_BF16) return QMM_ERR_DTYPE;
  if (!x || !y || !workspace) return x && y ? QMM_ERR_WORKSPACE : QMM_ERR_NULL;
  if (w->k % 128 != 0 || w->n % 128 != 0) return QMM_ERR_SHAPE;
  const size_t esz = y_dtype == QMM_F32 ? 4 : 2;
  if (!aligned(x, 2) || !aligned(y, esz) || (in_scale && !aligned(in_scale, 2)) ||
      (out_scale && !aligned(out_scale, 2)))
    return QMM_ERR_ALIGN;
  const HadWs h = had_ws(*w, m, y_dtype);
  if (workspace_bytes < h.total) return QMM_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return QMM_ERR_ALIGN;
  const Range ry = range(y, (size_t)m * w->n * esz);
  const Range rw = range(workspace, h.total);
  Range ins[10];
  int ni = weight_ranges(*w, ins);
  ins[ni++] = range(x, (size_t)m * w->k * 2);
  if (in_scale) ins[ni++] = range(in_scale, (size_t)w->k * 2);
  if (out_scale) ins[ni++] = range(out_scale, (size_t)w->n * 2);
  if (overlap(ry, rw)) return QMM_ERR_ALIAS;
  for (int i = 0; i < ni; ++i)
    if (overlap(ry, ins[i]) || overlap(rw, ins[i])) return QMM_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  char *ws = (char *)workspace;
  void *xp = ws;
  // the float32 product lands in y (finish then runs in place: each wave
  // reads its 128-block before writing it) or, for a bf16 y, in the workspace
  void *ylin = h.ylin ? (void *)(ws + h.xp) : y;
  void *gws = h.gemv ? (void *)(ws + h.xp + h.ylin) : nullptr;
  hipError_t e = qmm::launch_hadamard(true, x, m, w->k, in_scale, xp, 1, s);
  if (e != hipSuccess) return hip_status(e);
  e = qmm::launch_gemv(*w, xp, m, nullptr, ylin, QMM_F32, gws,
                       qmm::plan_gemv(w->format, w->n, w->k, m), s);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(qmm::launch_hadamard(false, ylin, m, w->n, out_scale, y, y_dtype == QMM_BF16, s));
}

int qquant_mxfp4(const void *x, int32_t m, int32_t k, void *codes, void *scales, void *stream) {
  if (!x || !codes || !scales) return QMM_ERR_NULL;
  if (m < 1) return QMM_ERR_M_RANGE;
  if (k < 32 || k % 32 != 0 || (uint64_t)m * (uint64_t)k >= (1ull << 32)) return QMM_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(codes, 16)) return QMM_ERR_ALIGN;
  const Range rx = range(x, (size_t)m * k * 2);
  const Range rc = range(codes, (size_t)m * (k / 2));
  const Range rs = range(scales, (size_t)m * (k / 32));
  if (overlap(rc, rx) || overlap(rs, rx) || overlap(rc, rs)) return QMM_ERR_ALIAS;
  return hip_status(qmm::launch_quant_mxfp4(x, m, k, codes, scales, (hipStream_t)stream));
}

size_t qgemm_w4a4_workspace_size(const qmm_weight *w, int32_t m) {
  if (check_weight(w) || w->format != QMM_MXFP4 || w->batch != 1 || m < 1) return 0;
  return qmm::w4a4_workspace_size(m, w->k);
}

int qgemm_w4a4(const qmm_weight *w, const void *x, int32_t m, const void *residual, void *y,
               void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_weight(w);
  if (st) return st;
  if (w->format != QMM_MXFP4) return QMM_ERR_FORMAT;
  if (w->batch != 1) return QMM_ERR_SHAPE;
  if (m < 1) return QMM_ERR_M_RANGE;
  if (!qmm::w4a4_fits(*w, m)) return QMM_ERR_SHAPE;
  if (!x || !y) return QMM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16) || (residual && !aligned(residual, 16)))
    return QMM_ERR_ALIGN;
  const size_t need = qmm::w4a4_workspace_size(m, w->k);
  if (!workspace || workspace_bytes < need) return QMM_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return QMM_ERR_ALIGN;
  const Range ry = range(y, (size_t)m * w->n * 2);
  const Range rw = range(workspace, need);
  Range ins[8];
  int ni = weight_ranges(*w, ins);
  ins[ni++] = range(x, (size_t)m * w->k * 2);
  if (residual) ins[ni++] = range(residual, (size_t)m * w->n * 2);
  if (overlap(ry, rw)) return QMM_ERR_ALIAS;
  for (int i = 0; i < ni; ++i)
    if (overlap(ry, ins[i]) || overlap(rw, ins[i])) return QMM_ERR_ALIAS;
  return hip_status(qmm::launch_gemm_w4a4(*w, x, m, residual, y, workspace, (hipStream_t)stream));
}

size_t qmoe_workspace_size(const qmm_weight *gate_up, const qmm_weight *down, int32_t num_routed,
                           int32_t num_shared, int32_t t, int32_t topk) {
  if (check_weight(gate_up) || check_weight(down) || num_routed < 1 || num_shared < 0 ||
      t < 1 || topk < 1)
    return 0;
  return qmm::moe_layout(num_routed + num_shared, t, topk, num_shared, gate_up->n / 2, down->n,
                         qmm::moe_tile_rows(*gate_up, *down, t, topk, num_routed))
      .bytes;
}

int qmoe_workspace_layout(const qmm_weight *gate_up, const qmm_weight *down, int32_t num_routed,
                          int32_t num_shared, int32_t t, int32_t topk, qmoe_layout *out) {
  if (!out) return QMM_ERR_NULL;
  if (check_weight(gate_up) || check_weight(down) || num_routed < 1 || num_shared < 0 ||
      t < 1 || topk < 1)
    return QMM_ERR_ARG;
  const qmm::MoeLayout L =
      qmm::moe_layout(num_routed + num_shared, t, topk, num_shared, gate_up->n / 2, down->n,
                      qmm::moe_tile_rows(*gate_up, *down, t, topk, num_routed));
  *out = qmoe_layout{L.counts, L.offsets, L.row_of_slot, L.row_of_shared, L.token_of_row,
                     L.active, L.scalars, L.tiles, L.h, L.d, L.bytes, L.max_rows, L.max_tiles,
                     qmm::moe_uses_gemv(*gate_up, *down, t, topk, num_shared) ? 1u : 0u,
                     L.tile_rows, L.slot_of_row};
  return QMM_OK;
}

}  // extern "C"

namespace {

// Every argument check of qmoe_grouped (QMM_OK or the error it returns).
int qmoe_grouped_check(const qmm_weight *gate_up, const qmm_weight *down, int32_t num_routed,
                       int32_t num_shared, const void *x, int32_t t, const int32_t *topk_ids,
                       const float *topk_w, int32_t topk, const float *shared_w, const void *y,
                       int32_t y_dtype, const void *workspace, size_t workspace_bytes) {
  int st = check_weight(gate_up);
  if (st) return st;
  st = check_weight(down);
  if (st) return st;
  if (num_routed < 1 || num_shared < 0 || num_routed + num_shared > qmm::kMoeMaxExperts)
    return QMM_ERR_ARG;
  if (topk < 1 || topk > 64) return QMM_ERR_ARG;
  if (t < 1 || (int64_t)t * (topk + num_shared) >= (1ll << 31)) return QMM_ERR_M_RANGE;
  const int experts = num_routed + num_shared;
  if (gate_up->batch != experts || down->batch != experts) return QMM_ERR_SHAPE;
  const int inter = gate_up->n / 2;
  if (gate_up->n % 128 != 0 || down->k != inter || down->n != gate_up->k) return QMM_ERR_SHAPE;
  if (gate_up->k % 64 != 0 || down->k % 64 != 0) return QMM_ERR_SHAPE;
  if (y_dtype != QMM_F32 && y_dtype != QMM_BF16) return QMM_ERR_DTYPE;
  // the grouped form addresses x, h and the weight planes with 32-bit offsets
  if (!qmm::moe_uses_gemv(*gate_up, *down, t, topk, num_shared) &&
      !(qmm::gemm_big_fits(*gate_up, (size_t)t) &&
        qmm::gemm_big_fits(*down, (size_t)t * (size_t)(topk + num_shared))))
    return QMM_ERR_SHAPE;
  if (!x || !topk_ids || !topk_w || !y) return QMM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(topk_ids, 4) || !aligned(topk_w, 4) ||
      (shared_w && !aligned(shared_w, 4)))
    return QMM_ERR_ALIGN;
  const qmm::MoeLayout L = qmm::moe_layout(experts, t, topk, num_shared, inter, down->n,
                                           qmm::moe_tile_rows(*gate_up, *down, t, topk, num_routed));
  if (!workspace || workspace_bytes < L.bytes) return QMM_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return QMM_ERR_ALIGN;
  const int hidden = down->n;
  const Range ry = range(y, (size_t)t * hidden * (y_dtype == QMM_F32 ? 4 : 2));
  Range ins[16];
  int ni = weight_ranges(*gate_up, ins);
  ni += weight_ranges(*down, ins + ni);
  ins[ni++] = range(x, (size_t)t * gate_up->k * 2);
  ins[ni++] = range(topk_ids, (size_t)t * topk * 4);
  ins[ni++] = range(topk_w, (size_t)t * topk * 4);
  if (shared_w) ins[ni++] = range(shared_w, (size_t)t * 4);
  ins[ni++] = range(workspace, L.bytes);
  for (int i = 0; i < ni; ++i)
    if (overlap(ry, ins[i])) return QMM_ERR_ALIAS;
  const Range rw = range(workspace, L.bytes);
  for (int i = 0; i < ni - 1; ++i)
    if (overlap(rw, ins[i])) return QMM_ERR_ALIAS;
  return QMM_OK;
}

}  // namespace

extern "C" {

int qmoe_grouped(const qmm_weight *gate_up, const qmm_weight *down, int32_t num_routed,
                 int32_t num_shared, const void *x, int32_t t, const int32_t *topk_ids,
                 const float *topk_w, int32_t topk, const float *shared_w, void *y,
                 int32_t y_dtype, void *workspace, size_t workspace_bytes, void *stream) {
  const int st = qmoe_grouped_check(gate_up, down, num_routed, num_shared, x, t, topk_ids, topk_w,
                                    topk, shared_w, y, y_dtype, workspace, workspace_bytes);
  if (st) return st;
  return hip_status(qmm::launch_moe(*gate_up, *down, num_routed, num_shared, x, t, topk_ids,
                                    topk_w, topk, shared_w, y, y_dtype, workspace,
                                    (hipStream_t)stream));
}

int qmoe_grouped_noalloc(const qmm_weight *gate_up, const qmm_weight *down, int32_t num_routed,
                         int32_t num_shared, const void *x, int32_t t, const int32_t *topk_ids,
                         const float *topk_w, int32_t topk, const float *shared_w, void *y,
                         int32_t y_dtype, void *stream) {
  // the size check first: it needs no device
  const size_t need = qmoe_workspace_size(gate_up, down, num_routed, num_shared, t, topk);
  if (need > qmm::kNoallocScratchBytes) return QMM_ERR_SCRATCH;
  void *ws = nullptr;
  const hipError_t e = qmm::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e);
  const int st = qmoe_grouped_check(gate_up, down, num_routed, num_shared, x, t, topk_ids, topk_w,
                                    topk, shared_w, y, y_dtype, ws, qmm::kNoallocScratchBytes);
  if (st) return st;
  return hip_status(qmm::launch_moe(*gate_up, *down, num_routed, num_shared, x, t, topk_ids,
                                    topk_w, topk, shared_w, y, y_dtype, ws, (hipStream_t)stream));
}

int qmoe_router(const float *logits, int32_t t, int32_t num_experts, int32_t topk,
                int32_t *topk_ids, float *topk_w, void *stream) {
  if (!logits || !topk_ids || !topk_w) return QMM_ERR_NULL;
  if (num_experts < 1 || num_experts > qmm::kMoeMaxExperts) return QMM_ERR_ARG;
  if (topk < 1 || topk > 64 || topk > num_experts) return QMM_ERR_ARG;
  if (t < 1 || (int64_t)t * num_experts >= (1ll << 31)) return QMM_ERR_M_RANGE;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_w, 4)) return QMM_ERR_ALIGN;
  const Range rl = range(logits, (size_t)t * num_experts * 4);
  const Range ri = range(topk_ids, (size_t)t * topk * 4);
  const Range rw = range(topk_w, (size_t)t * topk * 4);
  if (overlap(ri, rl) || overlap(rw, rl) || overlap(ri, rw)) return QMM_ERR_ALIAS;
  return hip_status(qmm::launch_router(logits, t, num_experts, topk, topk_ids, topk_w,
                                       (hipStream_t)stream));
}

int qmoe_grouped_logits(const qmm_weight *gate_up, const qmm_weight *down, int32_t num_routed,
                        int32_t num_shared, const void *x, int32_t t, const float *logits,
                        int32_t topk, int32_t *topk_ids, float *topk_w, const float *shared_w,
                        void *y, int32_t y_dtype, void *workspace, size_t workspace_bytes,
                        void *stream) {
  // every check of both calls before either launches
  if (!logits) return QMM_ERR_NULL;
  int st = qmoe_grouped_check(gate_up, down, num_routed, num_shared, x, t, topk_ids, topk_w, topk,
                              shared_w, y, y_dtype, workspace, workspace_bytes);
  if (st) return st;
  if (topk > num_routed) return QMM_ERR_ARG;
  if (!aligned(logits, 4)) return QMM_ERR_ALIGN;
  const Range rl = range(logits, (size_t)t * num_routed * 4);
  const Range ri = range(topk_ids, (size_t)t * topk * 4);
  const Range rw = range(topk_w, (size_t)t * topk * 4);
  const Range ry = range(y, (size_t)t * down->n * (y_dtype == QMM_F32 ? 4 : 2));
  const Range rs = range(workspace, workspace_bytes);
  if (overlap(ri, rl) || overlap(rw, rl) || overlap(ri, rw) || overlap(ry, rl) || overlap(rs, rl))
    return QMM_ERR_ALIAS;
  // the router's outputs must not land on the layer's other inputs
  Range ins[16];
  int ni = weight_ranges(*gate_up, ins);
  ni += weight_ranges(*down, ins + ni);
  ins[ni++] = range(x, (size_t)t * gate_up->k * 2);
  if (shared_w) ins[ni++] = range(shared_w, (size_t)t * 4);
  for (int i = 0; i < ni; ++i)
    if (overlap(ri, ins[i]) || overlap(rw, ins[i])) return QMM_ERR_ALIAS;
  return hip_status(qmm::launch_moe_logits(*gate_up, *down, num_routed, num_shared, x, t, logits,
                                           topk_ids, topk_w, topk, shared_w, y, y_dtype, workspace,
                                           (hipStream_t)stream));
}

}  // extern "C"
