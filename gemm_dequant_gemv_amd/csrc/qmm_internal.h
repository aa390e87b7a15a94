// Internal interface between the C-ABI layer (abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qmm.h"

namespace qmm {

// Decode-GEMV tiling: a workgroup of 4 waves covers 32 * R rows; inside a
// wave, 8 lanes share a row (each reading 16 consecutive bytes of codes = 32
// weights, so the 8 lanes read 128 contiguous bytes) and every lane carries R
// rows.  One K step is therefore 8 x 32 = 256 weights; D steps are kept in
// flight.  K is split over `splits` workgroups when the rows alone do not give
// enough workgroups.
constexpr int kGemvThreads = 256;
constexpr int kGemvStep = 256;      // K values per step (8 lanes x 32)
constexpr int kMaxSplitK = 2048;    // K values one workgroup covers at most

struct GemvPlan {
  int kind;           // 0: split-K kernel, 1: row-streaming kernel
  int rows_per_lane;  // R (row-streaming: rows per batch)
  int depth;          // D: steps (row-streaming: units) of weights in flight per lane
  int early;          // split-K: code loads issued before waiting for activations and scales
  int balanced;       // row-streaming split: 0 round-robin pairs, 1 each workgroup's units split
                      // evenly over its waves
  int lanes_k;        // lanes sharing a row (each reads 16 bytes per step)
  int steps;      // steps per row
  int tiles;      // split-K: ceil(n / rows per workgroup); row-streaming: workgroups
  int splits;     // K splits (workgroups per row tile)
  int max_steps;  // steps of the longest split
  size_t lds_bytes;
  size_t ws_bytes;        // workspace needed (0 when splits == 1)
  size_t counters_bytes;  // leading part of the workspace: one u32 per tile
};

GemvPlan plan_gemv(int format, int n, int k, int m);
// the row-streaming kernel's activation rows at most (qgemv takes 1 to 4;
// qgemm sends it calls of 5 up to this many rows)
constexpr int kRowsMaxM = 8;
bool plan_gemv_rows(int format, int n, int k, int m, GemvPlan &p);

// rows per tile of the MoE routing table (the grouped GEMMs' activation tiles)
constexpr int kMoeTileRows = 256;  // routing tile rows at most (the grouped GEMMs' tallest X tile)
// Experts (routed + shared) one MoE call may have.
constexpr int kMoeMaxExperts = 4096;

// Device tables of one MoE call, carved from the caller's workspace.
struct MoeTables {
  uint32_t *counts;         // [experts] grouped rows per expert
  uint32_t *offsets;        // [experts + 1] first grouped row of each expert
  uint32_t *row_of_slot;    // [t][topk] grouped row of each routed slot
  uint32_t *row_of_shared;  // [shared][t] grouped row of each shared slot
  uint32_t *token_of_row;   // [rows] token each grouped row reads
  uint32_t *slot_of_row;    // [rows] token slot of each grouped row (its row of d)
  uint32_t *active;         // [experts] experts with rows, in expert order
  uint32_t *n_active, *n_tiles, *err;
  uint32_t *tiles;          // [max_tiles][3] (expert, first row, rows)
  uint16_t *h;              // bf16 [rows][inter]
  float *d;                 // float32 [rows][hidden]
  uint32_t *wg_counts;      // parallel route: [groups][experts] rows per workgroup, then
                            // each workgroup's first position in the expert's group
  uint32_t *wg_err;         // parallel route: [groups] dropped ids seen
  int route_groups;         // 1: the one-workgroup route; else workgroups of the parallel one
};

struct MoeLayout {
  size_t counts, offsets, row_of_slot, row_of_shared, token_of_row, active, scalars, tiles, h, d;
  size_t slot_of_row;
  size_t wg_counts, wg_err, route_groups;
  size_t bytes, max_rows, max_tiles, tile_rows;
};

MoeLayout moe_layout(int num_experts, int t, int topk, int num_shared, int inter, int hidden,
                     int tile_rows);
// rows per routing tile of the grouped form: 32 .. kMoeTileRows
int moe_tile_rows(const qmm_weight &gu, const qmm_weight &dn, int t, int topk, int num_routed);
MoeTables moe_tables(const MoeLayout &L, void *ws);

hipError_t launch_dequant(const qmm_weight &w, int out_dtype, void *out, hipStream_t s);
hipError_t launch_gemv_rows(const qmm_weight &w, const void *x, int m, const void *residual,
                            void *y, int y_dtype, const GemvPlan &p, hipStream_t s);
// qgemm's 5 to kRowsMaxM rows on the row-streaming kernel (weights read and
// decoded once), bf16 y; false when the activations do not fit in LDS (the
// call then takes the MFMA tiles)
bool gemm_rows_fits(const qmm_weight &w, int m);
hipError_t launch_gemm_rows(const qmm_weight &w, const void *x, int m, const void *residual,
                            void *y, hipStream_t s);
hipError_t launch_gemv(const qmm_weight &w, const void *x, int m, const void *residual,
                       void *y, int y_dtype, void *workspace, const GemvPlan &p,
                       hipStream_t s);
hipError_t launch_gemm_big(const qmm_weight &w, const void *x, int m, const void *residual,
                           void *y, void *workspace, size_t workspace_bytes, hipStream_t s);
// workspace that lets a dense call of m rows split K (0: it never splits)
size_t gemm_big_workspace(const qmm_weight &w, int m);
// compute units of the current device (cached per device; 256 if the query fails)
long compute_units();
// the 256-row-tile kernels (gemm_big.hip) address X (x_rows rows) and the
// weight planes with 32-bit offsets
bool gemm_big_fits(const qmm_weight &w, size_t x_rows);
hipError_t launch_moe_big_gate_up(const qmm_weight &gu, const void *x, const MoeTables &t,
                                  int max_tiles, int tile_rows, hipStream_t s);
hipError_t launch_moe_big_down(const qmm_weight &dn, const MoeTables &t, int max_tiles,
                               int tile_rows, hipStream_t s);
size_t gemm_workspace_size(const qmm_weight &w, int m);
// decode form of qmoe_grouped: grouped GEMV over token slots (t <= 16 and
// at most kMoeGemvMaxSlots slots, when the staged vectors fit in LDS)
constexpr int kMoeGemvMaxTokens = 16;
constexpr int kMoeGemvMaxSlots = 128;  // token slots of the decode form (register table)
bool moe_gemv_fits(const qmm_weight &gu, const qmm_weight &dn, int t, int topk, int num_shared);
bool moe_uses_gemv(const qmm_weight &gu, const qmm_weight &dn, int t, int topk, int num_shared);
// logits non-null: the router runs inside the gate/up launch (num_routed <=
// 512, moe_router_folds) and writes the routing to ids_out / w_out, which
// the down launch reads (topk_ids / topk_w are then ignored)
bool moe_router_folds(int num_routed);
hipError_t launch_moe_gemv(const qmm_weight &gu, const qmm_weight &dn, int num_routed,
                           int num_shared, const void *x, int t, const int32_t *topk_ids,
                           const float *topk_w, int topk, const float *shared_w, void *y,
                           int y_bf16, const MoeTables &tb, hipStream_t s,
                           const float *logits = nullptr, int32_t *ids_out = nullptr,
                           float *w_out = nullptr);
hipError_t launch_moe(const qmm_weight &gu, const qmm_weight &dn, int num_routed, int num_shared,
                      const void *x, int t, const int32_t *topk_ids, const float *topk_w,
                      int topk, const float *shared_w, void *y, int y_dtype, void *workspace,
                      hipStream_t s);
// qmoe_grouped from router logits: the router folded into the decode form's
// first launch where it can be, else its own launch ahead of the layer
hipError_t launch_moe_logits(const qmm_weight &gu, const qmm_weight &dn, int num_routed,
                             int num_shared, const void *x, int t, const float *logits,
                             int32_t *topk_ids, float *topk_w, int topk, const float *shared_w,
                             void *y, int y_dtype, void *workspace, hipStream_t s);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);
// EXL3 rotation stages (hadamard.hip): prepare (bf16 in and out) or finish
// (float32 in, float32 or bf16 out), per 128-value block
hipError_t launch_hadamard(bool prepare, const void *in, int rows, int len, const void *scale,
                           void *out, int out_bf16, hipStream_t s);
// W4A4 (w4a4.hip): MXFP4 activation quantizer and the FP4 x FP4 GEMM; the
// workspace holds the quantized activations (codes, then E8M0 scales)
size_t w4a4_workspace_size(int m, int k);
bool w4a4_fits(const qmm_weight &w, int m);
hipError_t launch_quant_mxfp4(const void *x, int m, int k, void *codes, void *scales,
                              hipStream_t s);
hipError_t launch_gemm_w4a4(const qmm_weight &w, const void *x, int m, const void *residual,
                            void *y, void *workspace, hipStream_t s);
// the static scratch of qmoe_grouped_noalloc (noalloc.hip): its size, and the
// device address of the current device's copy (looked up once per device)
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
hipError_t noalloc_scratch(void **out);
// router top-k + softmax: one wave per token (router.hip)
hipError_t launch_router(const float *logits, int t, int e, int k, int32_t *ids, float *w,
                         hipStream_t s);
hipError_t launch_mfma_peak(int iters, float *sink, int blocks, hipStream_t s);
double mfma_peak_flops(int iters, int blocks);
hipError_t launch_stream_read(const void *p, size_t bytes, uint32_t *sink, int blocks,
                              hipStream_t s);

}  // namespace qmm
