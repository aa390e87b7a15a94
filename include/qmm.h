/*
 * qmm.h -- C ABI of libqmm: matrix multiplies whose weights are block-quantized
 * low-bit codes, dequantized inside the kernels against bfloat16 activations
 * (weights 4 or 6 bits, activations 16 bits), for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the pages call a W4A16 projection: every weight is
 * expanded to 16 bits inside the kernel and multiplied at 16-bit precision with
 * 32-bit accumulation, so that only the weights are approximated ("TurboEXL3",
 * section 2.2, W4A16 bullet).  Formats ("TurboEXL3", section 2.1; splash PR #19,
 * "What changed"):
 *
 *   QMM_AFFINE4_G64  4-bit unsigned codes q, one float16 scale s and one float16
 *                    bias b per 64 weights: w = s*q + b           (4.5 bits/weight)
 *   QMM_MXFP4        E2M1 codes, one E8M0 power-of-two scale E per 32 weights:
 *                    w = e2m1(c) * 2^(E-127)                      (4.25 bits/weight)
 *   QMM_NVFP4        E2M1 codes, one E4M3 scale S per 16 weights, one float32
 *                    multiplier g per tensor: w = e2m1(c)*e4m3(S)*g (4.5 bits/weight)
 *   QMM_Q6_K         6-bit codes q (4 low bits + 2 high bits), one int8 scale sc
 *                    per 16 weights, one float16 scale d per 256 weights:
 *                    w = d*sc*(q-32)                              (6.5625 bits/weight)
 *
 * E2M1: sign in bit 3, magnitude index in bits 0-2 into 0, 0.5, 1, 1.5, 2, 3, 4, 6
 * (code 8 is -0).  E8M0: 2^(e-127), 0xFF is NaN.  E4M3: bias 7 with subnormals,
 * largest finite 448, S.1111.111 is NaN.
 *
 * ----------------------------------------------------------------------------
 * Conventions for every entry point
 *
 * Matrices.  W is N x K (N outputs, K inputs), row-major; quantization blocks run
 * along K inside a row.  Activations X are M x K bfloat16, row-major; outputs are
 * M x N, row-major ("y[m][n] = sum_k w[n][k] * x[m][k]").  K must be a multiple
 * of the format's K granule, so that every row of codes starts on a 16-byte
 * boundary and every row of scales on a 4-byte boundary: 64 for AFFINE4_G64 and
 * NVFP4, 128 for MXFP4, 256 for Q6_K.  Each plane of a weight must be smaller
 * than 4 GiB (32-bit byte offsets).
 *
 * Pointers.  Every pointer is a device pointer unless stated otherwise; the
 * descriptor structs themselves live in host memory and are read before the call
 * returns.  The caller owns every buffer.  The library never allocates, frees or
 * synchronizes on a call path.  Codes, x and qdequant's output must be 16-byte
 * aligned, codes_hi 8-byte, scales 4-byte, scales2 2-byte; y and residual need
 * their element alignment.  Outputs may not alias any input.
 *
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null stream).
 * Every call is asynchronous on that stream; a kernel fault surfaces at the
 * caller's next synchronization.
 *
 * Errors.  Every entry point returns QMM_OK (0) or a negative QMM_ERR_* code.
 * Arguments are validated on the host before anything is launched; on an error
 * nothing is launched and nothing is written.  QMM_ERR_HIP means a HIP runtime
 * call failed; qlast_hip_error() then returns its hipError_t (thread-local).
 * Not checked (would need a device synchronization): expert ids in range, finite
 * scales.  No C++ exception crosses this interface.
 *
 * Workspaces.  Calls that split a reduction across workgroups take a caller-
 * owned workspace of at least *_workspace_size() bytes, 256-byte aligned.  Its
 * contents on entry do not matter and it needs no zero-fill: a call that uses
 * it writes everything it later reads, and the arrival counters of a split
 * reduction are cleared by a small kernel of the call's own, on its stream,
 * before the split launch.  One workspace serves one call at a time: calls
 * that may overlap (other streams) need their own.
 *
 * Determinism.  Every sum runs in a fixed order and no floating-point atomics
 * are used, so the same inputs give bitwise identical outputs on every run
 * ("TurboEXL3", section 4.4, Numerics).
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum qmm_format { QMM_AFFINE4_G64 = 1, QMM_MXFP4 = 2, QMM_NVFP4 = 3, QMM_Q6_K = 4 };
enum qmm_dtype { QMM_F32 = 0, QMM_BF16 = 1 };

enum qmm_status {
  QMM_OK = 0,
  QMM_ERR_NULL = -1,      /* a required pointer is NULL                        */
  QMM_ERR_FORMAT = -2,    /* unknown format or a plane that the format lacks    */
  QMM_ERR_SHAPE = -3,     /* n, k or batch out of range or not block-aligned    */
  QMM_ERR_ALIGN = -4,     /* a pointer is not aligned as required               */
  QMM_ERR_M_RANGE = -5,   /* m (rows of x) out of range for the call            */
  QMM_ERR_WORKSPACE = -6, /* workspace missing or smaller than *_workspace_size */
  QMM_ERR_ALIAS = -7,     /* an output overlaps an input                        */
  QMM_ERR_HIP = -8,       /* a HIP runtime call failed (see qlast_hip_error)    */
  QMM_ERR_DTYPE = -9,     /* unknown output dtype                               */
  QMM_ERR_ARG = -10,      /* another argument out of range (topk, experts ...)  */
  QMM_ERR_SCRATCH = -11   /* the call needs more than qmoe_grouped_noalloc's
                             static scratch holds                              */
};

/*
 * One N x K packed weight matrix, or a batch of `batch` of them with the same
 * shape stored back to back (the experts of an MoE layer).  Planes, for matrix
 * e of the batch ("[batch]" is the outermost index of every plane):
 *
 *   codes     u8 [batch][n][k/2]  4-bit codes; element k = 2j in bits 0-3 of
 *                                 byte j, element 2j+1 in bits 4-7.  For Q6_K the
 *                                 low 4 bits of each 6-bit code.
 *   codes_hi  u8 [batch][n][k/4]  Q6_K only: the 2 high bits; element k = 4j+i in
 *                                 bits 2i..2i+1 of byte j.  NULL otherwise.
 *   scales    AFFINE4_G64: f16 [batch][n][k/64][2], pairs (scale s, bias b)
 *             MXFP4:       u8  [batch][n][k/32], E8M0
 *             NVFP4:       u8  [batch][n][k/16], E4M3
 *             Q6_K:        i8  [batch][n][k/16], sub-block scale sc
 *   scales2   Q6_K: f16 [batch][n][k/256], super-block scale d.  NULL otherwise.
 *   tensor_scale  NVFP4: f32 [batch] (device), multiplier g of each matrix.
 *                 NULL otherwise.
 */
typedef struct qmm_weight {
  int32_t format; /* enum qmm_format                        */
  int32_t n;      /* rows (outputs), >= 1                   */
  int32_t k;      /* columns (inputs), multiple of the K granule */
  int32_t batch;  /* matrices stored back to back, >= 1     */
  const void *codes;
  const void *codes_hi;
  const void *scales;
  const void *scales2;
  const float *tensor_scale;
} qmm_weight;

/*
 * qdequant -- expand every weight of every matrix of `w` to out[batch][n][k]
 * ("TurboEXL3", section 4.3: past the GEMM paths' row counts the weights are
 * decoded to 16 bits and handed to a plain matrix multiply; section 2.1 for
 * each format's dequantization).
 * out_dtype QMM_F32: the exact weight rounded once to nearest float32; for
 * AFFINE4_G64 that is fma(s, q, b), for NVFP4 (e2m1*e4m3)*g; MXFP4 and Q6_K are
 * exact.  QMM_BF16: that float32 rounded to nearest-even bfloat16.
 * out  device, 16-byte aligned, batch*n*k elements of 4 (F32) or 2 (BF16)
 *      bytes; must not overlap the weight planes (QMM_ERR_ALIAS).
 * Used for bit-exact checks of the decoders and as a decode-then-multiply
 * building block.  No workspace.
 */
int qdequant(const qmm_weight *w, int32_t out_dtype, void *out, void *stream);

/*
 * qgemv -- decode matrix-vector product for 1 to 4 activation rows
 * ("TurboEXL3", section 4.3: one GEMV launch for 1 to 4 rows, whose output
 * blocks are finished by the workgroup that arrives last; section 4.2: split-K
 * partial sums keep enough workgroups in flight; splash PR #19: lanes 1-4 and
 * the "+res" projections).
 *
 *   y[m][n] = g * sum_k w[n][k] * x[m][k]  (+ residual[m][n])     0 <= m < M
 *
 * w         one matrix (batch must be 1)
 * x         bf16 [m][k]
 * m         1..4
 * residual  bf16 [m][n] or NULL (added in float32 after the sum)
 * y         [m][n], float32 (y_dtype QMM_F32) or bfloat16 rounded to nearest
 *           even (QMM_BF16)
 * workspace at least qgemv_workspace_size(w, m) bytes (may be NULL when that is 0)
 */
size_t qgemv_workspace_size(const qmm_weight *w, int32_t m);
int qgemv(const qmm_weight *w, const void *x, int32_t m, const void *residual,
          void *y, int32_t y_dtype, void *workspace, size_t workspace_bytes,
          void *stream);

/*
 * qbench_stream_read -- measurement helper: read `bytes` (multiple of 16) of
 * `buf` with 16-byte non-temporal loads, the access pattern of the weight
 * stream, on `blocks` workgroups of 256 threads.  Writes at most 4 bytes to
 * `sink` (device).  Timing it gives the achievable HBM read bandwidth that the
 * GEMV figures are compared with (the Conifer note likewise measures its own
 * peak with a triad microbenchmark instead of trusting the nominal figure).
 */
int qbench_stream_read(const void *buf, size_t bytes, void *sink, int32_t blocks, void *stream);

/*
 * qbench_mfma_peak -- measurement helper: `blocks` workgroups of 4 waves, each
 * wave issuing `iters` (1 .. 2^24, rounded up to a multiple of 4) rounds of 4
 * independent v_mfma_f32_32x32x16_bf16 on random register operands, the
 * instruction of the prefill GEMM.  Stores the launch's floating-point operation count in *flops
 * (host, may be NULL) and writes at most 4 bytes to `sink` (device).  Timing it
 * gives the achievable dense bf16 matrix rate that the GEMM figures are
 * compared with, beside the nominal 2.5 PFLOP/s.
 */
int qbench_mfma_peak(int32_t iters, int32_t blocks, void *sink, double *flops, void *stream);

/*
 * qgemm -- prefill matrix multiply for many activation rows ("TurboEXL3",
 * section 4.1, decode once, multiply many times: each K-slice of the weights is
 * decoded once per workgroup into on-chip memory as 16-bit values and multiplied
 * against a tile of activations with 32-bit accumulation; the decoded weights
 * never reach device memory).
 *
 *   y[m][n] = bf16( g * sum_k w16[n][k] * x[m][k]  (+ residual[m][n]) )
 *
 * where w16 is the weight rounded to bfloat16 (exact for MXFP4 and NVFP4;
 * affine and Q6_K values are rounded to nearest even, a relative error of at
 * most 2^-9 per weight), summed in float32 on the matrix cores.  Calls of 5 to
 * 8 rows whose activations fit in LDS (k * m * 2 bytes plus block sums, about
 * k <= 8192 at 8 rows) take the decode GEMV's row-streaming kernel instead
 * ("TurboEXL3" section 4.3: 5 to 16 rows decode each weight once per chunk of
 * up to 8 rows), which multiplies with the exact weights; fewer than 5 rows
 * and the rest take the MFMA tiles.
 *
 * w         one matrix (batch must be 1); k must be a multiple of 64; fewer
 *           than 2^32 weights (QMM_ERR_SHAPE otherwise)
 * x         bf16 [m][k], m >= 1 (tuned for m >= 128); m * k * 2 < 4 GiB
 *           (QMM_ERR_SHAPE otherwise: x is addressed with 32-bit offsets)
 * residual  bf16 [m][n] or NULL
 * y         bf16 [m][n], rounded to nearest even
 * x, y and residual must be 16-byte aligned.
 * workspace  optional.  For calls of up to 32 rows, and of up to 256 rows
 *            where the weight has few row blocks and a long K (e.g. 5120 x
 *            17408), qgemm_workspace_size returns the bytes (256-byte
 *            aligned, any contents) with which the call splits K over several
 *            workgroups: each writes float32 partial sums and the last of a
 *            tile's workgroups adds them in split order (a fixed order, so
 *            results are the same on every run; they differ from an unsplit
 *            call's only in summation order).  With a NULL or smaller
 *            workspace the call runs unsplit.  Otherwise it returns 0.
 */
size_t qgemm_workspace_size(const qmm_weight *w, int32_t m);
int qgemm(const qmm_weight *w, const void *x, int32_t m, const void *residual, void *y,
          void *workspace, size_t workspace_bytes, void *stream);

/*
 * qmoe_grouped -- one mixture-of-experts layer: routed experts chosen per token
 * plus shared experts that every token visits ("TurboEXL3" section 4.1 and 4.2:
 * route, gate and up in one multiply, SwiGLU in 32-bit, down, and the
 * score-weighted sum of each token's expert outputs; tokens that chose the
 * same expert share one decode of its weights).
 *
 *   h_e(x)  = bf16( silu(g) * u ),  [g; u] = W_gu[e] x   (gate rows 0..I-1, up rows I..2I-1)
 *   d_e(x)  = W_d[e] h_e(x)                                (float32)
 *   y[t]    = sum_j topk_w[t][j] * d_{topk_ids[t][j]}(x[t])
 *             + sum_s shared_w[t] * d_{E+s}(x[t])          (fixed order: j, then s)
 *
 * gate_up      batch = E + S matrices of 2I x H (routed experts 0..E-1, then the
 *              S shared experts); 2I a multiple of 128
 * down         batch = E + S matrices of H x I
 * num_routed   E >= 1;  num_shared  S >= 0;  E + S <= 4096
 * x            bf16 [t][H]
 * topk_ids     int32 [t][topk], each in [0, E); a slot with an id outside that
 *              range contributes nothing (it is never read out of bounds)
 * topk_w       float32 [t][topk]
 * shared_w     float32 [t] or NULL (weight 1 for every shared expert)
 * y            [t][H], float32 (QMM_F32) or bf16 rounded to nearest even (QMM_BF16)
 * workspace    at least qmoe_workspace_size(...) bytes, 256-byte aligned; it holds
 *              the routing tables, h and d.  No zero-fill is needed.
 * The grouped form addresses x, h and the weight planes with 32-bit offsets:
 * t * H * 2 and t * (topk + S) * I * 2 must stay below 4 GiB and each weight
 * below 2^32 elements (QMM_ERR_SHAPE otherwise).
 * The gate/up and down weights may use different formats.
 *
 * Two forms, the same result contract: up to 16 tokens with at most 128 token
 * slots (t * (topk + S)), when the activations
 * fit in LDS) take the decode form, one grouped matrix-vector launch per
 * projection over the token slots, the second also running the combine
 * ("TurboEXL3" section 3.1: decode verifies 1 to 4 tokens; more here, where
 * one pass per token slot still costs less than the grouped form's mostly
 * empty tiles); more tokens take the grouped-GEMM form
 * (route, gate/up, down, combine; section 4.1).  qmoe_workspace_layout says
 * which form a call takes.
 */
/*
 * qhadamard_prepare / qhadamard_finish -- the rotation stages that surround
 * an EXL3 projection's inner product ("TurboEXL3", section 3.1: prepare
 * scales the input by the input-channel vector and applies the Hadamard
 * transform one 128-element block at a time; finish applies the transform to
 * the output, then scales it by the output-channel vector; section 2.3: the
 * transforms are sign-randomized Hadamard transforms in blocks of 128, and
 * the two 16-bit channel vectors are a matrix's only scales).
 *
 *   prepare: out[m][j] = bf16( sum_i H[j%128][i] * s_in[b+i] * x[m][b+i] )
 *   finish:  out[m][j] = s_out[j] * sum_i H[j%128][i] * y[m][b+i]
 *            (b = 128 * (j / 128): the block of j)
 *
 * H is the orthonormal 128-point Hadamard matrix H_128 / sqrt(128), H_128 in
 * Sylvester's order (entry (i, j) = (-1)^popcount(i & j)); the pages do not
 * say where the random signs are kept: here they are the sign bits of the
 * float16 channel scales.  Sums are float32.
 *
 * x          bf16 [m][k]; y float32 [m][n]; k and n multiples of 128
 * in_scale, out_scale  float16 [k] or [n], or NULL (all ones)
 * out        prepare: bf16 [m][k]; finish: [m][n] float32 (out_dtype QMM_F32)
 *            or bf16 rounded to nearest even (QMM_BF16); must not overlap
 *            the input or the scale (QMM_ERR_ALIAS)
 * Element alignment for every pointer.  No workspace.
 */
int qhadamard_prepare(const void *x, int32_t m, int32_t k, const void *in_scale, void *out,
                      void *stream);
int qhadamard_finish(const float *y, int32_t m, int32_t n, const void *out_scale, void *out,
                     int32_t out_dtype, void *stream);

/*
 * qgemv_hadamard -- one EXL3-style projection at decode in one call: the
 * prepare stage, the matrix-vector product and the finish stage ("TurboEXL3",
 * section 3.1: the prepare and finish stages around the inner product;
 * section 2.3: 128-block sign-randomized Hadamard transforms and the two
 * channel vectors):
 *
 *   y = finish( W . prepare(x) )      (prepare and finish as above)
 *
 * Three launches on the stream, bitwise the result of qhadamard_prepare,
 * qgemv and qhadamard_finish in sequence.  (Prepare was also built into the
 * row-streaming GEMV's prologue, transforming the staged activations in LDS:
 * every workgroup then repeats the whole transform of x, and it measured
 * 0.7-25 us slower than the separate launch on the decode shapes, so the
 * separate launch stays.)
 *
 * w          one matrix (batch 1) in any format; n and k multiples of 128
 * x          bf16 [m][k], m = 1..4 (raw activations: prepare is applied here)
 * in_scale, out_scale  float16 [k] / [n] or NULL (all ones)
 * y          [m][n] float32 (QMM_F32) or bf16 (QMM_BF16)
 * workspace  qgemv_hadamard_workspace_size bytes, 256-byte aligned, never
 *            NULL: the prepared activations, the float32 product when y is
 *            bf16 (a float32 y takes it, and finish runs in place), then
 *            qgemv's split-K workspace if the call needs one; no zero-fill
 * Nothing may overlap y or the workspace (QMM_ERR_ALIAS).
 */
size_t qgemv_hadamard_workspace_size(const qmm_weight *w, int32_t m, int32_t y_dtype);
int qgemv_hadamard(const qmm_weight *w, const void *x, int32_t m, const void *in_scale,
                   const void *out_scale, void *y, int32_t y_dtype, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * qquant_mxfp4 -- quantize bfloat16 activations to MXFP4 on the GPU, the
 * activation half of W4A4 ("TurboEXL3", section 2.2, W4A4 bullet: the
 * activations are quantized to a 4-bit block format on the fly; section 2.1,
 * MXFP4: E2M1 values with one E8M0 power-of-two scale per 32).  Per row of x
 * and block of 32 values along K: E = floor(log2 amax) - 2 (the largest E2M1
 * magnitude is 1.5 * 2^2), stored as E8M0 = max(E + 127, 0); each value is
 * divided by 2^(E8M0 - 127) and rounded to the nearest E2M1 value, ties to
 * the even code, past 6 saturating to 6; a value that rounds to zero gets
 * code 0; an all-zero block gets E8M0 0 and zero codes.
 *
 * x       bf16 [m][k], finite values, 16-byte aligned; k a multiple of 32
 * codes   u8 [m][k/2] (out), element 2j in the low nibble of byte j, 16-byte
 *         aligned
 * scales  u8 [m][k/32] (out), E8M0
 * The outputs must not overlap x or each other (QMM_ERR_ALIAS).
 */
int qquant_mxfp4(const void *x, int32_t m, int32_t k, void *codes, void *scales, void *stream);

/*
 * qgemm_w4a4 -- W4A4 matrix multiply: MXFP4 weights times activations
 * quantized to MXFP4 on the fly (qquant_mxfp4, into the workspace), both
 * operands multiplied as FP4 on the block-scaled matrix cores with float32
 * sums ("TurboEXL3", section 2.2, W4A4 bullet).  The result differs from the
 * W4A16 qgemm by design: every activation is rounded to 4 bits.
 *
 *   y[m][n] = bf16( sum_k w[n][k] * q(x)[m][k]  (+ residual[m][n]) )
 *
 * w          one MXFP4 matrix (QMM_ERR_FORMAT otherwise), batch 1
 * x          bf16 [m][k], m >= 1, finite; residual bf16 [m][n] or NULL
 * y          bf16 [m][n], rounded to nearest even
 * x, y and residual 16-byte aligned; m * k / 2 and n * k / 2 below 4 GiB
 * workspace  at least qgemm_w4a4_workspace_size(w, m) bytes, 256-byte
 *            aligned, any contents: the quantized activations (codes, then
 *            E8M0 scales at the next 256-byte boundary)
 * Two launches on the stream (quantizer, GEMM).  The products are exact;
 * sums run in a fixed order, so results are the same on every run.
 */
size_t qgemm_w4a4_workspace_size(const qmm_weight *w, int32_t m);
int qgemm_w4a4(const qmm_weight *w, const void *x, int32_t m, const void *residual, void *y,
               void *workspace, size_t workspace_bytes, void *stream);

size_t qmoe_workspace_size(const qmm_weight *gate_up, const qmm_weight *down, int32_t num_routed,
                           int32_t num_shared, int32_t t, int32_t topk);
int qmoe_grouped(const qmm_weight *gate_up, const qmm_weight *down, int32_t num_routed,
                 int32_t num_shared, const void *x, int32_t t, const int32_t *topk_ids,
                 const float *topk_w, int32_t topk, const float *shared_w, void *y,
                 int32_t y_dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * qmoe_grouped_noalloc -- qmoe_grouped for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, result and kernels as qmoe_grouped
 * (bit-identical output), but no workspace argument: the routing tables, h
 * and d go to a static device buffer of 16 MiB that the library holds on each
 * GPU it runs on until the process ends.  The call allocates nothing.
 *
 * Size limit: calls whose qmoe_workspace_size(...) exceeds 16 MiB return
 * QMM_ERR_SCRATCH before anything is checked further or launched (on the
 * 512 + 1-expert layer, hidden 2048, intermediate 512, top-10: up to about
 * 160 tokens).
 * Concurrency: every call on one GPU uses that GPU's single buffer, so calls
 * that may overlap on one GPU (different streams, or different host threads
 * without ordering) race on it and give undefined results; serialize them.
 * The buffer keeps the last call's contents; the call needs no particular
 * contents on entry.
 * The first call on each device looks up that device's buffer address
 * (hipGetSymbolAddress) with the device current; a failure there returns
 * QMM_ERR_HIP.
 */
int qmoe_grouped_noalloc(const qmm_weight *gate_up, const qmm_weight *down, int32_t num_routed,
                         int32_t num_shared, const void *x, int32_t t, const int32_t *topk_ids,
                         const float *topk_w, int32_t topk, const float *shared_w, void *y,
                         int32_t y_dtype, void *stream);

/*
 * qmoe_router -- the router's top-k and softmax ("TurboEXL3" section 4.2: in
 * the decode chain the router's top-k and softmax run on the GPU, in the
 * layer's first launch; the model routes each token to 10 of 512 experts).
 *
 *   topk_ids[t][0..k-1] = the k experts with the largest logits[t][*], in
 *                         descending logit order; equal logits go to the lower
 *                         expert id, and -0 equals +0
 *   topk_w[t][r]        = exp(l_r - l_0) / sum_{j<k} exp(l_j - l_0) in float32
 *                         (l_r the logit of topk_ids[t][r]; the sum runs in a
 *                         fixed order, so the same logits give the same bits)
 *
 * logits       float32 [t][num_experts], finite (a NaN gets an unspecified but
 *              repeatable place in the order)
 * num_experts  1 .. 4096;  topk  1 .. min(64, num_experts);  t >= 1
 * topk_ids     int32 [t][topk] (out);  topk_w  float32 [t][topk] (out)
 * All pointers 4-byte aligned; the outputs must not overlap the logits or each
 * other (QMM_ERR_ALIAS).  No workspace.
 */
int qmoe_router(const float *logits, int32_t t, int32_t num_experts, int32_t topk,
                int32_t *topk_ids, float *topk_w, void *stream);

/*
 * qmoe_grouped_logits -- qmoe_grouped from router logits: qmoe_router over the
 * num_routed routed experts into topk_ids / topk_w (outputs, also kept for the
 * caller), then qmoe_grouped with them, on one stream.  The result is
 * bit-identical to calling the two in sequence.  Every argument check of both
 * calls runs before anything is launched; in addition the router's outputs
 * must not overlap the logits, x, the weights, shared_w, y or the workspace
 * (QMM_ERR_ALIAS).  The workspace is qmoe_workspace_size(...) bytes as for
 * qmoe_grouped.  In the decode form with up to 512 routed experts the
 * router runs inside the layer's first launch (every workgroup routes the
 * tokens itself; "TurboEXL3" section 4.2); otherwise it is its own launch ahead
 * of the layer's.
 */
int qmoe_grouped_logits(const qmm_weight *gate_up, const qmm_weight *down, int32_t num_routed,
                        int32_t num_shared, const void *x, int32_t t, const float *logits,
                        int32_t topk, int32_t *topk_ids, float *topk_w, const float *shared_w,
                        void *y, int32_t y_dtype, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * Where a qmoe_grouped call with these arguments keeps its intermediates inside
 * the workspace, for inspection after the call.  Byte offsets from the
 * workspace start; rows = t * (topk + S) grouped rows (slots sorted by expert).
 */
typedef struct {
  size_t counts;        /* uint32 [E+S]     rows of each expert                       */
  size_t offsets;       /* uint32 [E+S+1]   first grouped row of each expert; last =
                           number of valid rows                                     */
  size_t row_of_slot;   /* uint32 [t][topk] grouped row of each routed slot, or
                           0xFFFFFFFF for an expert id outside [0, E)               */
  size_t row_of_shared; /* uint32 [S][t]    grouped row of each shared-expert slot   */
  size_t token_of_row;  /* uint32 [rows]    token each grouped row reads              */
  size_t active;        /* uint32 [n_active] experts with at least one row, ascending */
  size_t scalars;       /* uint32 [3]       n_active, n_tiles, err (1 = an id was
                           outside [0, E) and its slot was dropped)                 */
  size_t tiles;         /* uint32 [n_tiles][3] expert, first grouped row, rows
                           (<= tile_rows) of each row tile, experts ascending       */
  size_t h;             /* bf16  [rows][I]  SwiGLU outputs, by grouped row (grouped
                           form) or token slot (decode form)                        */
  size_t d;             /* float [rows][H]  down-projection outputs by token slot, in
                           both forms: routed slot (i, j) of token i at row
                           i * topk + j, shared expert s's slot of token i at
                           t * topk + s * t + i                                     */
  size_t bytes;         /* = qmoe_workspace_size                                     */
  size_t max_rows, max_tiles;
  size_t slot_rows;     /* 1: the call takes the decode form (t <= 16, t * (topk + S)
                           <= 128 and the
                           vectors fit in LDS): no routing pass; h and d row s is
                           token slot s (routed slots in list order, then shared
                           expert j's slot of token i at t*topk + j*t + i); of the
                           tables only scalars[2] (err) is written.
                           0: the grouped form; every table above is written.   */
  size_t tile_rows;     /* rows per routing tile of the grouped form: the smallest
                           of 32, 64, 128, 192, 256 that holds 1.2 times an
                           average routed expert's rows (t * topk / E), so that
                           most experts fill one tile and tiles are not mostly
                           padding                                                */
  size_t slot_of_row;   /* uint32 [rows]    token slot of each grouped row (its row of
                           d; grouped form only)                                    */
} qmoe_layout;

/* Fill *out for these arguments (host-side arithmetic only, no launch).
 * QMM_ERR_NULL / QMM_ERR_ARG on bad arguments. */
int qmoe_workspace_layout(const qmm_weight *gate_up, const qmm_weight *down, int32_t num_routed,
                          int32_t num_shared, int32_t t, int32_t topk, qmoe_layout *out);

/* Zero-fill a workspace on `stream` (a kernel, not a memset node).  No call
 * needs it: workspaces may hold anything on entry.  For callers that want a
 * known state, e.g. to compare workspaces between runs. */
int qworkspace_init(void *workspace, size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *qstatus_string(int status);

/* hipError_t of the last QMM_ERR_HIP returned on this thread (0 if none). */
int qlast_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
