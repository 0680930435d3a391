/*
 * fp8sg.h -- C ABI of libfp8sg.so: FP8 quantisation under a scaling recipe and
 * the scaled FP8 GEMMs of a linear layer, as HIP kernels for MI355X (gfx950).
 *
 * What the calls compute is stated by these pages (cited by title and section):
 *   [guide]    "FP8 quantisation training practical guide" (scrxy.com): section
 *              "format choice: E4M3 and E5M2"; section "three scaling
 *              algorithms" (tensor-level, delayed with a buffer of past maxima,
 *              just-in-time from the current batch's maximum); section
 *              "blockwise scaling" (E4M3 only, 1x128 tiles for inputs and
 *              gradients, 128x128 blocks for weights, one scale per block);
 *              section "MXFP8 scaling" (1x32 blocks, E8M0 scales); section
 *              "code changes" (the three GEMMs of a Transformer layer take
 *              quantised inputs, outputs stay BF16).
 *   [colossal] QbitAI story on Colossal-AI FP8 mixed-precision training:
 *              paragraph on delayed vs real-time scaling.
 *   [snippets] "fp8+bf8" search-result page: the forward-pass snippet (BF16
 *              input, weights quantised to FP8, output back to BF16 after
 *              accumulation; dgrad cast to BF16 after the FP8 backward GEMM).
 *
 * Conventions for every call
 *   Memory      Every pointer argument except `stream` is device memory owned by
 *               the caller.  Tensors are dense and row-major.  The library
 *               allocates nothing and keeps no state between calls.
 *   Workspace   The calls that produce an amax (fp8_amax*, fp8_quantize_tensor*
 *               with amax_out, fp8_quantize_tensor_current,
 *               fp8_quantize_pair_current, fp8_gemm_fprop_fused with y_amax)
 *               reduce through a caller-owned device workspace of
 *               FP8_WORKSPACE_BYTES, 256-byte aligned: partial maxima, and
 *               the counters and flags of the one-launch grid-wide maximum.
 *               Before its first use it must be zero-filled (any zero fill,
 *               or fp8_workspace_init); every call leaves it ready for the
 *               next.  Calls that may run at the same time (on different
 *               streams, or graph replays on different streams) must use
 *               different workspaces; calls ordered on one stream may share
 *               one.  A graph captures the workspace address it was given.
 *   Stream      `stream` is a hipStream_t (NULL = the null stream).  Calls only
 *               enqueue kernels and return; nothing synchronises.  Outputs are
 *               valid once the stream has passed the call.
 *   Formats     FP8 bytes follow the OCP 8-bit formats: E4M3 is E4M3FN (bias 7,
 *               no infinity, max 448, NaN = S.1111.111); E5M2 has bias 15, max
 *               57344, IEEE-style inf/NaN.  BF16 tensors are passed as 16-bit
 *               words.  The cast is: one FP32 multiply x*scale, magnitudes above
 *               the format's maximum (and +-inf) saturate to +-max, any NaN
 *               becomes the canonical NaN code (0xFF for E4M3, 0xFE for E5M2,
 *               the gfx950 converter's codes), the rest rounds to nearest even.
 *   Scale rule  scale = fmax / amax in FP32 (fmax = 448 or 57344); 1 when amax
 *               is 0, inf or NaN; FLT_MAX when the quotient overflows.
 *               scale_inv = 1 / scale in FP32.  Quantise multiplies by scale,
 *               dequantise multiplies by scale_inv.
 *   amax        max |x| under the order NaN > inf > finite on magnitude bits, so
 *               a NaN anywhere gives a NaN amax.  Always exactly a BF16 value.
 *   Errors      Arguments are checked on the host before anything is enqueued;
 *               a failing check returns its status and has no side effect.
 *               FP8_ERR_HIP reports a launch failure.  NaN/inf data are not
 *               errors; they follow the rules above.
 *   Alignment   Data pointers must be 16-byte aligned (FP8_ERR_ALIGN).
 *   Empty       A tensor with zero elements may be passed as NULL; required
 *               pointers to non-empty tensors and to outputs such as amax may
 *               not (FP8_ERR_NULL).
 */
#ifndef FP8SG_H
#define FP8SG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Size in bytes of the workspace of the amax-producing calls (see Workspace):
 * 65536 words of partial maxima (one per workgroup of a quantise launch, at
 * most 2048, or one per 256x256 output tile of the fused GEMM epilogue),
 * 8320 words of grid-wide maximum counters, maxima and flags (two sets of 65
 * cache lines), and one 128-byte line of settings. */
#define FP8_WORKSPACE_BYTES 295552

typedef enum { FP8_E4M3 = 0, FP8_E5M2 = 1 } fp8_format_t;

typedef enum {
  FP8_SCALE_TENSOR = 0,        /* scale_inv: float[1]                                */
  FP8_SCALE_BLOCK_1x128 = 1,   /* scale_inv: float[rows][K/128]                      */
  FP8_SCALE_BLOCK_128x128 = 2, /* scale_inv: float[rows/128][K/128]                  */
  FP8_SCALE_MX_1x32 = 3        /* scale_inv: uint8 E8M0 [rows][K/32], byte = e + 127 */
} fp8_scaling_t;

typedef enum {
  FP8_OK = 0,
  FP8_ERR_NULL = 1,        /* a required pointer is NULL                          */
  FP8_ERR_SHAPE = 2,       /* negative size, or a size that breaks a block rule   */
  FP8_ERR_ALIGN = 3,       /* pointer or row length not suitably aligned          */
  FP8_ERR_UNSUPPORTED = 4, /* unknown enum value or unsupported combination       */
  FP8_ERR_HIP = 5          /* the HIP runtime rejected a launch                   */
} fp8_status_t;

/* One quantised GEMM operand: `data` is FP8 [rows][K] row-major (K contiguous,
 * K = the GEMM's contraction length), with its dequantisation scales. */
typedef struct {
  const uint8_t* data;
  int32_t fmt;             /* fp8_format_t  */
  int32_t scaling;         /* fp8_scaling_t */
  const void* scale_inv;   /* layout per fp8_scaling_t above */
} fp8_operand_t;

/* Prepare a workspace (FP8_WORKSPACE_BYTES, 256-byte aligned) for first
 * use: zero-fills it with a kernel on `stream` (no memset, so the call may be
 * captured in a graph) and sets the bound on the grid-wide wait of the
 * one-launch current scaling.
 *   wait_polls  0: the default bound (2^12 polls, about a millisecond);
 *               n > 0: n polls.  When a workgroup's wait runs out, one
 *               workgroup completes the amax from the maxima already in and
 *               the inputs of the workgroups that have not arrived, and
 *               publishes it, so results never change, only speed; 1 makes
 *               that path the common one (for tests).
 * Errors: NULL workspace; wait_polls < 0 (FP8_ERR_SHAPE); alignment. */
fp8_status_t fp8_workspace_init(void* workspace, int32_t wait_polls, void* stream);

/* amax of a BF16 tensor and, optionally, the scale pair it implies.
 * [colossal] real-time scaling / [guide] just-in-time scaling: the scale comes
 * from the maximum of the tensor being cast.
 *   x_bf16     [rows][cols] BF16, 16-byte aligned (any rows, cols >= 0)
 *   amax       out float[1]
 *   scale, scale_inv   out float[1] each, nullable (scale rule above)
 *   workspace  see Workspace
 * Errors: NULL x/amax/workspace; negative sizes; misaligned x or workspace;
 * fmt not E4M3/E5M2. */
fp8_status_t fp8_amax(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt,
                      float* amax, float* scale, float* scale_inv, void* workspace,
                      void* stream);

/* Per-tensor cast q = cast(x * scale[0]).  [guide] code changes: the GEMM
 * inputs are quantised; the transposed copy qT is the K-contiguous operand the
 * weight-gradient GEMM reads.
 *   x_bf16   [rows][cols] BF16;  cols % 16 == 0 (FP8_ERR_ALIGN)
 *   scale    in float[1] (device)
 *   q        out uint8 [rows][cols]
 *   qT       out uint8 [cols][rows], nullable; needs rows % 16 == 0
 *   amax_out out float[1], nullable: amax of x, fused into the same pass
 *            (delayed scaling records it in its history; [colossal] delayed
 *            scaling fuses the scale update with the GEMM pipeline)
 *   workspace  see Workspace; needed with amax_out, else may be NULL
 * Errors: NULL x/scale/q (or workspace with amax_out); negative sizes;
 * alignment; fmt. */
fp8_status_t fp8_quantize_tensor(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt,
                                 const float* scale, uint8_t* q, uint8_t* qT, float* amax_out,
                                 void* workspace, void* stream);

/* Per-tensor current scaling in one call: amax -> scale pair -> cast, the
 * sequence fp8_amax + fp8_quantize_tensor with identical results
 * ([colossal] real-time scaling takes the scale from the current tensor;
 * [guide] three scaling algorithms).  Without qT, when the tensor fits the
 * registers of a grid the device holds at once (up to about 50M elements on
 * MI355X), one launch: each thread keeps its share of x in registers, a
 * grid-wide maximum built from device-scope atomics gives every workgroup
 * the amax, and the workgroups cast what they hold, so x is read once.
 * Otherwise two launches: the amax pass, then the cast, whose workgroups
 * each reduce the amax pass's partial maxima and derive the scale
 * themselves.  The one-launch grid waits on itself: if other work keeps
 * part of it from being resident for about a millisecond, one waiting
 * workgroup reads the shares of the missing workgroups itself and publishes
 * the amax (same result, slower).
 *   x_bf16     [rows][cols] BF16, cols % 16 == 0
 *   q          out uint8 [rows][cols];  qT  out [cols][rows], nullable
 *              (rows % 16 == 0)
 *   amax       out float[1];  scale  out float[1], nullable;
 *   scale_inv  out float[1]
 *   workspace  see Workspace (the one-launch wait's bound is set there)
 * Errors as fp8_amax and fp8_quantize_tensor. */
fp8_status_t fp8_quantize_tensor_current(const void* x_bf16, int64_t rows, int64_t cols,
                                         int32_t fmt, uint8_t* q, uint8_t* qT, float* amax,
                                         float* scale, float* scale_inv, void* workspace,
                                         void* stream);

/* fp8_quantize_tensor_current for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same results, but no workspace argument.  The
 * call reduces through a static scratch array of the library, 24832 bytes
 * per GPU (2048 partial maxima, 129 lines of grid-wide maximum words, one
 * settings line), held from the first call on a GPU until the process ends;
 * that first call takes the array's device address and clears it with a
 * kernel on `stream`.  The scratch suffices for every tensor the regular
 * call accepts (a quantise launch writes at most 2048 partial maxima
 * whatever the tensor's size), so no size is rejected for it; the wait
 * bound is the default one.  All calls on one GPU share the array and each
 * leaves it ready for the next: calls ordered on one stream are safe, calls
 * that may overlap on one GPU (other streams, concurrent graph replays)
 * race and must not be made.  Nothing is allocated: no hipMalloc, hipFree
 * or allocating library routine.
 * Arguments and errors as fp8_quantize_tensor_current (without workspace);
 * FP8_ERR_HIP also reports a failure to find or clear the scratch. */
fp8_status_t fp8_quantize_tensor_current_noalloc(const void* x_bf16, int64_t rows, int64_t cols,
                                                 int32_t fmt, uint8_t* q, uint8_t* qT,
                                                 float* amax, float* scale, float* scale_inv,
                                                 void* stream);

/* Per-tensor current scaling of a GEMM's two operands (for instance X and W
 * of fprop) in one call: the results are exactly those of
 * fp8_quantize_tensor_current on each tensor without a transposed copy
 * ([colossal] real-time scaling; [guide] three scaling algorithms: each
 * tensor's scale comes from its own current maximum).  When the device holds
 * both tensors at once (about 67M elements in total on MI355X), one launch
 * does both: each workgroup keeps its share of one tensor in VGPRs and LDS,
 * and each tensor has a grid-wide maximum of its own, so the two tensors'
 * reads, waits and casts overlap.  Otherwise one fp8_quantize_tensor_current
 * per tensor.  The one-launch wait is bounded as in that call.
 *   a_bf16, b_bf16   [rows][cols] BF16 each, cols % 16 == 0
 *   a_fmt, b_fmt     their FP8 formats
 *   a_q, b_q         out uint8 [rows][cols] each
 *   a_amax, a_scale, a_scale_inv, b_amax, ...   out float[1] each; the scale
 *                    pointers are nullable
 * The two tensors' outputs must not overlap each other or either input.
 *   workspace        see Workspace (one for both tensors)
 * Errors as fp8_quantize_tensor_current, checked for a, then for b, before
 * any launch. */
fp8_status_t fp8_quantize_pair_current(const void* a_bf16, int64_t a_rows, int64_t a_cols,
                                       int32_t a_fmt, uint8_t* a_q, float* a_amax,
                                       float* a_scale, float* a_scale_inv, const void* b_bf16,
                                       int64_t b_rows, int64_t b_cols, int32_t b_fmt,
                                       uint8_t* b_q, float* b_amax, float* b_scale,
                                       float* b_scale_inv, void* workspace, void* stream);

/* FP32 master-weight input.  [snippets] forward-pass snippet: the master
 * weights are FP32 and are quantised to FP8 for the GEMM.  The same calls as
 * fp8_amax and fp8_quantize_tensor for an FP32 tensor: amax is the largest
 * |x| under NaN > inf > finite on the FP32 magnitude bits (exactly an FP32
 * value); the cast is sat_rne(fl32(x * scale)).  Shapes, alignment (16-byte
 * data), the workspace and errors as for the BF16 calls. */
fp8_status_t fp8_amax_f32(const float* x_f32, int64_t rows, int64_t cols, int32_t fmt,
                          float* amax, float* scale, float* scale_inv, void* workspace,
                          void* stream);
fp8_status_t fp8_quantize_tensor_f32(const float* x_f32, int64_t rows, int64_t cols, int32_t fmt,
                                     const float* scale, uint8_t* q, uint8_t* qT,
                                     float* amax_out, void* workspace, void* stream);

/* One delayed-scaling step.  [guide] delayed scaling keeps a buffer of the
 * maxima of past steps; [colossal] delayed scaling takes the scale from a
 * window of past values.
 *   history  in/out float[history_len] (1..1024), ring buffer; zeros initially
 *   step     >= 0: amax[0] is written to history[step % history_len]
 *   amax     in float[1] (device), this step's amax
 *   scale, scale_inv  out float[1]: the scale rule applied to max(history)
 *            (NaN propagates), i.e. the pair step+1 uses.
 * Order on one stream at step t: quantise with scale_t (fused amax) -> GEMMs
 * reading scale_inv_t -> this call with step = t.
 * Errors: NULL pointers; history_len out of range; step < 0; fmt. */
fp8_status_t fp8_amax_history_update(float* history, int32_t history_len, int64_t step,
                                     const float* amax, int32_t fmt, float* scale,
                                     float* scale_inv, void* stream);

/* Blockwise cast.  [guide] blockwise scaling: E4M3, inputs and gradients in
 * 1x128 tiles, weights in 128x128 blocks, each block scaled on its own.
 * Tiles run along the contiguous (contraction) dimension.
 *   block_rows  1 or 128;  block_cols  128
 *   x_bf16      [rows][cols] BF16, cols % 128 == 0, rows % block_rows == 0
 *   q           out uint8 [rows][cols]
 *   scale_inv   out float [rows/block_rows][cols/128]
 * Both FP8 formats are accepted (the pages use E4M3).
 * Errors: NULL; sizes; a block shape other than 1x128 / 128x128 or an unknown
 * fmt (FP8_ERR_UNSUPPORTED); cols % 128 or rows % block_rows (FP8_ERR_SHAPE);
 * alignment. */
fp8_status_t fp8_quantize_block(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt,
                                int32_t block_rows, int32_t block_cols, uint8_t* q,
                                float* scale_inv, void* stream);

/* MX cast.  [guide] MXFP8 scaling: uniform 1x32 blocks with E8M0 scales.
 * Per block along the contiguous dimension: e = the smallest integer with
 * amax <= fmax * 2^e (clamped to [-127, 127]), byte = e + 127; an all-zero
 * block gets 127; a block with inf/NaN gets 0xFF and its elements are cast
 * unscaled; q = cast(x * 2^-e).  Dequantisation multiplies by 2^e.
 *   x_bf16     [rows][cols] BF16, cols % 32 == 0
 *   q          out uint8 [rows][cols]
 *   scale_e8m0 out uint8 [rows][cols/32]
 * Both FP8 formats are accepted (the MXFP8 workloads use E4M3).
 * Errors: NULL; sizes; alignment; fmt. */
fp8_status_t fp8_quantize_mx(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt,
                             uint8_t* q, uint8_t* scale_e8m0, void* stream);

/* Blockwise cast with a transposed, column-wise copy for the backward GEMMs.
 * [guide] blockwise scaling: inputs and gradients in 1x128 tiles, weights in
 * 128x128 blocks.  dgrad contracts over the output features and wgrad over
 * the tokens, so next to the row-wise copy of a tensor x they need the
 * quantisation of x^T (W^T for dgrad, G^T and X^T for wgrad), whose
 * 128-long tiles run along x's rows:
 *   block_rows = 1    q, scale_inv   as fp8_quantize_block(x, 1, 128)
 *                     qT, scale_inv_T as fp8_quantize_block(x^T, 1, 128):
 *                     each column of x is cut into 128-row tiles, each tile
 *                     scaled on its own (re-quantised from BF16)
 *   block_rows = 128  q, scale_inv   as fp8_quantize_block(x, 128, 128)
 *                     qT = q^T, scale_inv_T = scale_inv^T (same blocks)
 *   x_bf16       [rows][cols] BF16, rows % 128 == 0, cols % 128 == 0
 *   q            out uint8 [rows][cols], nullable (then scale_inv NULL too)
 *   scale_inv    out float [rows/block_rows][cols/128]
 *   qT           out uint8 [cols][rows]
 *   scale_inv_T  out float [cols][rows/128] (block_rows 1) or
 *                [cols/128][rows/128] (block_rows 128)
 * One read of x writes both copies.  Errors: NULL (or q / scale_inv not both
 * given); sizes; block shape; alignment; fmt. */
fp8_status_t fp8_quantize_block_t(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt,
                                  int32_t block_rows, uint8_t* q, float* scale_inv, uint8_t* qT,
                                  float* scale_inv_T, void* stream);

/* MX cast with a transposed, column-wise copy for the backward GEMMs
 * ([guide] MXFP8 scaling: 1x32 blocks, E8M0 scales):
 *   q, scale_e8m0      as fp8_quantize_mx(x)   (blocks along x's rows)
 *   qT, scale_e8m0_T   as fp8_quantize_mx(x^T) (each column of x cut into
 *                      32-row blocks, re-quantised from BF16)
 *   x_bf16        [rows][cols] BF16, rows % 32 == 0, cols % 32 == 0
 *   q             out uint8 [rows][cols], nullable (then scale_e8m0 NULL too)
 *   scale_e8m0    out uint8 [rows][cols/32]
 *   qT            out uint8 [cols][rows]
 *   scale_e8m0_T  out uint8 [cols][rows/32]
 * Errors: NULL (or q / scale_e8m0 not both given); sizes; alignment; fmt. */
fp8_status_t fp8_quantize_mx_t(const void* x_bf16, int64_t rows, int64_t cols, int32_t fmt,
                               uint8_t* q, uint8_t* scale_e8m0, uint8_t* qT,
                               uint8_t* scale_e8m0_T, void* stream);

/* The three GEMMs of a linear layer ([guide] code changes; [snippets] forward
 * and backward flow), FP32 accumulation on MFMA, BF16 output (round to nearest
 * even).  Both operands are K-contiguous ("TN"), so one kernel serves all three:
 *   fprop  y[M][N]  = sum_k x[M][K](m,k)   * w[N][K](n,k)      (contract K)
 *   dgrad  dx[M][K] = sum_n dy[M][N](m,n)  * wT[K][N](k,n)     (contract N)
 *   wgrad  dw[N][K] = sum_m dyT[N][M](n,m) * xT[K][M](k,m)     (contract M)
 * Scaling of each output element c[i][j] over contraction index t:
 *   tensor x tensor:  (sa[0] * sb[0]) * sum_t a(i,t) b(j,t)
 *   block  x block :  sum_b sa(i,b) * sb(j,b) * sum_{t in block b} a(i,t) b(j,t)
 *                     (each operand 1x128 or 128x128; 128-wide blocks along t)
 *   MX     x MX    :  sum_t a(i,t) 2^ea(i,t/32) * b(j,t) 2^eb(j,t/32)
 * Shape rules: sizes >= 0; contraction % 16 == 0 (FP8_ERR_ALIGN); block
 * operands need contraction % 128 == 0 and, for 128x128, rows % 128 == 0; MX
 * needs contraction % 32 == 0; contraction <= 2^23 (FP8_ERR_SHAPE).  Mixed families are
 * FP8_ERR_UNSUPPORTED.  Output pointers must be 16-byte aligned.
 * Errors: NULL operand/data/scale/output; shapes; alignment; enums. */
fp8_status_t fp8_gemm_fprop(const fp8_operand_t* x, const fp8_operand_t* w, int64_t M,
                            int64_t N, int64_t K, void* y_bf16, void* stream);
fp8_status_t fp8_gemm_dgrad(const fp8_operand_t* dy, const fp8_operand_t* wT, int64_t M,
                            int64_t N, int64_t K, void* dx_bf16, void* stream);
fp8_status_t fp8_gemm_wgrad(const fp8_operand_t* dyT, const fp8_operand_t* xT, int64_t M,
                            int64_t N, int64_t K, void* dw_bf16, void* stream);

/* fprop with the next layer's quantisation fused into the epilogue.
 * [colossal] scaling paragraph: delayed scaling updates its scales fused
 * with the GEMM.  Besides (optionally) y = BF16(fprop result) it writes
 *   y_q     = cast(BF16(y) * y_scale[0]) in y_fmt: exactly the bytes
 *             fp8_quantize_tensor would produce from the BF16 y (NULL: skip;
 *             then y_scale may be NULL too);
 *   y_amax  = max |BF16(y)| (NaN > inf > finite), exactly what fp8_amax of
 *             the BF16 y gives (NULL: skip);
 * so the next layer reads the FP8 activation without another pass over y.
 *   y_bf16  out [M][N] BF16, may be NULL when y_q is given
 *   y_fmt   FP8 format of y_q;  y_scale  in float[1]
 *   y_q     out uint8 [M][N];   y_amax   out float[1]
 *   workspace  see Workspace; needed with y_amax, else may be NULL
 * At least one of y_q / y_amax must be given (else FP8_ERR_NULL; the plain
 * call is fp8_gemm_fprop).  N % 16 == 0 (FP8_ERR_ALIGN); at most 65536
 * 256x256 output tiles (FP8_ERR_SHAPE).  Other rules and errors as
 * fp8_gemm_fprop. */
fp8_status_t fp8_gemm_fprop_fused(const fp8_operand_t* x, const fp8_operand_t* w, int64_t M,
                                  int64_t N, int64_t K, void* y_bf16, int32_t y_fmt,
                                  const float* y_scale, uint8_t* y_q, float* y_amax,
                                  void* workspace, void* stream);

/* wgrad with an FP32 result, optionally accumulated.  [snippets] forward-
 * pass snippet: the master weights are FP32, so their gradient is too;
 * accumulating into it is how a weight gradient sums over micro-batches.
 *   dw_f32[N][K] = (accumulate ? dw_f32 : 0) + the wgrad sum of
 *                  fp8_gemm_wgrad (same operands, scaling and shape rules),
 * computed in FP32 and stored without rounding to BF16; with accumulate the
 * previous value is added in FP32 (one rounding).
 *   accumulate  0 or 1 (else FP8_ERR_UNSUPPORTED)
 *   dw_f32      in/out float [N][K], 16-byte aligned
 * Errors: as fp8_gemm_wgrad. */
fp8_status_t fp8_gemm_wgrad_f32(const fp8_operand_t* dyT, const fp8_operand_t* xT, int64_t M,
                                int64_t N, int64_t K, float* dw_f32, int32_t accumulate,
                                void* stream);

/* The cast's rounding step alone: q[i] = cast(x[i]) for FP32 inputs (no
 * scaling).  Every quantise kernel above rounds through the same device
 * routine; this entry point lets that routine be checked on any FP32 input.
 *   x  in float[n];  q  out uint8[n].  Errors: NULL; n < 0; alignment; fmt. */
fp8_status_t fp8_convert_f32(const float* x, int64_t n, int32_t fmt, uint8_t* q, void* stream);

/* Text for a status code (static storage). */
const char* fp8_status_string(fp8_status_t status);

#ifdef __cplusplus
}
#endif
#endif /* FP8SG_H */
