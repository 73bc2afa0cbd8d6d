/*
 * bsfp8.h -- block-scaled FP8 grouped quantize and GEMMs for MoE expert layers (gfx950).
 *
 * C ABI of libbsfp8.so.  The library computes, on one GPU, the three steps of the expert-layer
 * path that the following pages turn on:
 *   - DeepGEMM issue #365, "Non-deterministic numerical problem of
 *     k_grouped_fp8_gemm_nt_contiguous" (reproducer: per-channel cast, K-major pack,
 *     k-grouped weight-gradient GEMM with a 1 x 128 fp32 scale recipe, determinism stress);
 *   - TransformerEngine issue #3484, "NaN expert weight gradients at num_groups == 1 with a
 *     padded token buffer for SReLU" (MXFP8 1x32 block scaling, padded token buffers, wgrad
 *     accumulated into an fp32 main_grad, expected behaviour: padding never matters);
 *   - TransformerEngine PR #3224, "Improve device-init grouped linear module with single
 *     grouped weight support" (per-group scale strides in grouped quantize, output reuse,
 *     zero-row early return, device-resident split sizes).
 *
 * Conventions for every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library allocates
 *     nothing, keeps no global mutable state, and is reentrant.  Every call is asynchronous
 *     on `stream` (a hipStream_t; NULL = the default stream) with no host synchronization and
 *     no device-to-host copy; it may be captured in a HIP graph.
 *   - Groups: `split_sizes` is a device int32 array of `num_groups` row counts k_e.  Group e
 *     owns rows [off_e, off_e + k_e) of a token buffer of `capacity_rows` rows, where
 *     off_e = k_0 + ... + k_{e-1}.  Rows at or past T = sum(k_e) are padding: they are never
 *     read and may hold any bits.  num_groups == 1, empty groups and groups of any size
 *     (no alignment of k_e is required) take the same code path.
 *   - Padded group extents (the colwise layouts): Kp_e = 128 * ceil(k_e / 128) and
 *     P_e = Kp_0 + ... + Kp_{e-1}.
 *   - Host-checkable errors return a negative BSFP8_ERR_* code before anything is launched.
 *     Data errors that only the device can see (a negative k_e, or T > capacity_rows) set bits
 *     in `*status` (when `status` is not NULL) with a bitwise OR; the kernels of that call then
 *     write nothing at all.  The library never clears `*status`.
 *   - Results are deterministic: no atomics on data, no split-K; repeated calls on the same
 *     inputs give bitwise identical outputs.
 */
#ifndef BSFP8_H
#define BSFP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Quantization recipes. */
#define BSFP8_RECIPE_MX_1X32_E8M0 1       /* e4m3 data, one E8M0 power-of-two scale per 32 values */
#define BSFP8_RECIPE_PER_CHANNEL_128_F32 2 /* e4m3 data, one fp32 scale per channel per 128 rows */
#define BSFP8_RECIPE_MXFP4_1X32_E8M0 3     /* e2m1 data (two per byte), one E8M0 scale per 32 values */

/*
 * GEMM arithmetic modifier, OR-ed into the recipe argument of the three GEMM calls only:
 * BSFP8_RECIPE_MX_1X32_E8M0 | BSFP8_GEMM_FP8_MFMA multiplies the same MXFP8 operands on the
 * scaled FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, codes and E8M0 bytes as they are) instead
 * of widening them exactly to bf16.  Twice the MFMA rate, but the instruction does not sum the
 * products of 8 consecutive K values exactly (smaller products are cut to a window under the
 * largest, toward zero): on MXFP8-quantized Gaussian data the relative Frobenius error is about
 * 1.5e-5 instead of about 1e-7, above the 1e-5 bound the widened path meets.  For callers that
 * accept that error; the widened path stays the default.  Other recipes, and the quantize
 * calls, reject the modifier (BSFP8_ERR_RECIPE).
 */
#define BSFP8_GEMM_FP8_MFMA 0x100

/* Layout selection bits for bsfp8_grouped_quantize. */
#define BSFP8_ROWWISE 1 /* blocks along a row (channels); used by the forward GEMM */
#define BSFP8_COLWISE 2 /* blocks along the token axis within each group; used by wgrad */

/* Activations of bsfp8_grouped_act_quantize. */
#define BSFP8_ACT_SRELU 1      /* y = p * max(h, 0)^2 (scaled squared ReLU) */
#define BSFP8_ACT_SRELU_GRAD 2 /* g = dy * p * 2 max(h, 0) (its gradient with respect to h) */
#define BSFP8_ACT_SWIGLU 3     /* y = p * silu(a) * b, (a | b) the halves of fc1's output row */
#define BSFP8_ACT_SWIGLU_GRAD 4 /* (da | db): the gradient of the scaled SwiGLU */

/* Output element types of bsfp8_grouped_gemm_fprop. */
#define BSFP8_OUT_F32 0
#define BSFP8_OUT_BF16 1

/* Device status bits. */
#define BSFP8_STATUS_NEGATIVE_SPLIT 1u   /* some k_e < 0 */
#define BSFP8_STATUS_EXCEEDS_CAPACITY 2u /* sum(k_e) > capacity_rows */

/* Return codes. */
#define BSFP8_OK 0
#define BSFP8_ERR_NULL_POINTER (-1)  /* a required pointer is NULL */
#define BSFP8_ERR_NUM_GROUPS (-2)    /* num_groups <= 0 or > BSFP8_MAX_GROUPS */
#define BSFP8_ERR_RECIPE (-3)        /* unknown recipe */
#define BSFP8_ERR_SHAPE (-4)         /* a dimension is negative or not a multiple of 32 */
#define BSFP8_ERR_ALIGNMENT (-5)     /* a pointer is not 16-byte aligned */
#define BSFP8_ERR_LAYOUT (-6)        /* layout/recipe combination not supported */
#define BSFP8_ERR_ARGUMENT (-7)      /* other invalid argument (flags, zero_amax_scale) */
#define BSFP8_ERR_LAUNCH (-8)        /* the HIP runtime refused a launch */

#define BSFP8_MAX_GROUPS 1024

/* ----------------------------------------------------------------------------------------- */
/* Buffer sizes.  Pure host functions; they return 0 for invalid arguments.                   */
/* ----------------------------------------------------------------------------------------- */

/* Upper bound of sum(Kp_e) over all valid split sizes: 128 * floor((R + 127 * E) / 128). */
int64_t bsfp8_colwise_rows_bound(int64_t capacity_rows, int32_t num_groups);
/* Bytes of a colwise data buffer: cols * bsfp8_colwise_rows_bound(R, E) (half that for MXFP4). */
size_t bsfp8_colwise_data_bytes(int64_t capacity_rows, int64_t cols, int32_t num_groups, int recipe);
/* Bytes of a colwise scale buffer: rows_bound * cols / 32 (MX, MXFP4) or rows_bound * cols / 128 * 4. */
size_t bsfp8_colwise_scale_bytes(int64_t capacity_rows, int64_t cols, int32_t num_groups, int recipe);
/* Bytes of rowwise data (rows * cols for MXFP8, rows * cols / 2 for MXFP4; 0 for the
 * per-channel recipe, which has no rowwise layout) and of its E8M0 scales (rows * cols / 32). */
size_t bsfp8_rowwise_data_bytes(int64_t rows, int64_t cols, int recipe);
size_t bsfp8_rowwise_scale_bytes(int64_t rows, int64_t cols);

/* ----------------------------------------------------------------------------------------- */
/* Grouped quantize: bf16 -> e4m3 / e2m1 with block scales (DeepGEMM #365 reproducer,         */
/* per-channel cast; TE #3484 MXFP8 block scaling, and the 4-bit quantizer its additional     */
/* context says the same gated paths accept; TE PR #3224, per-member columnwise scale strides). */
/* ----------------------------------------------------------------------------------------- */
/*
 * in_bf16         [capacity_rows][cols] bf16, row-major.
 * split_sizes     device int32[num_groups]; may be NULL only when which == BSFP8_ROWWISE,
 *                 meaning that all capacity_rows rows are live (e.g. a weight [E*N][K]).
 * which           BSFP8_ROWWISE, BSFP8_COLWISE or both (rowwise needs an MX recipe).
 * zero_amax_scale per-channel recipe only: the scale used when a block's amax is 0 (the
 *                 reproducer's sf_val, default 1e-30); must be finite and >= 0.
 *
 * MX 1x32 E8M0 (both layouts): for a block of up to 32 live values with maximum magnitude
 *   amax, e is the smallest integer in [-127, 127] with amax <= 448 * 2^e (amax == 0 gives
 *   -127); the scale byte is e + 127 and each value v becomes e4m3(v * 2^-e).
 * Per-channel 128 (colwise only): for a block of up to 128 live rows of one channel,
 *   sf = fp32(amax / 448); sf == 0 becomes zero_amax_scale; sf = max(sf, 1e-30);
 *   each value v becomes e4m3(fp32(v * fp32(1 / sf))); the fp32 sf is stored.
 * e4m3 is OCP E4M3FN, round to nearest even, sign kept (both recipes keep |v| <= 448).
 * MXFP4 1x32 E8M0 (both layouts): as MXFP8 with 6 in place of 448 (e is the smallest integer in
 *   [-127, 127] with amax <= 6 * 2^e) and each value becoming e2m1(v * 2^-e): OCP FP4 E2M1
 *   (0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives), round to nearest even, sign kept.  The codes of
 *   elements 2i and 2i + 1 along the contiguous axis share a byte, 2i in bits 3..0.
 *
 * Outputs (all caller-allocated; only the requested ones may be non-NULL).  The offsets below
 * count data elements; for MXFP4 element i is a nibble of byte i / 2 (see above).
 *   row_q  [capacity_rows][cols] e4m3: row r, column c at r*cols + c      (live rows only)
 *   row_s  [cols/32][capacity_rows] E8M0: row r, block b at b*capacity_rows + r (live rows only)
 *   col_q  bsfp8_colwise_data_bytes(): group e, row t < Kp_e, column c at
 *          cols*P_e + c*Kp_e + t (each group's rows transposed, token axis contiguous);
 *          lanes k_e <= t < Kp_e hold 0x00.
 *   col_s  MX : E8M0 byte (e, b, c) at cols*P_e/32 + b*cols + c, b < Kp_e/32
 *               (a block with no live row holds byte 0);
 *          PC : fp32 (e, b, c) at cols*P_e/128 + b*cols + c, b < Kp_e/128.
 *   Blocks restart at every group start; a partial block takes its amax over live rows only.
 *   Bytes of col_q / col_s past cols*sum(Kp_e) are not written.
 * noop_flag       NULL, or a device fp32 scalar read by the kernels when they run (TE PR #3224,
 *                 group_quantize output reuse: the noop flag of the FP8 block-scaling path).  A
 *                 nonzero value makes the call a no-op on the device: no output byte and no status
 *                 bit is written, so storage filled by an earlier call (a cached quantized weight)
 *                 is reused as it stands.  Zero (or NULL) quantizes as usual, overwriting the
 *                 caller's pre-allocated outputs in place.  The flag is read on the device, so one
 *                 captured graph serves both the first microbatch (flag 0) and the rest (flag 1).
 *                 4-byte aligned.
 * capacity_rows == 0 returns BSFP8_OK without touching any pointer.
 */
int bsfp8_grouped_quantize(const void* in_bf16, int64_t capacity_rows, int64_t cols,
                           const int32_t* split_sizes, int32_t num_groups, int recipe, int which,
                           float zero_amax_scale, uint8_t* row_q, uint8_t* row_s, uint8_t* col_q,
                           void* col_s, const float* noop_flag, uint32_t* status, void* stream);

/* ----------------------------------------------------------------------------------------- */
/* Activation fused with the grouped quantize (TE #3484 reproducer: fc1 -> ScaledSReLU -> fc2   */
/* with per-token probs; its additional context names the ScaledSwiGLU family beside it; the  */
/* formulas are the usual scaled squared ReLU and scaled SwiGLU).                             */
/* ----------------------------------------------------------------------------------------- */
/*
 * SReLU (activation 1, 2): cols is the row length of h and of the output.
 *   h_bf16   [capacity_rows][cols] bf16: fc1's output (forward) or fc1's output saved for the
 *            backward (BSFP8_ACT_SRELU_GRAD).
 *   dy_bf16  [capacity_rows][cols] bf16, the gradient arriving at the activation's output
 *            (BSFP8_ACT_SRELU_GRAD only; NULL otherwise).
 *   BSFP8_ACT_SRELU:      y = (r * r) * p
 *   BSFP8_ACT_SRELU_GRAD: g = ((2 * r) * p) * dy
 *   with r = h for h > 0 and +0 otherwise.
 * SwiGLU (activation 3, 4): cols is the GLU width F; h_bf16 is [capacity_rows][2F] with
 *   a = columns [0, F) and b = [F, 2F) of each row; dy_bf16 [capacity_rows][F] (gradient only).
 *   With t = exp2s(-a * log2(e)), sg = 1 / (1 + t), s = a * sg:
 *   BSFP8_ACT_SWIGLU:      y = (s * b) * p, quantized as [capacity_rows][F]
 *   BSFP8_ACT_SWIGLU_GRAD: q = dy * p; da = (q * b) * (sg * (1 + a * (1 - sg))); db = q * s,
 *                          quantized as [capacity_rows][2F] = (da | db)
 *   exp2s is a stated fp32 2^x: x clamped to [-126, 126], k = floor(x + 1/2), r = x - k, the
 *   degree-7 Taylor polynomial of exp(r ln 2) with fp32 coefficients (ln 2)^n / n! in Horner
 *   form, times 2^k (relative error below 3e-7; reproducible bit for bit on any IEEE machine).
 * probs      device fp32 [capacity_rows]: the token's routing probability p, or NULL for p = 1.
 * Every operation is rounded to fp32 in the order written (no fused multiply-add); division is
 * correctly rounded.  The fp32 values of the live rows are quantized the way
 * bsfp8_grouped_quantize quantizes a bf16 input, for recipe BSFP8_RECIPE_MX_1X32_E8M0 or
 * BSFP8_RECIPE_MXFP4_1X32_E8M0, into the same layouts (rowwise for the next GEMM's forward,
 * colwise for its weight gradient), sized by the size queries for the output's shape:
 * [capacity_rows][cols] (SReLU), [capacity_rows][F] (SwiGLU) or [capacity_rows][2F] (its
 * gradient).
 * split_sizes is required; rows at or past sum(split_sizes) (of h, dy and probs) are never read.
 * Outputs, status and errors as bsfp8_grouped_quantize; capacity_rows == 0 returns BSFP8_OK
 * without touching any pointer.
 */
int bsfp8_grouped_act_quantize(int activation, const void* h_bf16, const float* probs,
                               const void* dy_bf16, int64_t capacity_rows, int64_t cols,
                               const int32_t* split_sizes, int32_t num_groups, int recipe, int which,
                               uint8_t* row_q, uint8_t* row_s, uint8_t* col_q, void* col_s,
                               uint32_t* status, void* stream);

/* ----------------------------------------------------------------------------------------- */
/* k-grouped weight-gradient GEMM (DeepGEMM #365, k_grouped_fp8_gemm_nt_contiguous; TE #3484, */
/* accumulate into an fp32 main_grad; the contraction runs over each group's tokens only).    */
/* All three recipes, and MXFP8 with BSFP8_GEMM_FP8_MFMA.                                     */
/* ----------------------------------------------------------------------------------------- */
/*
 * dy_col_q, dy_col_s  colwise output of bsfp8_grouped_quantize for dy [capacity_rows][n]
 * x_col_q,  x_col_s   colwise output for x [capacity_rows][h], same split_sizes and recipe
 * out                 fp32 [num_groups][n][h]:
 *     dW[e][i][j] = sum_{t < k_e} deq(dy)[off_e + t][i] * deq(x)[off_e + t][j]
 *   accumulate == 0 : out[e] = dW[e]           (an empty group gets zeros)
 *   accumulate == 1 : out[e] = out[e] + dW[e]  (one fp32 add per element; an empty group's
 *                                               slice is neither read nor written)
 * MX recipe: every e4m3 value is widened exactly with its E8M0 scale folded in; products
 *   accumulate in fp32.
 * Per-channel recipe: each 128-row block's unit-scale partial sum p is folded in as
 *   acc = fma(p, sdy_i * sx_j, acc) in block order.
 * MXFP4 recipe: the scaled fp4 MFMA takes the codes and E8M0 scales as they are (its sums of
 *   e2m1 products within a block are exact); products accumulate in fp32.
 * MX | BSFP8_GEMM_FP8_MFMA: the scaled fp8 MFMA takes the e4m3 codes and E8M0 scales as they
 *   are; results accumulate in fp32 across instructions, with the in-instruction error above.
 * n and h must be multiples of 32, h at most 2^21; capacity_rows + 127 must stay below
 * 2^24 - 128 (BSFP8_ERR_SHAPE otherwise): the kernels address an operand tile and a 128-row
 * output block with 32-bit offsets.
 */
int bsfp8_grouped_gemm_wgrad(const uint8_t* dy_col_q, const void* dy_col_s, int64_t n,
                             const uint8_t* x_col_q, const void* x_col_s, int64_t h,
                             const int32_t* split_sizes, int32_t num_groups, int64_t capacity_rows,
                             int recipe, float* out, int accumulate, uint32_t* status, void* stream);

/* ----------------------------------------------------------------------------------------- */
/* m-grouped forward GEMM (TE PR #3224, grouped GEMM over a single grouped weight; the token   */
/* axis is a free dimension).  recipe: BSFP8_RECIPE_MX_1X32_E8M0 (optionally with             */
/* BSFP8_GEMM_FP8_MFMA) or BSFP8_RECIPE_MXFP4_1X32_E8M0.                                      */
/* ----------------------------------------------------------------------------------------- */
/*
 * x_row_q, x_row_s  rowwise output of bsfp8_grouped_quantize for x [capacity_rows][k]
 *                   (the same recipe as the weight's)
 * w_q, w_s          rowwise output for the weight [num_groups * n][k] (split_sizes NULL):
 *                   expert e's row j is buffer row e*n + j; scales [k/32][num_groups * n]
 * out               [capacity_rows][n], fp32 or bf16 (round to nearest even from fp32):
 *     out[off_e + t][j] = sum_c deq(x)[off_e + t][c] * deq(W_e)[j][c]   for t < k_e
 *   rows at or past sum(k_e) are not written.
 * k and n must be multiples of 32, k below 2^24 - 128, n at most 2^21 (BSFP8_ERR_SHAPE
 * otherwise).  capacity_rows == 0 returns BSFP8_OK
 * without touching any pointer.
 */
int bsfp8_grouped_gemm_fprop(const uint8_t* x_row_q, const uint8_t* x_row_s, int64_t capacity_rows,
                             int64_t k, const uint8_t* w_q, const uint8_t* w_s, int64_t n,
                             const int32_t* split_sizes, int32_t num_groups, int recipe, void* out,
                             int out_dtype, uint32_t* status, void* stream);

/* ----------------------------------------------------------------------------------------- */
/* m-grouped data-gradient GEMM (the remaining GEMM of the expert backward beside wgrad and    */
/* fprop: TE #3484 scope -- the token axis is a free dimension of everything but wgrad).      */
/* recipe: BSFP8_RECIPE_MX_1X32_E8M0 (optionally with BSFP8_GEMM_FP8_MFMA) or                */
/* BSFP8_RECIPE_MXFP4_1X32_E8M0.                                                             */
/* ----------------------------------------------------------------------------------------- */
/*
 * dy_row_q, dy_row_s  rowwise output of bsfp8_grouped_quantize for dy [capacity_rows][n]
 * w_col_q, w_col_s    colwise output of bsfp8_grouped_quantize for the weight viewed as
 *                     [num_groups * n][k] with split sizes n, ..., n (num_groups of them): the
 *                     32-blocks run along n inside each expert, so expert e's matrix is
 *                     transposed in the buffer -- output channel j, contraction index c at
 *                     element k*np*e + j*np + c with np = 128 * ceil(n / 128); E8M0 (e, b, j) at
 *                     k*np*e/32 + b*k + j (bsfp8_colwise_data_bytes / _scale_bytes with
 *                     capacity_rows = num_groups * n give the sizes)
 * out                 [capacity_rows][k], fp32 or bf16 (round to nearest even from fp32):
 *     out[off_e + t][j] = sum_c deq(dy)[off_e + t][c] * deq(W_e)[c][j]   for t < k_e
 *   rows at or past sum(k_e) are not written.
 * n and k must be multiples of 32, n at most 2^24 - 256, k at most 2^21 (BSFP8_ERR_SHAPE
 * otherwise).  capacity_rows == 0 returns BSFP8_OK without touching any pointer.
 */
int bsfp8_grouped_gemm_dgrad(const uint8_t* dy_row_q, const uint8_t* dy_row_s, int64_t capacity_rows,
                             int64_t n, const uint8_t* w_col_q, const void* w_col_s, int64_t k,
                             const int32_t* split_sizes, int32_t num_groups, int recipe, void* out,
                             int out_dtype, uint32_t* status, void* stream);

/* Static description of a return code. */
const char* bsfp8_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* BSFP8_H */
