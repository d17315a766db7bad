/*
 * gptq.h -- C ABI of the GPTQ per-layer quantization path for AMD Instinct
 * MI355X (gfx950).
 *
 * The path quantizes one linear layer W [d_out, d_in] against calibration
 * inputs X [d_in, N] in four stages:
 *   1. H = 2 X X^T             (gptq_hessian_set, gptq_hessian_accumulate,
 *                               gptq_hessian_accumulate_chunks)
 *   2. H <- H + lambda I, dead channels skipped   (gptq_prepare_hinv)
 *   3. U upper with H^-1 = U^T U                  (gptq_prepare_hinv)
 *   4. fixed-order, block-lazy quantize-and-compensate sweep
 *                                                 (gptq_quantize_layer)
 * and, after the path, few-bit storage of the codes, dequantization and the
 * per-row output error (gptq_pack_codes, gptq_dequantize,
 * gptq_output_error), and the propagation of a quantized layer's output to
 * the next layer of a chain (gptq_propagate).
 *
 * Conventions shared by every entry point
 *   - Tensor arguments are DEVICE pointers allocated and owned by the caller;
 *     the library never allocates, frees or keeps caller memory.  Scratch
 *     memory is a caller-provided device workspace whose minimum size the
 *     *_workspace() queries return.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     default stream) and returns; results are valid once the stream has
 *     reached that point.  Calls on one stream run in order.
 *   - Matrices are row-major with the leading dimension stated per argument.
 *   - The return value reports argument and launch errors only
 *     (gptq_status).  Argument checks happen before any HIP call, so an
 *     invalid call touches no device state.  Numerical failure (a Hessian
 *     that is not positive definite) is reported through the device word
 *     `info` of gptq_prepare_hinv.
 *   - A size of 0 (d_out, d_in or n_tokens) is a valid empty problem: the
 *     call checks the other arguments and enqueues nothing.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GPTQ_OK = 0,
    GPTQ_EINVAL = 1,       /* invalid argument (null pointer, negative size, bits out of [2,8], ...) */
    GPTQ_EUNSUPPORTED = 2, /* valid request these kernels do not handle (documented per call) */
    GPTQ_EHIP = 3,         /* a HIP runtime call or kernel launch failed */
    GPTQ_EWORKSPACE = 4,   /* workspace pointer null or smaller than the *_workspace() size */
    GPTQ_ESCRATCH = 5      /* problem larger than the fixed scratch of a no-allocation entry point */
} gptq_status;

typedef enum {
    GPTQ_F16 = 0, /* IEEE binary16 */
    GPTQ_F32 = 1  /* IEEE binary32 */
} gptq_dtype;

/*
 * Stage 1 -- Hessian accumulation.
 * Operation (aicassindra.com "tm_gptq_math", section "Why it is
 * second-order: the Hessian"; math4ai "GPTQ Hessian", damping sentence):
 *     H += 2 * X * X^T
 * over the n_tokens columns of X; calling it once per token chunk streams a
 * long calibration set into one H (X X^T is a sum over tokens).  There is no
 * 1/N normalisation.
 *
 *   H        [d_in, d_in] float32, leading dimension d_in.  Only the lower
 *            triangle including the diagonal (row >= col) is read and
 *            written; the strictly upper triangle is left untouched.  The
 *            caller zeroes H before the first chunk, or writes the first
 *            chunk with gptq_hessian_set.
 *   X        [d_in, n_tokens] of x_dtype, row stride ldx elements (>= n_tokens):
 *            row i holds channel i's value for each token, so a token chunk
 *            of a larger X is the pointer X + t0 with the same ldx.
 *   Products of float16 inputs are exact in float32; accumulation is float32
 *   (MFMA), with one float32 add into H per call.
 * Errors: GPTQ_EINVAL for H or X null (when the problem is not empty),
 * d_in < 0, n_tokens < 0, ldx < n_tokens, unknown x_dtype.
 */
int gptq_hessian_accumulate(float* H, int64_t d_in, const void* X, int x_dtype,
                            int64_t n_tokens, int64_t ldx, void* stream);

/*
 * Stage 1, first (or only) token chunk -- the same operation without the
 * previous H (same sections of the same pages):
 *     H = 2 * X * X^T
 * on the lower triangle including the diagonal; the strictly upper triangle
 * is not written.  The old values of H are neither read nor needed, so the
 * caller does not zero H first; later chunks go through
 * gptq_hessian_accumulate.  n_tokens = 0 writes zeros (an empty sum).  The
 * products and the float32 accumulation are those of
 * gptq_hessian_accumulate, so setting and then accumulating gives the same
 * H, bit for bit, as accumulating every chunk into a zeroed H.
 * Arguments as gptq_hessian_accumulate.
 * Errors: GPTQ_EINVAL for H null (d_in > 0), X null with n_tokens > 0,
 * d_in < 0, n_tokens < 0, ldx < n_tokens, unknown x_dtype.
 */
int gptq_hessian_set(float* H, int64_t d_in, const void* X, int x_dtype,
                     int64_t n_tokens, int64_t ldx, void* stream);

/*
 * Stage 1 over several token chunks in one call (same sections of the same
 * pages):
 *     H = [H +] sum_c 2 * X_c * X_c^T,   c = 0 .. n_chunks-1
 * on the lower triangle including the diagonal; the strictly upper triangle
 * is not written.  For callers that hold several chunks at once (separate
 * buffers, one shape): up to 32 float16 chunks whose rows start 16-byte
 * aligned and whose n_tokens is a multiple of 64 are summed in one launch,
 * with a single float32 add into H, instead of one read-modify-write of H
 * per chunk.  Other chunks (float32, unaligned, ragged) are added one call
 * per chunk, as by gptq_hessian_set / gptq_hessian_accumulate.  The sum
 * over a group of chunks equals, bit for bit, one gptq_hessian_accumulate
 * call over the same tokens stored contiguously; against one call per
 * chunk it differs only by float32 rounding of the per-chunk adds.
 *
 *   X_chunks  HOST array of n_chunks DEVICE pointers; chunk c is
 *             [d_in, n_tokens] of x_dtype with row stride ldx.
 *   set       1: the first chunk writes H (old values neither read nor
 *             needed; n_chunks = 0 or n_tokens = 0 writes zeros);
 *             0: every chunk adds into H.
 *   other arguments as gptq_hessian_accumulate.
 * Errors: GPTQ_EINVAL for H null (when anything is written), X_chunks or a
 * chunk pointer null with n_chunks, n_tokens > 0, d_in < 0, n_chunks < 0,
 * n_tokens < 0, ldx < n_tokens, set not 0 or 1, unknown x_dtype.
 */
int gptq_hessian_accumulate_chunks(float* H, int64_t d_in, const void* const* X_chunks, int64_t n_chunks,
                                   int x_dtype, int64_t n_tokens, int64_t ldx, int set, void* stream);

/*
 * Stages 2 and 3 -- damping, dead channels and the factor U.
 * Operation (aicassindra "The Cholesky trick for the inverse Hessian";
 * math4ai "GPTQ Hessian", damping sentence and column-sweep paragraph;
 * mbrenndoerfer "GPTQ > Mathematical Details of the Update", Cholesky
 * paragraph):
 *     dead_i  = (H_ii == 0)                 channels the data never excited
 *     lambda  = damp_frac * mean_i H_ii      over all d_in entries (dead = 0)
 *     H_dd    = 1 for dead d, then H_ii += lambda for every i
 *     U       upper triangular, U_ii > 0, with H^-1 = U^T U
 * U is computed as the inverse of the reverse-order Cholesky factor
 * (H = R R^T, R upper, U = R^-1), which equals the Cholesky factor of H^-1
 * by uniqueness, in float64 (MFMA f64), and is rounded to float32 once.
 *
 *   H          [d_in, d_in] float32, lower triangle read (as written by
 *              gptq_hessian_accumulate); not modified.
 *   damp_frac  lambda as a fraction of the mean diagonal (0.01 = 1%); >= 0.
 *   U          [d_in, d_in] float32 output, leading dimension d_in; the
 *              strictly lower triangle is written as 0.
 *   dead       [d_in] uint8 output (1 = dead channel), may be NULL.
 *   info       device int32 output: 0 on success; k > 0 if the damped
 *              Hessian is not positive definite, where k is the order of the
 *              smallest trailing principal submatrix H[d_in-k:, d_in-k:]
 *              found not positive definite (U is then undefined).
 *   lambda_out device double output (lambda used), may be NULL.
 *   workspace  device memory of at least gptq_prepare_hinv_workspace(d_in)
 *              bytes, 256-byte aligned; clobbered.
 * Errors: GPTQ_EINVAL (null H, U or info when d_in > 0; d_in < 0;
 * damp_frac < 0 or not finite), GPTQ_EWORKSPACE.
 */
size_t gptq_prepare_hinv_workspace(int64_t d_in);
int gptq_prepare_hinv(const float* H, int64_t d_in, double damp_frac, float* U, uint8_t* dead,
                      int32_t* info, double* lambda_out, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * gptq_prepare_hinv with the factorization in float32: the same operation,
 * route, arguments, outputs and errors, but G = J H J is held in float32
 * and every product of the blocked factorization runs on MFMA f32 with
 * float32 accumulation (the pages run the Cholesky of the damped H in the
 * working precision; aicassindra "The Cholesky trick for the inverse
 * Hessian").  Rounding grows with the condition number of the damped H:
 * with damp_frac = 0.01 the relative Frobenius error of U against a float64
 * factorization stays near 1e-6 on Hessians whose damped condition number
 * is up to about 1e5; inputs worse conditioned than that belong on
 * gptq_prepare_hinv.  The damping statistics (lambda, dead flags) are
 * computed in float64 as there.  info reports a failed pivot in the same
 * way, judged on the float32 pivots.
 *   workspace  at least gptq_prepare_hinv_fp32_workspace(d_in) bytes,
 *              256-byte aligned; clobbered.
 */
size_t gptq_prepare_hinv_fp32_workspace(int64_t d_in);
int gptq_prepare_hinv_fp32(const float* H, int64_t d_in, double damp_frac, float* U, uint8_t* dead,
                           int32_t* info, double* lambda_out, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * gptq_prepare_hinv without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight loops, harnesses that forbid hipMalloc).  Same operation,
 * arguments, kernels and results as gptq_prepare_hinv; the workspace is a
 * fixed device array inside the library instead, sized for
 * d_in <= gptq_prepare_hinv_noalloc_max_din() (4096: about 134 MiB, held on
 * every device the library runs on until the process ends).  Its device
 * address is looked up once per device on the first call there (with that
 * device current).  The call makes no hipMalloc, hipFree or other
 * allocating call and records no timing events.
 * Every call on one device shares that device's array: calls that overlap
 * on one device (concurrent streams, or host threads) race and give
 * undefined results; calls in order on one stream are safe.  Nothing in the
 * array needs clearing between calls (every byte read is written first by
 * the same call).
 * Errors: as gptq_prepare_hinv, except that GPTQ_EWORKSPACE cannot occur;
 * GPTQ_ESCRATCH for d_in above gptq_prepare_hinv_noalloc_max_din();
 * GPTQ_EHIP if the array's address cannot be obtained.
 */
int gptq_prepare_hinv_noalloc(const float* H, int64_t d_in, double damp_frac, float* U, uint8_t* dead,
                              int32_t* info, double* lambda_out, void* stream);
int64_t gptq_prepare_hinv_noalloc_max_din(void);

/*
 * Stage 4 -- the quantize-and-compensate sweep.
 * Operation (aicassindra "Greedy quantization with error compensation" and
 * "GPTQ's speedups: fixed order and lazy batches"; math4ai "GPTQ Hessian",
 * column-sweep paragraph): columns j = 0 .. d_in-1 in order, all rows in
 * lockstep, in blocks of block_size columns.  For each column j:
 *     v       = fl32(fl32(w_j / s) + z)           position on the grid
 *     q       = clamp(rint(v), 0, 2^bits - 1)     the code (round half to even)
 *     e       = (w_j - s (q - z)) / U_jj           scaled error
 *     w_k    -= e U_jk   for later columns k of the same block (at once)
 * and after each block [b0, b1):
 *     W[:, b1:] -= E[:, b0:b1] U[b0:b1, b1:]      (lazy batched update)
 * Grid: asymmetric min-max over [min(0, min w), max(0, max w)] (an all-zero
 * range becomes [-1, 1]), s = fl32(fl32(mx - mn) / maxq),
 * z = clamp(rint(fl32(-mn / s)), 0, maxq), all IEEE float32.
 * group_size == 0: one grid per row from the input W.  group_size > 0: a new
 * grid at every column j with j % group_size == 0, from the current
 * (partially compensated) W[:, j : j + group_size].
 * Dead channels: W[:, dead] is set to 0 after the per-row grid, so their code
 * is z and they move nothing.
 *
 *   W           [d_out, d_in] of w_dtype, leading dimension d_in; not modified.
 *   U           [d_in, d_in] float32 upper factor (gptq_prepare_hinv output).
 *   dead        [d_in] uint8 or NULL (no dead channels).
 *   bits        2..8.
 *   group_size  0, or a multiple of 16 that divides d_in and either divides
 *               block_size or is a multiple of it (GPTQ_EUNSUPPORTED
 *               otherwise).
 *   block_size  1..128 columns per lazy block (the U block of the current
 *               lazy block is staged in LDS).
 *   codes       [d_out, d_in] uint8 output (one code per byte).
 *   scales      [d_out, n_groups] float32 output, n_groups = 1 if group_size
 *               == 0 else d_in / group_size.
 *   zeros       [d_out, n_groups] int32 output.
 *   err_row     [d_out] float32 output or NULL: sum over j of e_j^2 per row
 *               (the layer loss in the metric of the damped H).
 *   minmax      [d_out, n_groups, 2] float32 output or NULL: the range
 *               (min(0, min w), max(0, max w)) each grid was built from.
 *   workspace   at least gptq_quantize_layer_workspace(d_out, d_in,
 *               block_size) bytes of device memory, 256-byte aligned.
 * Errors: GPTQ_EINVAL (null required pointer, negative sizes, bits outside
 * [2, 8], block_size outside [1, 128], negative group_size, group_size not
 * dividing d_in, unknown w_dtype), GPTQ_EUNSUPPORTED (group_size not a
 * multiple of 16, or neither dividing nor a multiple of block_size),
 * GPTQ_EWORKSPACE.
 */
size_t gptq_quantize_layer_workspace(int64_t d_out, int64_t d_in, int64_t block_size);
int gptq_quantize_layer(const void* W, int w_dtype, int64_t d_out, int64_t d_in, const float* U,
                        const uint8_t* dead, int bits, int64_t group_size, int64_t block_size,
                        uint8_t* codes, float* scales, int32_t* zeros, float* err_row,
                        float* minmax, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gptq_quantize_layer with the lazy trailing update's products in split
 * precision (aicassindra "GPTQ's speedups: fixed order and lazy batches":
 * the batched update is the dense product that carries the arithmetic).
 * For W[:, b1:] -= E U[b0:b1, b1:] each fp32 operand is written as the sum
 * of three bf16 pieces, x = x0 + x1 + x2 (x0 the nearest bf16 to x, x1 that
 * of x - x0, x2 that of x - x0 - x1), and the product is formed from the six
 * piece products with i + j <= 2 on bf16 MFMA with fp32 accumulation: every
 * piece product is exact in fp32 and the three left out are below 2^-26 of
 * |e u|, so the update carries fp32-level error at the bf16 MFMA rate.  The
 * in-block sweep, the grids and everything else are as in
 * gptq_quantize_layer; arguments, outputs and errors are the same, except
 * that the workspace must hold gptq_quantize_layer_split_workspace() bytes:
 * it also keeps the bf16 pieces of U, written once per call,
 * 6 ceil(d_in/block_size) d_in ceil(block_size/16)*16 bytes (100 MB at
 * d_in = 4096, block 128).
 */
size_t gptq_quantize_layer_split_workspace(int64_t d_out, int64_t d_in, int64_t block_size);
int gptq_quantize_layer_split(const void* W, int w_dtype, int64_t d_out, int64_t d_in, const float* U,
                              const uint8_t* dead, int bits, int64_t group_size, int64_t block_size,
                              uint8_t* codes, float* scales, int32_t* zeros, float* err_row, float* minmax,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Few-bit storage of the codes (aicassindra.com "tm_gptq_math",
 * "Post-training quantization and the per-layer objective": weights go from
 * 16-bit floats to low-bit integers, 4-bit being the example given; the
 * pages fix no bit layout).  Layout: each
 * row's codes form one little-endian bit stream, code j in bits
 * [j bits, (j+1) bits), least significant bit first, cut into 32-bit words;
 * a row holds gptq_packed_words(d_in, bits) = ceil(d_in bits / 32) words,
 * the last one zero-padded.  Codes may straddle two words.
 *
 * gptq_packed_words: words per row, or -1 for d_in < 0 or bits outside
 *   [2, 8].
 * gptq_pack_codes:
 *   codes   [d_out, d_in] uint8 input (bits above the low `bits` ignored).
 *   packed  [d_out, gptq_packed_words(d_in, bits)] uint32 output.
 * Errors: GPTQ_EINVAL (negative sizes, bits outside [2, 8], null pointer),
 * GPTQ_EUNSUPPORTED (d_out or d_in above 2^24).
 */
int64_t gptq_packed_words(int64_t d_in, int bits);
int gptq_pack_codes(const uint8_t* codes, int64_t d_out, int64_t d_in, int bits, uint32_t* packed,
                    void* stream);

/*
 * Dequantization What = s (q - z) from packed codes (aicassindra
 * "Post-training quantization and the per-layer objective", the grid of "A worked
 * two-weight example").  The exact product of the scale and the integer
 * q - z is rounded once to the output type, to nearest even (one fp32
 * multiply, or one mixed-precision multiply with an fp16 result).
 *   packed      [d_out, gptq_packed_words(d_in, bits)] uint32 (as above).
 *   scales      [d_out, n_groups] float32, zeros [d_out, n_groups] int32,
 *               n_groups = 1 if group_size == 0 else d_in / group_size
 *               (the outputs of gptq_quantize_layer).
 *   out         [d_out, d_in] of out_dtype (GPTQ_F16 or GPTQ_F32).
 * Errors: GPTQ_EINVAL (negative sizes, bits outside [2, 8], negative
 * group_size or one not dividing d_in, unknown out_dtype, null pointer),
 * GPTQ_EUNSUPPORTED (d_out or d_in above 2^24).
 */
int gptq_dequantize(const uint32_t* packed, int bits, int64_t d_out, int64_t d_in, const float* scales,
                    const int32_t* zeros, int64_t group_size, void* out, int out_dtype, void* stream);

/*
 * Per-row layer output error ||dw X||^2 without X, from the loss identity
 * (aicassindra "The reconstruction objective, written out" with the damped
 * Hessian of "The Cholesky trick for the inverse Hessian"): a row's sum of
 * squared scaled errors is dw H_damped dw^T = 2 ||dw X||^2 + lambda ||dw||^2,
 * so out_row[r] = (err_row[r] - lambda ||dw_r||^2) / 2 with dw = W0 - What,
 * W0 the weights with the dead columns zeroed and What dequantized from the
 * packed codes.  ||dw||^2 is summed in float64.
 *   W        [d_out, d_in] of w_dtype: the weights given to
 *            gptq_quantize_layer.
 *   dead     [d_in] uint8 or NULL (no dead columns).
 *   packed, scales, zeros, group_size: as for gptq_dequantize.
 *   err_row  [d_out] float32: the err_row output of gptq_quantize_layer.
 *   lambda   device float64 scalar: the damping of gptq_prepare_hinv
 *            (its lambda_out).
 *   out_row  [d_out] float32 output.
 * Errors: as gptq_dequantize (w_dtype in place of out_dtype), plus
 * GPTQ_EINVAL for a null err_row, lambda or out_row.
 */
int gptq_output_error(const void* W, int w_dtype, const uint8_t* dead, const uint32_t* packed, int bits,
                      const float* scales, const int32_t* zeros, int64_t group_size, int64_t d_out, int64_t d_in,
                      const float* err_row, const double* lambda, float* out_row, void* stream);

/*
 * Propagation to the next layer: Y = act(What X).  The pages quantize a
 * network one linear layer at a time, each layer against its own input
 * activations (math4ai "GPTQ Hessian", opening paragraph; aicassindra
 * "Post-training quantization and the per-layer objective"); in a chain the
 * next layer's X is the already-quantized layer's output.  The f16
 * products are exact and summed in float32; each output is rounded once to
 * f16 after the activation.
 *   W_hat     [d_out, d_in] f16, row-major (row stride d_in): the
 *             dequantized layer (gptq_dequantize with GPTQ_F16 output).
 *   X         [d_in, n_tokens] f16 with row stride ldx (elements).
 *   Y         [d_out, n_tokens] f16 output with row stride ldy (elements);
 *             it must not overlap W_hat or X.
 *   activation 0: none; 1: max(0, .) (the pages name no nonlinearity).
 * d_in = 0 gives Y = act(0).  All pointers are device pointers owned by the
 * caller; the call is asynchronous on `stream`.
 * Errors: GPTQ_EINVAL (negative sizes, ldx or ldy below n_tokens, unknown
 * dtype or activation, null pointer), GPTQ_EUNSUPPORTED (a dtype other than
 * GPTQ_F16, d_out above 2^24, d_in above 2^22, ldx above 2^23, or 2^31 or
 * more 128 x 128 tiles of Y).
 */
int gptq_propagate(const void* W_hat, int w_dtype, int64_t d_out, int64_t d_in, const void* X, int x_dtype,
                   int64_t n_tokens, int64_t ldx, void* Y, int64_t ldy, int activation, void* stream);

/*
 * Greedy-order quantization of small layers (OBQ), the variant the fixed
 * column order replaces (aicassindra "Greedy quantization with error
 * compensation" and "GPTQ's speedups: fixed order and lazy batches";
 * mbrenndoerfer "Mathematical Details of the Update" for the Schur
 * downdate).  Per row, with Hf^-1 the inverse Hessian restricted to the
 * free weights (initially H_damped^-1 = U^T U): round every free weight to
 * the row's grid, quantize next the one with the smallest
 * e_q^2 / [Hf^-1]_qq (lowest index among equal scores), move the free
 * weights by -(e_q / [Hf^-1]_qq) Hf^-1[:, q], then
 * Hf^-1 -= Hf^-1[:, q] Hf^-1[q, :] / [Hf^-1]_qq.  The grid, the fp32 rounding
 * decision and the dead columns are those of gptq_quantize_layer with
 * group_size 0; the inverse and the weights are kept in float64.
 *   W          [d_out, d_in] of w_dtype, d_in <= 128.
 *   U          [d_in, d_in] float32 from gptq_prepare_hinv.
 *   dead       [d_in] uint8 or NULL.
 *   codes      [d_out, d_in] uint8 output; scales [d_out] float32 and
 *              zeros [d_out] int32 outputs (the per-row grid).
 *   order      [d_out, d_in] int32 output or NULL: the column quantized at
 *              each step.
 *   loss       [d_out] float64 output or NULL: the sum of the pick scores,
 *              equal to dw H_damped dw^T with dw = W0 - What.
 *   workspace  at least gptq_obq_workspace(d_in) bytes of device memory,
 *              256-byte aligned (H^-1 in float64).
 * Errors: GPTQ_EINVAL (negative sizes, bits outside [2, 8], unknown
 * w_dtype, null required pointer), GPTQ_EUNSUPPORTED (d_in above 128 or
 * d_out above 2^24), GPTQ_EWORKSPACE.  Empty inputs return GPTQ_OK.
 */
size_t gptq_obq_workspace(int64_t d_in);
int gptq_obq_quantize(const void* W, int w_dtype, int64_t d_out, int64_t d_in, const float* U, const uint8_t* dead,
                      int bits, uint8_t* codes, float* scales, int32_t* zeros, int32_t* order, double* loss,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a gptq_status value (static string). */
const char* gptq_status_string(int status);

/*
 * Kernel timing (measurement aid, not part of the method).
 * gptq_timing_enable(id) makes every later launch of kernel `id` (see
 * gptq_kernel_name) record a HIP event pair on its stream; id < 0 turns
 * timing off.  gptq_timing_read waits for the recorded events, returns the
 * summed duration in milliseconds and the launch count since the last read,
 * and resets them.  Host-side state, not thread-safe.
 */
int gptq_kernel_count(void);
const char* gptq_kernel_name(int id);
int gptq_timing_enable(int id);
int gptq_timing_read(double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
