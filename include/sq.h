/*
 * sq.h -- C ABI of the SmoothQuant W8A8 linear layer on MI355X (gfx950).
 *
 * The layer computes Y = X W^T with X [T x K] activations (T tokens, K input
 * channels) and W [N x K] weights (N output channels), rewritten exactly as
 *     Y = (X diag(s)^-1) (W diag(s))^T
 * (inferenceinterviews.com, "Why do activation outliers break INT8 W8A8 on
 * LLMs...", section "A strong answer"; maitreyasuin.github.io "...01-one-outlier",
 * section "Route it, or move it"), then quantises both smoothed operands to
 * symmetric int8 and multiplies them in integer arithmetic:
 *   - offline: per-input-channel smoothing factors s from column absolute maxima,
 *     W diag(s) quantised with one scale per output channel;
 *   - at run time: X diag(s)^-1 quantised with one scale per token, computed
 *     from the values present (dynamic), then an int8 x int8 -> int32 GEMM whose
 *     epilogue multiplies by the token scale times the channel scale;
 *   - or, coarser, one activation scale for the whole tensor, from its own
 *     range (dynamic) or from a calibrated range (static).
 *
 * Quantiser (maitreyasuin page, section "The four operations"): for one row v,
 * amax = max |v|; scale = amax / 127 (binary32 division); code =
 * clamp(round_half_even(v / scale), -127, 127).  -128 is never produced.  A row
 * with amax = 0 gets scale 1.0 and all codes 0.
 *
 * Conventions common to every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library
 *     never frees or retains them.  Matrices are row-major and contiguous: X and
 *     Xq are [T][K], W and Wq are [N][K] (K contiguous), Y is [T][N].
 *   - Work is enqueued on `stream` (0 = the null stream) and runs
 *     asynchronously; no call synchronises the stream or allocates device
 *     memory.  Outputs are valid once the stream reaches the enqueued work.
 *     Buffers that accumulate are cleared by kernels, not by memory-set
 *     commands, so a sequence of calls can be captured in a HIP graph and
 *     replayed (the graph replays the same pointers and sizes).
 *   - Arguments are validated on the host before anything is enqueued.  On any
 *     error other than SQ_ERR_HIP nothing is launched and no output is written.
 *     SQ_ERR_HIP means a kernel launch was rejected by the HIP runtime; outputs
 *     are then unspecified.
 *   - Calls are thread-safe.  The only library state is a per-device cache of
 *     device attributes.
 *   - NaN and infinite inputs are outside the contract.
 *   - Any T, N, K >= 1 is accepted.  Rows whose byte length is a multiple of 16
 *     with 16-byte aligned base pointers take the vectorised kernels; other
 *     shapes take slower scalar kernels with identical results.
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sq_status {
    SQ_OK = 0,
    SQ_ERR_NULL = 1,       /* a required pointer is NULL                         */
    SQ_ERR_SHAPE = 2,      /* a size is < 1, or K exceeds SQ_MAX_K for the GEMM  */
    SQ_ERR_ALPHA = 3,      /* alpha is NaN or outside [0, 1]                     */
    SQ_ERR_DTYPE = 4,      /* dtype not accepted for that argument               */
    SQ_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than required            */
    SQ_ERR_HIP = 6,        /* the HIP runtime rejected a launch                  */
    SQ_ERR_ARG = 7,        /* an argument value is not accepted (see the call)   */
    SQ_ERR_SCRATCH = 8     /* more scratch than the no-allocation call holds     */
} sq_status;

typedef enum sq_dtype {
    SQ_F32 = 0,            /* IEEE binary32                                      */
    SQ_BF16 = 1,           /* bfloat16 (upper half of a binary32)                */
    SQ_I32 = 2             /* int32; only as GEMM output: the raw accumulators   */
} sq_dtype;

/* Largest K for which 127 * 127 * K fits in int32, so the GEMM's int32
 * accumulators cannot overflow. */
#define SQ_MAX_K 133144

/* Human-readable name of a status code (static string, never NULL). */
const char *sq_status_string(sq_status status);

/*
 * Column absolute maximum of a [rows x cols] matrix:
 *     amax[j] = max_i |A[i][j]|            (or max(amax[j], that) if accumulate)
 * These are the statistics max_t |X_tj| and max_n |W_nj| of the smoothing factor
 * (inferenceinterviews page, "A strong answer"; maitreyasuin page, "Route it, or
 * move it").  accumulate = 1 keeps a running maximum across calls (calibration
 * over several batches); amax must then hold non-negative values already.
 *   A     device, a_t = SQ_F32 or SQ_BF16, [rows][cols]
 *   amax  device float [cols], written (read too if accumulate)
 */
sq_status sq_col_absmax(const void *A, sq_dtype a_t, int64_t rows, int64_t cols,
                        float *amax, int accumulate, hipStream_t stream);

/*
 * Smoothing factors from precomputed column maxima (multigrid.ai "SmoothQuant
 * Explained", section "Alpha: how much difficulty to move"; maxima clamped below
 * at 1e-8 as on the maitreyasuin page, "Route it, or move it"):
 *     s[j] = max(xa[j], 1e-8)^alpha / max(wa[j], 1e-8)^(1 - alpha)
 * evaluated in binary64 and rounded once to binary32; alpha = 0 gives exactly
 * 1 / max(wa, 1e-8) and alpha = 1 exactly max(xa, 1e-8).
 *   x_absmax, w_absmax  device float [K];   s  device float [K], written
 */
sq_status sq_smooth_scales_from_absmax(const float *x_absmax, const float *w_absmax,
                                       int64_t K, float alpha, float *s,
                                       hipStream_t stream);

/*
 * Smoothing factors from a calibration batch X [T x K] and the weights W [N x K]:
 * the two column maxima above followed by the formula above
 * (inferenceinterviews page, "A strong answer": s_j from max over t of |X_tj|
 * and max over n of |W_nj|).  The maxima are returned too when asked for.
 *   X         device, x_t = SQ_F32 or SQ_BF16, [T][K]
 *   W         device, w_t = SQ_F32 or SQ_BF16, [N][K]
 *   s         device float [K], written
 *   x_absmax  device float [K], written (max_t |X_tj|), or NULL: the maxima
 *             are then formed in s and replaced by the factors
 *   w_absmax  device float [K], written (max_n |W_nj|), or NULL: each
 *             workgroup then forms the maxima of a strip of columns over all of
 *             W and writes those columns' factors (no buffer, fewer workgroups:
 *             slower on wide W, the same s bit for bit)
 */
sq_status sq_smooth_scales(const void *X, sq_dtype x_t, int64_t T,
                           const void *W, sq_dtype w_t, int64_t N, int64_t K,
                           float alpha, float *s, float *x_absmax, float *w_absmax,
                           hipStream_t stream);

/*
 * Offline weight preparation: W_hat = W diag(s) (binary32 multiply), then one
 * symmetric int8 scale per output channel n (row of W):
 *     w_scale[n] = max_k |W_hat[n][k]| / 127,  Wq[n][k] = code of W_hat[n][k]
 * (inferenceinterviews page, "A strong answer": the weight input-columns absorb
 * s before quantisation; per-output-channel scales factor out of the sum,
 * maitreyasuin page, "Which scales factor out, and why").
 *   W        device, w_t = SQ_F32 or SQ_BF16, [N][K]
 *   s        device float [K], or NULL for no smoothing
 *   Wq       device int8 [N][K], written;  w_scale  device float [N], written
 */
sq_status sq_quantize_weights(const void *W, sq_dtype w_t, int64_t N, int64_t K,
                              const float *s, int8_t *Wq, float *w_scale,
                              hipStream_t stream);

/*
 * Dynamic per-token activation quantisation fused with the smoothing division:
 *     X_hat[t][k] = X[t][k] / s[k]          (binary32, correctly rounded)
 *     x_scale[t]  = max_k |X_hat[t][k]| / 127,  Xq[t][k] = code of X_hat[t][k]
 * (inferenceinterviews page, "A strong answer": divide activation channel j by
 * s_j; katajob.com "Why are activations harder to quantize...", section
 * "Activations are a distribution, not a tensor": dynamic per-token scales).
 * X is read once.
 *   X        device, x_t = SQ_F32 or SQ_BF16, [T][K]
 *   s        device float [K], or NULL if X is already smoothed (for example
 *            when 1/s was folded into the preceding normalisation gain)
 *   Xq       device int8 [T][K], written;  x_scale  device float [T], written
 */
sq_status sq_quant_act(const void *X, sq_dtype x_t, int64_t T, int64_t K,
                       const float *s, int8_t *Xq, float *x_scale, hipStream_t stream);

/*
 * Per-tensor activation range (multigrid.ai "SmoothQuant Explained", section
 * "Where it fits, and where it does not": the O2 and O3 levels quantise the
 * activations with one scale for the whole tensor, dynamic or static; katajob.com
 * "Why are activations harder to quantize...", section "Activations are a
 * distribution, not a tensor": static ranges are estimated during calibration
 * and frozen):
 *     amax[0] = max over all t, k of |X[t][k] / s[k]|      (binary32 quotients)
 * With accumulate = 1 the result is max(amax[0], that value), so a calibration
 * range can be gathered over several batches; with 0 the old value is ignored.
 *   X        device, x_t = SQ_F32 or SQ_BF16, [T][K]
 *   s        device float [K] (entries nonzero), or NULL for no smoothing
 *   amax     device float [1], written (read as well when accumulate = 1)
 */
sq_status sq_act_absmax(const void *X, sq_dtype x_t, int64_t T, int64_t K,
                        const float *s, float *amax, int accumulate, hipStream_t stream);

/*
 * Per-tensor activation quantisation against a given range, fused with the
 * smoothing division (maitreyasuin page, "The four operations": quantize_dequantize
 * with a clip; multigrid page, "Where it fits": the static level, which clips an
 * input beyond the calibrated range):
 *     X_hat[t][k] = X[t][k] / s[k]
 *     scale = clip[0] / 127 (binary32), or 1.0 when clip[0] = 0
 *     Xq[t][k] = clamp(round_half_even(X_hat[t][k] / scale), -127, 127)
 *                (every code is 0 when clip[0] = 0)
 *     x_scale[t] = scale for every t, so sq_w8a8_gemm applies unchanged
 * Values beyond the range clamp to +-127.  X is read once; no reduction.
 *   clip     device float [1]: a finite value >= 0 (for example a calibration
 *            range from sq_act_absmax); it is read by the kernels, so another
 *            value is outside the contract and is not diagnosed
 *   X, s, Xq as for sq_quant_act;  x_scale  device float [T], written
 */
sq_status sq_quant_act_static(const void *X, sq_dtype x_t, int64_t T, int64_t K,
                              const float *s, const float *clip, int8_t *Xq,
                              float *x_scale, hipStream_t stream);

/*
 * Dynamic per-tensor activation quantisation (the O2 level): sq_act_absmax of X
 * (accumulate = 0) into amax, then sq_quant_act_static with clip = amax.  X is
 * read twice (the scale depends on the whole tensor before any code exists).
 *   amax     device float [1], written with the tensor's range
 *   X, s, Xq, x_scale as for sq_quant_act_static
 */
sq_status sq_quant_act_per_tensor(const void *X, sq_dtype x_t, int64_t T, int64_t K,
                                  const float *s, float *amax, int8_t *Xq, float *x_scale,
                                  hipStream_t stream);

/* Normalisation in front of the layer. */
typedef enum sq_norm {
    SQ_NORM_RMS = 0,       /* RMSNorm: no centring, no bias  */
    SQ_NORM_LAYER = 1      /* LayerNorm: centring, optional bias */
} sq_norm;

/*
 * Fold the smoothing division into the preceding normalisation's per-channel
 * vector (multigrid.ai "SmoothQuant Explained", section "Why the rescaling is
 * free at runtime": divide the norm's weight vector elementwise by s; a
 * LayerNorm bias is folded the same way):  out[k] = v[k] / s[k]  (binary32).
 *   v, s     device float [K];  out  device float [K], written (may alias v)
 */
sq_status sq_fold_norm_gain(const float *v, const float *s, int64_t K, float *out,
                            hipStream_t stream);

/*
 * Normalisation fused with per-token int8 quantisation: the producer of a
 * smoothed W8A8 layer's input (multigrid page, "Why the rescaling is free at
 * runtime": with diag(s)^-1 folded into its gain the norm emits smoothed
 * activations; inferenceinterviews page, "A strong answer": 1/s_j folds into the
 * preceding RMSNorm gain).  The pages name the norms without writing them out;
 * the textbook forms are used, per token t:
 *   RMSNorm    rstd_t = 1 / sqrt(mean_k X[t][k]^2 + eps),  mean_t = 0
 *              h[t][k] = (X[t][k] * rstd_t) * gain[k]
 *   LayerNorm  mean_t = mean_k X[t][k],
 *              rstd_t = 1 / sqrt(mean_k (X[t][k] - mean_t)^2 + eps)
 *              h[t][k] = ((X[t][k] - mean_t) * rstd_t) * gain[k] + bias[k]
 * The statistics are rounded once to binary32 and are within 1e-6 relative of
 * their binary64 values (sums in binary64 except within 8-element chunks of
 * squares); h is binary32, one rounding per operation in the order written,
 * from those binary32 statistics.  Then h is
 * quantised exactly as sq_quant_act quantises X_hat (x_scale[t] = max_k |h| / 127,
 * scale 1 and codes 0 for a zero row).  X is read once; h is never stored.
 *   X          device, x_t = SQ_F32 or SQ_BF16, [T][K] (the norm's input)
 *   kind       SQ_NORM_RMS or SQ_NORM_LAYER
 *   gain       device float [K]: the norm's gain with 1/s folded in
 *              (sq_fold_norm_gain), or the plain gain for an unsmoothed layer
 *   bias       device float [K] or NULL (LayerNorm only, folded the same way)
 *   eps        finite, >= 0
 *   Xq         device int8 [T][K], written;  x_scale  device float [T], written
 *   mean, rstd device float [T] each, or NULL; written with the statistics
 * SQ_ERR_ARG: unknown kind, a bias with SQ_NORM_RMS, or eps negative / not finite.
 */
sq_status sq_norm_quant_act(const void *X, sq_dtype x_t, int64_t T, int64_t K, sq_norm kind,
                            const float *gain, const float *bias, float eps, int8_t *Xq,
                            float *x_scale, float *mean, float *rstd, hipStream_t stream);

/*
 * Mixed-precision decomposition, the alternative to smoothing (mercemay.com
 * "Activation Outlier Channels and Mixed-Precision Decomposition", section
 * "Decomposition: keep the outliers in high precision"; maitreyasuin page,
 * "Route it, or move it"): the sum over K splits into the bulk channels, run in
 * int8 with per-token / per-output-channel scales, and a few outlier channels
 * kept in binary32:
 *     Y[t][n] = fl32(acc_bulk[t][n] * fl32(x_scale[t] * w_scale[n]))
 *               + (sum over o ascending of X[t][idx[o]] * W[n][idx[o]], binary32)
 * The outlier set is static (chosen once from calibration).  The int8 operands
 * keep their full width with the outlier columns zeroed, so the bulk scales
 * ignore the outliers and the GEMM main loop is the ordinary one.  No smoothing
 * is applied on this path.
 *
 * sq_decomp_select: the n_o input channels with the largest absmax (for example
 * calibration column maxima from sq_col_absmax), ties to the lower index
 * (maitreyasuin page: dimensions ranked by max magnitude).
 *   absmax  device float [K];  0 <= n_o <= K
 *   idx     device int32 [n_o], written: the chosen channels, ascending
 *   mask    device float [K], written: 0 at the chosen channels, 1 elsewhere
 */
sq_status sq_decomp_select(const float *absmax, int64_t K, int64_t n_o, int32_t *idx, float *mask,
                           hipStream_t stream);

/*
 * Offline weight side: Wq = per-output-channel int8 of W with the outlier columns
 * zeroed (w_scale from the bulk columns only), W_out[o][n] = W[n][idx[o]] in
 * binary32 (bf16 widened exactly).
 *   W        device, w_t = SQ_F32 or SQ_BF16, [N][K]
 *   mask, idx, n_o   from sq_decomp_select (idx ascending, entries in [0, K);
 *            an entry outside that range reads as a zero column)
 *   Wq       device int8 [N][K], written;  w_scale  device float [N], written
 *   W_out    device float [n_o][N], written (may be NULL when n_o = 0)
 */
sq_status sq_decomp_prepare_weights(const void *W, sq_dtype w_t, int64_t N, int64_t K,
                                    const float *mask, const int32_t *idx, int64_t n_o,
                                    int8_t *Wq, float *w_scale, float *W_out, hipStream_t stream);

/*
 * Run-time activation side: Xq = per-token int8 of X with the outlier columns
 * zeroed (x_scale from the bulk columns only), X_out[o][t] = X[t][idx[o]] in
 * binary32.  X is read once by the quantiser; the outlier columns are gathered
 * by a second, small launch.
 *   X        device, x_t = SQ_F32 or SQ_BF16, [T][K]
 *   Xq       device int8 [T][K], written;  x_scale  device float [T], written
 *   X_out    device float [n_o][T], written (may be NULL when n_o = 0)
 */
sq_status sq_decomp_quant_act(const void *X, sq_dtype x_t, int64_t T, int64_t K,
                              const float *mask, const int32_t *idx, int64_t n_o,
                              int8_t *Xq, float *x_scale, float *X_out, hipStream_t stream);

/*
 * The decomposed layer's GEMM: sq_w8a8_gemm on the bulk operands with the
 * binary32 outlier product added in the epilogue (no second launch, no second
 * output pass).  y_t = SQ_F32 or SQ_BF16 (bf16 is the RNE rounding of the
 * binary32 sum).  X_out and W_out must be 16-byte aligned (SQ_ERR_ARG).
 */
sq_status sq_decomp_gemm(const int8_t *Xq, const float *x_scale, const int8_t *Wq,
                         const float *w_scale, const float *X_out, const float *W_out,
                         int64_t T, int64_t N, int64_t K, int64_t n_o, void *Y, sq_dtype y_t,
                         hipStream_t stream);

/*
 * FP8 E4M3 variant (inferenceinterviews page, "A strong answer", formats
 * paragraph: per-token FP8 activations keep about 3 mantissa bits whatever the
 * token's maximum).  The quantiser is the int8 one with the E4M3 grid:
 *     scale = amax / 448 (binary32), code = the E4M3 value nearest to v / scale
 *     (ties to the even code), saturated at +-448; scale 1 and codes 0 for a
 *     zero row.  E4M3 is the OCP format: bias 7, 3 mantissa bits, exponent
 *     field 0 for the subnormals m * 2^-9; codes 0x7F / 0xFF (NaN) never occur.
 * sq_quantize_weights_fp8: per output channel of W diag(s) (as sq_quantize_weights);
 * sq_quant_act_fp8: per token of X diag(s)^-1 (as sq_quant_act).
 *   Wq / Xq  device uint8 [N][K] / [T][K] of E4M3 codes, written
 */
sq_status sq_quantize_weights_fp8(const void *W, sq_dtype w_t, int64_t N, int64_t K,
                                  const float *s, uint8_t *Wq, float *w_scale, hipStream_t stream);
sq_status sq_quant_act_fp8(const void *X, sq_dtype x_t, int64_t T, int64_t K, const float *s,
                           uint8_t *Xq, float *x_scale, hipStream_t stream);

/*
 * FP8 GEMM:  acc[t][n] = sum_k e4m3(Xq[t][k]) * e4m3(Wq[n][k]),
 *            Y[t][n]   = fl32(acc * fl32(x_scale[t] * w_scale[n]))   (then bf16 RNE)
 * on the FP8 matrix cores (binary32 accumulation).  Every product of two E4M3
 * values is exact, but the hardware sums them at less than full binary32
 * precision when their magnitudes differ widely, so acc is not the exact sum:
 * it is within 2^-10 * sum_k |products| of it (a measured property of the
 * instruction; the exact sum is the reference).  y_t = SQ_F32 or SQ_BF16;
 * K <= SQ_MAX_K as for sq_w8a8_gemm.
 */
sq_status sq_fp8_gemm(const uint8_t *Xq, const float *x_scale, const uint8_t *Wq,
                      const float *w_scale, int64_t T, int64_t N, int64_t K, void *Y,
                      sq_dtype y_t, hipStream_t stream);

/*
 * W8A8 GEMM with int32 accumulation and the dequantising epilogue
 * (mercemay.com "Activation Outlier Channels and Mixed-Precision Decomposition",
 * section "Decomposition": integer matmul, float epilogue multiplying by the
 * product of the two scales; maitreyasuin page, "Which scales factor out"):
 *     acc[t][n] = sum_k Xq[t][k] * Wq[n][k]                (exact int32)
 *     Y[t][n]   = fl32( fl32(acc[t][n]) * fl32(x_scale[t] * w_scale[n]) )
 * y_t = SQ_F32 stores that value; SQ_BF16 stores it rounded to nearest-even
 * bfloat16; SQ_I32 stores acc itself (x_scale and w_scale may then be NULL).
 * Requires K <= SQ_MAX_K.
 *   Xq  device int8 [T][K];  Wq  device int8 [N][K];  Y  device [T][N], written
 */
sq_status sq_w8a8_gemm(const int8_t *Xq, const float *x_scale,
                       const int8_t *Wq, const float *w_scale,
                       int64_t T, int64_t N, int64_t K, void *Y, sq_dtype y_t,
                       hipStream_t stream);

/* Bytes of device workspace sq_w8a8_linear needs for T tokens of width K
 * (the int8 codes and the per-token scales, each 256-byte aligned); 0 when
 * T or K is below 1, SIZE_MAX when the size does not fit a size_t. */
size_t sq_w8a8_linear_workspace_size(int64_t T, int64_t K);

/*
 * The run-time layer: sq_quant_act of X with s into the workspace, then
 * sq_w8a8_gemm against the prepared weights, on one stream.
 *   X          device, x_t = SQ_F32 or SQ_BF16, [T][K]
 *   s          device float [K] or NULL (as for sq_quant_act)
 *   Wq, w_scale  from sq_quantize_weights
 *   Y          device [T][N] of y_t = SQ_F32 or SQ_BF16, written
 *   workspace  device memory of at least sq_w8a8_linear_workspace_size(T, K)
 *              bytes, 256-byte aligned; the caller must not touch it until the
 *              stream has passed this call
 */
sq_status sq_w8a8_linear(const void *X, sq_dtype x_t, const float *s,
                         const int8_t *Wq, const float *w_scale,
                         int64_t T, int64_t N, int64_t K, void *Y, sq_dtype y_t,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of the library's fixed per-GPU scratch used by sq_w8a8_linear_noalloc. */
#define SQ_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * sq_w8a8_linear with the workspace taken from a fixed array of
 * SQ_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on, from
 * the first such call until the process ends.  The call allocates nothing; the
 * caller passes inputs and outputs as for sq_w8a8_linear, and the results are
 * bit for bit those of sq_w8a8_linear.
 *   SQ_ERR_SCRATCH  sq_w8a8_linear_workspace_size(T, K) exceeds
 *                   SQ_NOALLOC_SCRATCH_BYTES (T * K up to ~32 M int8 codes);
 *                   nothing is launched
 *   SQ_ERR_HIP      also when the scratch's address cannot be obtained
 * Every call on one GPU uses the same scratch: calls that overlap on one GPU
 * (other streams, other host threads) race and must be ordered by the caller.
 * Nothing in the scratch needs to start at zero (each call writes the codes
 * and scales before its GEMM reads them).
 */
sq_status sq_w8a8_linear_noalloc(const void *X, sq_dtype x_t, const float *s,
                                 const int8_t *Wq, const float *w_scale,
                                 int64_t T, int64_t N, int64_t K, void *Y, sq_dtype y_t,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SQ_H */
