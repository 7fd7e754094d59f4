/*
 * sq_oracle.c -- plain, slow CPU reference of the SmoothQuant W8A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or run
 * this file; only the tests, the smoke check and the benchmark's CPU baseline
 * use it.  It shares no code, header or constant with the HIP library.
 *
 * Every step is the plain definition, written with ordinary loops, in the order
 * the pages give it.  Floating point is IEEE binary32 wherever the layer's
 * contract fixes fp32 (scales, smoothed values, the dequantised output); the
 * smoothing factor is evaluated in binary64 and rounded once.  Build with
 *   gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp
 * so that each C operator is exactly one correctly rounded IEEE operation.
 *
 * Sources (pages as they are titled; sections / equations named):
 *   [P2] multigrid.ai "SmoothQuant Explained", section "Alpha: how much
 *        difficulty to move" (the s_j formula and its alpha = 0 / 1 forms).
 *   [P3] inferenceinterviews.com "Why do activation outliers break INT8 W8A8 on
 *        LLMs...", section "A strong answer" (the identity
 *        XW^T = (X diag(s)^-1)(W diag(s))^T, the s_j formula with max over
 *        tokens t and output rows n, per-token and per-output-channel scales
 *        applied in the epilogue).
 *   [P4] mercemay.com "Activation Outlier Channels and Mixed-Precision
 *        Decomposition", section "Decomposition" (integer matmul followed by a
 *        float epilogue that multiplies by the product of the two scales).
 *   [P5] maitreyasuin.github.io "...01-one-outlier", sections "The four
 *        operations" (q = clamp(round(x/s), -n, n), scale = limit/n, n = 127,
 *        round then clamp, the all-zero case gives codes 0 and scale 1),
 *        "Which scales factor out, and why" (Y_tn = sum_k X_tk W_nk with
 *        W_nk = s_n Q_nk and X_tk = a_t P_tk) and "Route it, or move it"
 *        (maxima clamped below at 1e-8 before the powers).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SQO_N 127        /* [P5] n = 2^(bits-1) - 1 for 8 bits                 */
#define SQO_EPS 1e-8f    /* [P5] "Route it, or move it": clamp_min(eps) on maxima */

/* Column absolute maximum: out[j] = max_i |A[i][j]|.  [P3] max_t |X_tj| and
 * max_n |W_nj|; [P5] amax over dim 0 of act and of the weights. */
void sqo_col_absmax(const float *A, int64_t rows, int64_t cols, float *out)
{
    for (int64_t j = 0; j < cols; ++j) out[j] = 0.0f;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) {
            float a = fabsf(A[i * cols + j]);
            if (a > out[j]) out[j] = a;
        }
}

/* Smoothing factor.  [P2]/[P3]: s_j = max|X_j|^alpha / max|W_j|^(1-alpha);
 * [P5]: both maxima clamped below at 1e-8 first.  Evaluated in binary64 and
 * rounded once to binary32.  pow(x, 0) = 1 and pow(x, 1) = x exactly (C99
 * Annex F), which gives the alpha = 0 and alpha = 1 forms of [P2]. */
void sqo_smooth_scales(const float *xa, const float *wa, int64_t K, float alpha, float *s)
{
    double a = (double)alpha;
    for (int64_t j = 0; j < K; ++j) {
        float x = xa[j] < SQO_EPS ? SQO_EPS : xa[j];
        float w = wa[j] < SQO_EPS ? SQO_EPS : wa[j];
        double num = pow((double)x, a);
        double den = pow((double)w, 1.0 - a);
        s[j] = (float)(num / den);
    }
}

/* [P5] "The four operations": code = clamp(round(v / scale), -n, n), with
 * round = nearest, ties to even (torch.round and np.round both do this). */
static int8_t code_of(float v, float scale)
{
    float q = rintf(v / scale);               /* default mode: ties to even   */
    if (q > (float)SQO_N) q = (float)SQO_N;   /* round first, then clamp      */
    if (q < -(float)SQO_N) q = -(float)SQO_N;
    return (int8_t)q;
}

/* Quantise one row of `len` smoothed values: scale = amax / 127; amax = 0 gives
 * scale 1 and all codes 0 ([P5] zero-range case). */
static void quantize_row(const float *v, int64_t len, int8_t *q, float *scale)
{
    float amax = 0.0f;
    for (int64_t k = 0; k < len; ++k) {
        float a = fabsf(v[k]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *scale = 1.0f;
        for (int64_t k = 0; k < len; ++k) q[k] = 0;
        return;
    }
    float sc = amax / (float)SQO_N;
    *scale = sc;
    for (int64_t k = 0; k < len; ++k) q[k] = code_of(v[k], sc);
}

/* Offline weight preparation.  [P3]: multiply weight input-column j by s_j
 * (W_hat = W diag(s)), then quantise per output channel (one scale per row n of
 * W [N x K]).  s == NULL means no smoothing. */
void sqo_quantize_weights(const float *W, int64_t N, int64_t K, const float *s,
                          int8_t *Wq, float *w_scale)
{
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k)
                row[k] = s ? W[n * K + k] * s[k] : W[n * K + k];
            quantize_row(row, K, Wq + n * K, w_scale + n);
        }
        free(row);
    }
}

/* Dynamic per-token activation quantisation.  [P3]: divide activation channel j
 * by s_j (X_hat = X diag(s)^-1); then one scale per token (row t of X [T x K]).
 * s == NULL means the input is already smoothed. */
void sqo_quant_act(const float *X, int64_t T, int64_t K, const float *s,
                   int8_t *Xq, float *x_scale)
{
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t k = 0; k < K; ++k)
                row[k] = s ? X[t * K + k] / s[k] : X[t * K + k];
            quantize_row(row, K, Xq + t * K, x_scale + t);
        }
        free(row);
    }
}

/* Per-tensor activation range.  [P2] "Where it fits, and where it does not":
 * the O2 and O3 levels quantise the activations with one scale for the whole
 * tensor, found from the values present (dynamic) or from calibration and then
 * frozen (static); [P1] "Activations are a distribution, not a tensor" (static
 * ranges come from calibration, dynamic ones cost a reduction over the tensor).
 * amax = max over every t, k of |X_tk / s_k|: one IEEE division per element. */
float sqo_act_tensor_absmax(const float *X, int64_t T, int64_t K, const float *s)
{
    float amax = 0.0f;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t k = 0; k < K; ++k) {
            float v = s ? X[t * K + k] / s[k] : X[t * K + k];
            float a = fabsf(v);
            if (a > amax) amax = a;
        }
    return amax;
}

/* Per-tensor quantisation against a given range `clip`.  [P5] "The four
 * operations", quantize_dequantize with its clip argument: scale = clip / n,
 * code = clamp(round(v / scale), -n, n), so values beyond the range clamp to
 * +-127; a zero range gives codes 0 and scale 1.  v = X_tk / s_k as for the
 * per-token case.  Every token carries the same scale (x_scale[t] = scale for
 * all t), so the per-token epilogue applies unchanged. */
void sqo_quant_act_static(const float *X, int64_t T, int64_t K, const float *s, float clip,
                          int8_t *Xq, float *x_scale)
{
    if (clip == 0.0f) {
        for (int64_t t = 0; t < T; ++t) x_scale[t] = 1.0f;
        memset(Xq, 0, (size_t)(T * K));
        return;
    }
    float sc = clip / (float)SQO_N;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            float v = s ? X[t * K + k] / s[k] : X[t * K + k];
            Xq[t * K + k] = code_of(v, sc);
        }
        x_scale[t] = sc;
    }
}

/* Folding the smoothing division into the preceding normalisation.  [P2] "Why
 * the rescaling is free at runtime": divide the norm's per-channel weight vector
 * elementwise by s, so the norm emits already-smoothed activations; [P3] "A
 * strong answer": 1/s_j folds into the preceding RMSNorm gain.  A LayerNorm's
 * bias is divided the same way (it is added after the gain, so it must carry the
 * same 1/s).  out[k] = in[k] / s[k], one IEEE division. */
void sqo_fold_gain(const float *in, const float *s, int64_t K, float *out)
{
    for (int64_t k = 0; k < K; ++k) out[k] = in[k] / s[k];
}

/* Per-token statistics of the normalisation that precedes the linear layer.
 * The pages name RMSNorm and LayerNorm but do not write them out; the textbook
 * definitions are used:
 *   RMSNorm   rstd_t = 1 / sqrt(mean_k x_tk^2 + eps)                (mean_t = 0)
 *   LayerNorm mean_t = mean_k x_tk,  rstd_t = 1 / sqrt(mean_k (x_tk - mean_t)^2 + eps)
 * Sums and the square root in binary64 (two passes for the variance), each
 * statistic rounded once to binary32. */
void sqo_norm_stats(const float *X, int64_t T, int64_t K, int layer, float eps,
                    float *mean, float *rstd)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *x = X + t * K;
        double mu = 0.0;
        if (layer) {
            for (int64_t k = 0; k < K; ++k) mu += (double)x[k];
            mu /= (double)K;
        }
        double v = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double d = (double)x[k] - mu;
            v += d * d;
        }
        v /= (double)K;
        mean[t] = (float)mu;
        rstd[t] = (float)(1.0 / sqrt(v + (double)eps));
    }
}

/* Normalised, gained activations in binary32, one rounding per operation, in
 * the order the definitions read (centre, scale by rstd, multiply by the gain,
 * add the bias):
 *   RMSNorm   h = (x * rstd) * gain
 *   LayerNorm h = ((x - mean) * rstd) * gain + bias      (bias may be NULL)
 * With the smoothing folded into gain and bias, h is the smoothed activation
 * that the per-token quantiser takes. */
void sqo_norm_apply(const float *X, int64_t T, int64_t K, int layer, const float *mean,
                    const float *rstd, const float *gain, const float *bias, float *H)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            float x = X[t * K + k];
            float c = layer ? x - mean[t] : x;
            float n = c * rstd[t];
            float h = n * gain[k];
            if (layer && bias) h = h + bias[k];
            H[t * K + k] = h;
        }
    }
}

/* Mixed-precision decomposition ([P4] "Decomposition: keep the outliers in
 * high precision"; [P5] "Route it, or move it": the sum over K splits into the
 * ordinary dimensions, run in int8, and the outlier dimensions, kept in full
 * precision).  The outlier set is static, chosen once from calibration ([P4]:
 * determined once and stored with the weights) as the n_o input channels with
 * the largest absolute maximum ([P5]: dimensions ranked by max magnitude); ties
 * go to the lower index.  Output: the chosen indices in ascending order. */
static const float *g_sel_key;
static int cmp_sel(const void *a, const void *b)
{
    int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
    if (g_sel_key[i] > g_sel_key[j]) return -1;
    if (g_sel_key[i] < g_sel_key[j]) return 1;
    return (i > j) - (i < j);
}
static int cmp_i32(const void *a, const void *b)
{
    int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
    return (i > j) - (i < j);
}
void sqo_decomp_select(const float *absmax, int64_t K, int64_t n_o, int32_t *idx)
{
    int32_t *ord = (int32_t *)malloc((size_t)K * sizeof(int32_t));
    for (int64_t k = 0; k < K; ++k) ord[k] = (int32_t)k;
    g_sel_key = absmax;
    qsort(ord, (size_t)K, sizeof(int32_t), cmp_sel);
    for (int64_t o = 0; o < n_o; ++o) idx[o] = ord[o];
    qsort(idx, (size_t)n_o, sizeof(int32_t), cmp_i32);
    free(ord);
}

/* The ordinary ("bulk") columns of A [rows x K], in order, and the outlier
 * columns listed in idx, as two compact matrices ([P4]: x[keep], x[outlier_idx]). */
void sqo_decomp_split(const float *A, int64_t rows, int64_t K, const int32_t *idx, int64_t n_o,
                      float *bulk, float *outl)
{
    for (int64_t r = 0; r < rows; ++r) {
        int64_t o = 0, b = 0;
        for (int64_t k = 0; k < K; ++k) {
            if (o < n_o && idx[o] == k) outl[r * n_o + o++] = A[r * K + k];
            else bulk[r * (K - n_o) + b++] = A[r * K + k];
        }
    }
}

/* The full-precision part: y_out[t][n] = sum over o (ascending) of
 * Xo[t][o] * Wo[n][o], binary32, one rounding per multiply and per add, from 0. */
void sqo_decomp_outlier_product(const float *Xo, const float *Wo, int64_t T, int64_t N, int64_t n_o,
                                float *Yo)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            float acc = 0.0f;
            for (int64_t o = 0; o < n_o; ++o) {
                float p = Xo[t * n_o + o] * Wo[n * n_o + o];
                acc = acc + p;
            }
            Yo[t * N + n] = acc;
        }
}

/* y = y_bulk + y_out, one binary32 addition. */
void sqo_add(const float *a, const float *b, int64_t n, float *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = a[i] + b[i];
}

/* FP8 variant ([P3] "A strong answer", the formats paragraph: per-token FP8
 * E4M3 activations keep about 3 mantissa bits of relative precision whatever the
 * token's maximum, so smoothing matters less there).  The page does not write
 * the FP8 quantiser out; the reading used is the int8 round trip with the E4M3
 * grid in place of the integers: scale = amax / 448 (448 is the largest finite
 * E4M3 value), code = the E4M3 value nearest to v / scale (ties to even mantissa),
 * saturated to +-448; an all-zero row gets scale 1 and codes 0.
 *
 * E4M3 (OCP FP8): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent field 0 holds the subnormals m * 2^-9; 0x7F / 0xFF are NaN (never
 * produced).  Decoding is exact in binary32. */
static float e4m3_value(int e, int m)
{
    return e == 0 ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
}

uint8_t sqo_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    float a = fabsf(v);
    if (a >= 448.0f) return sign | 0x7E;
    /* the E4M3 neighbours below and above a, found by walking the grid */
    int best = 0;
    for (int c = 1; c <= 0x7E; ++c) {
        float x = e4m3_value(c >> 3, c & 7);
        if (x <= a) best = c;
        else break;
    }
    float lo = e4m3_value(best >> 3, best & 7);
    if (lo == a || best == 0x7E) return sign | (uint8_t)best;
    int up = best + 1;
    float hi = e4m3_value(up >> 3, up & 7);
    double dl = (double)a - (double)lo, dh = (double)hi - (double)a;
    int pick = dl < dh ? best : dh < dl ? up : ((best & 1) ? up : best);   /* tie: even code */
    return sign | (uint8_t)pick;
}

float sqo_e4m3_decode(uint8_t c)
{
    float v = e4m3_value((c >> 3) & 15, c & 7);
    return (c & 0x80) ? -v : v;
}

/* One row of smoothed values -> E4M3 codes and the row scale. */
static void quantize_row_fp8(const float *v, int64_t len, uint8_t *q, float *scale)
{
    float amax = 0.0f;
    for (int64_t k = 0; k < len; ++k) {
        float a = fabsf(v[k]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *scale = 1.0f;
        for (int64_t k = 0; k < len; ++k) q[k] = 0;
        return;
    }
    float sc = amax / 448.0f;
    *scale = sc;
    for (int64_t k = 0; k < len; ++k) q[k] = sqo_e4m3_encode(v[k] / sc);
}

/* FP8 counterparts of sqo_quantize_weights (W diag(s), per output channel) and
 * sqo_quant_act (X diag(s)^-1, per token). */
void sqo_quantize_weights_fp8(const float *W, int64_t N, int64_t K, const float *s,
                              uint8_t *Wq, float *w_scale)
{
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k)
                row[k] = s ? W[n * K + k] * s[k] : W[n * K + k];
            quantize_row_fp8(row, K, Wq + n * K, w_scale + n);
        }
        free(row);
    }
}

void sqo_quant_act_fp8(const float *X, int64_t T, int64_t K, const float *s,
                       uint8_t *Xq, float *x_scale)
{
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t k = 0; k < K; ++k)
                row[k] = s ? X[t * K + k] / s[k] : X[t * K + k];
            quantize_row_fp8(row, K, Xq + t * K, x_scale + t);
        }
        free(row);
    }
}

/* Exact dot products of decoded E4M3 codes at the listed (t, n) pairs: every
 * product has at most 8 significant bits and lies in [2^-18, 448^2], so a
 * binary64 sum of up to 2^16 of them is exact; also the sum of |products|. */
void sqo_fp8_dot_at(const uint8_t *Xq, const uint8_t *Wq, int64_t K, const int64_t *ti,
                    const int64_t *ni, int64_t count, double *acc, double *acc_abs)
{
    float lut[256];
    for (int c = 0; c < 256; ++c) lut[c] = sqo_e4m3_decode((uint8_t)c);
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < count; ++p) {
        const uint8_t *x = Xq + ti[p] * K, *w = Wq + ni[p] * K;
        double sum = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double pr = (double)lut[x[k]] * (double)lut[w[k]];
            sum += pr;
            sa += fabs(pr);
        }
        acc[p] = sum;
        acc_abs[p] = sa;
    }
}

/* Integer matmul.  [P5] "Which scales factor out": acc_tn = sum_k P_tk Q_nk.
 * Accumulated in int64; returns 1 if any sum does not fit int32, else 0. */
int sqo_int_gemm(const int8_t *Xq, const int8_t *Wq, int64_t T, int64_t N, int64_t K,
                 int32_t *acc)
{
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int64_t)Xq[t * K + k] * (int64_t)Wq[n * K + k];
            if (sum > INT32_MAX || sum < INT32_MIN) overflow = 1;
            acc[t * N + n] = (int32_t)sum;
        }
    return overflow;
}

/* The same sums for a list of (t, n) pairs only (for problems too large to
 * multiply out on the CPU). */
int sqo_int_gemm_at(const int8_t *Xq, const int8_t *Wq, int64_t K, const int64_t *ti,
                    const int64_t *ni, int64_t count, int32_t *acc)
{
    int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
    for (int64_t i = 0; i < count; ++i) {
        int64_t sum = 0;
        for (int64_t k = 0; k < K; ++k)
            sum += (int64_t)Xq[ti[i] * K + k] * (int64_t)Wq[ni[i] * K + k];
        if (sum > INT32_MAX || sum < INT32_MIN) overflow = 1;
        acc[i] = (int32_t)sum;
    }
    return overflow;
}

/* Dequantising epilogue.  [P4] "integer matmul, float epilogue": the integer
 * result times (sx * sw); [P3] per-token and per-output-channel scales applied
 * in the epilogue.  y = fl32( fl32(acc) * fl32(x_scale[t] * w_scale[n]) ). */
void sqo_dequant(const int32_t *acc, const float *x_scale, const float *w_scale,
                 int64_t T, int64_t N, float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            float sxw = x_scale[t] * w_scale[n];
            y[t * N + n] = (float)acc[t * N + n] * sxw;
        }
}

/* Same epilogue for a list of pairs (acc[i] belongs to (ti[i], ni[i])). */
void sqo_dequant_at(const int32_t *acc, const float *x_scale, const float *w_scale,
                    const int64_t *ti, const int64_t *ni, int64_t count, float *y)
{
    for (int64_t i = 0; i < count; ++i) {
        float sxw = x_scale[ti[i]] * w_scale[ni[i]];
        y[i] = (float)acc[i] * sxw;
    }
}

/* binary32 -> bfloat16, round to nearest, ties to even (finite inputs). */
void sqo_to_bf16(const float *y, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &y[i], sizeof u);
        uint32_t lower = u & 0xFFFFu;
        uint32_t upper = u >> 16;
        if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
        out[i] = (uint16_t)upper;
    }
}
