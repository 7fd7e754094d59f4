/*
 * Driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the CPU
 * oracle (test infrastructure, CPU only): every entry point of oracle/sq_oracle.c
 * on small, ragged and degenerate shapes (one row, one column, zero rows and
 * columns, ties, every FP8 code), so that an out-of-bounds index, an overflowing
 * integer or a misaligned access in the oracle fails under the sanitizers.
 * Prints "ok" and exits 0 when every call finished.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void sqo_col_absmax(const float *A, int64_t rows, int64_t cols, float *out);
void sqo_smooth_scales(const float *xa, const float *wa, int64_t K, float alpha, float *s);
void sqo_quantize_weights(const float *W, int64_t N, int64_t K, const float *s, int8_t *Wq, float *ws);
void sqo_quant_act(const float *X, int64_t T, int64_t K, const float *s, int8_t *Xq, float *xs);
float sqo_act_tensor_absmax(const float *X, int64_t T, int64_t K, const float *s);
void sqo_quant_act_static(const float *X, int64_t T, int64_t K, const float *s, float clip, int8_t *Xq,
                          float *xs);
void sqo_fold_gain(const float *in, const float *s, int64_t K, float *out);
void sqo_norm_stats(const float *X, int64_t T, int64_t K, int layer, float eps, float *mean, float *rstd);
void sqo_norm_apply(const float *X, int64_t T, int64_t K, int layer, const float *mean, const float *rstd,
                    const float *gain, const float *bias, float *H);
void sqo_decomp_select(const float *absmax, int64_t K, int64_t n_o, int32_t *idx);
void sqo_decomp_split(const float *A, int64_t rows, int64_t K, const int32_t *idx, int64_t n_o, float *bulk,
                      float *outl);
void sqo_decomp_outlier_product(const float *Xo, const float *Wo, int64_t T, int64_t N, int64_t n_o, float *Yo);
void sqo_add(const float *a, const float *b, int64_t n, float *out);
uint8_t sqo_e4m3_encode(float v);
float sqo_e4m3_decode(uint8_t c);
void sqo_quantize_weights_fp8(const float *W, int64_t N, int64_t K, const float *s, uint8_t *Wq, float *ws);
void sqo_quant_act_fp8(const float *X, int64_t T, int64_t K, const float *s, uint8_t *Xq, float *xs);
void sqo_fp8_dot_at(const uint8_t *Xq, const uint8_t *Wq, int64_t K, const int64_t *ti, const int64_t *ni,
                    int64_t count, double *acc, double *acc_abs);
int sqo_int_gemm(const int8_t *Xq, const int8_t *Wq, int64_t T, int64_t N, int64_t K, int32_t *acc);
int sqo_int_gemm_at(const int8_t *Xq, const int8_t *Wq, int64_t K, const int64_t *ti, const int64_t *ni,
                    int64_t count, int32_t *acc);
void sqo_dequant(const int32_t *acc, const float *x_scale, const float *w_scale, int64_t T, int64_t N,
                 float *y);
void sqo_dequant_at(const int32_t *acc, const float *x_scale, const float *w_scale, const int64_t *ti,
                    const int64_t *ni, int64_t count, float *y);
void sqo_to_bf16(const float *y, int64_t n, uint16_t *out);

/* exact-size heap buffers, so that a read or write one past the end is caught */
static void *buf(size_t bytes) { return malloc(bytes ? bytes : 1); }

static float frand(unsigned *state) {
    *state = *state * 1664525u + 1013904223u;
    return ((float)(*state >> 8) / 16777216.0f - 0.5f) * 8.0f;
}

static void run_shape(int64_t T, int64_t N, int64_t K, unsigned seed) {
    unsigned st = seed;
    float *X = buf(sizeof(float) * T * K), *W = buf(sizeof(float) * N * K);
    for (int64_t i = 0; i < T * K; ++i) X[i] = frand(&st);
    for (int64_t i = 0; i < N * K; ++i) W[i] = 0.02f * frand(&st);
    if (T > 1) memset(X, 0, sizeof(float) * K);            /* an all-zero token */
    if (N > 1) memset(W + K, 0, sizeof(float) * K);        /* an all-zero output channel */
    if (K > 1) for (int64_t t = 0; t < T; ++t) X[t * K + K - 1] = 0.0f;   /* an all-zero column */

    float *xa = buf(sizeof(float) * K), *wa = buf(sizeof(float) * K), *s = buf(sizeof(float) * K);
    sqo_col_absmax(X, T, K, xa);
    sqo_col_absmax(W, N, K, wa);
    sqo_smooth_scales(xa, wa, K, 0.5f, s);
    sqo_smooth_scales(xa, wa, K, 0.0f, s);
    sqo_smooth_scales(xa, wa, K, 1.0f, s);
    sqo_smooth_scales(xa, wa, K, 0.75f, s);

    int8_t *Wq = buf(N * K), *Xq = buf(T * K);
    float *ws = buf(sizeof(float) * N), *xs = buf(sizeof(float) * T);
    sqo_quantize_weights(W, N, K, s, Wq, ws);
    sqo_quantize_weights(W, N, K, NULL, Wq, ws);
    sqo_quant_act(X, T, K, NULL, Xq, xs);
    sqo_quant_act(X, T, K, s, Xq, xs);
    float amax = sqo_act_tensor_absmax(X, T, K, s);
    sqo_act_tensor_absmax(X, T, K, NULL);
    int8_t *Xq2 = buf(T * K);
    float *xs2 = buf(sizeof(float) * T);
    sqo_quant_act_static(X, T, K, s, amax, Xq2, xs2);
    sqo_quant_act_static(X, T, K, s, 0.0f, Xq2, xs2);

    int32_t *acc = buf(sizeof(int32_t) * T * N);
    float *y = buf(sizeof(float) * T * N);
    uint16_t *yb = buf(sizeof(uint16_t) * T * N);
    if (sqo_int_gemm(Xq, Wq, T, N, K, acc)) { printf("int32 overflow flagged\n"); exit(1); }
    sqo_dequant(acc, xs, ws, T, N, y);
    sqo_to_bf16(y, T * N, yb);
    int64_t ti[3] = {0, T - 1, T / 2}, ni[3] = {N - 1, 0, N / 2};
    int32_t acc3[3];
    float y3[3];
    sqo_int_gemm_at(Xq, Wq, K, ti, ni, 3, acc3);
    sqo_dequant_at(acc3, xs, ws, ti, ni, 3, y3);

    float *g = buf(sizeof(float) * K), *b = buf(sizeof(float) * K), *gf = buf(sizeof(float) * K);
    for (int64_t k = 0; k < K; ++k) { g[k] = 1.0f + 0.1f * frand(&st); b[k] = 0.1f * frand(&st); }
    sqo_fold_gain(g, s, K, gf);
    float *mean = buf(sizeof(float) * T), *rstd = buf(sizeof(float) * T), *H = buf(sizeof(float) * T * K);
    for (int layer = 0; layer < 2; ++layer) {
        sqo_norm_stats(X, T, K, layer, 1e-6f, mean, rstd);
        sqo_norm_apply(X, T, K, layer, mean, rstd, gf, layer ? b : NULL, H);
    }

    for (int64_t n_o = 0; n_o <= K; n_o += (K > 3 ? K / 3 : 1)) {
        int32_t *idx = buf(sizeof(int32_t) * n_o);
        sqo_decomp_select(xa, K, n_o, idx);
        float *xb = buf(sizeof(float) * T * (K - n_o)), *xo = buf(sizeof(float) * T * n_o);
        float *wb = buf(sizeof(float) * N * (K - n_o)), *wo = buf(sizeof(float) * N * n_o);
        sqo_decomp_split(X, T, K, idx, n_o, xb, xo);
        sqo_decomp_split(W, N, K, idx, n_o, wb, wo);
        float *yo = buf(sizeof(float) * T * N), *ys = buf(sizeof(float) * T * N);
        sqo_decomp_outlier_product(xo, wo, T, N, n_o, yo);
        sqo_add(y, yo, T * N, ys);
        free(idx); free(xb); free(xo); free(wb); free(wo); free(yo); free(ys);
    }

    uint8_t *Wq8 = buf(N * K), *Xq8 = buf(T * K);
    sqo_quantize_weights_fp8(W, N, K, s, Wq8, ws);
    sqo_quant_act_fp8(X, T, K, s, Xq8, xs);
    sqo_quant_act_fp8(X, T, K, NULL, Xq8, xs);
    double d3[3], a3[3];
    sqo_fp8_dot_at(Xq8, Wq8, K, ti, ni, 3, d3, a3);

    free(X); free(W); free(xa); free(wa); free(s); free(Wq); free(Xq); free(ws); free(xs); free(Xq2);
    free(xs2); free(acc); free(y); free(yb); free(g); free(b); free(gf); free(mean); free(rstd); free(H);
    free(Wq8); free(Xq8);
}

int main(void) {
    /* every FP8 code and its neighbours through the codec */
    for (int c = 0; c < 256; ++c) {
        if ((c & 0x7F) == 0x7F) continue;
        float v = sqo_e4m3_decode((uint8_t)c);
        if (sqo_e4m3_encode(v) != (uint8_t)c && !(v == 0.0f)) { printf("codec mismatch at %d\n", c); return 1; }
    }
    sqo_e4m3_encode(1e30f);
    sqo_e4m3_encode(-1e-30f);
    const int64_t shapes[][3] = {{1, 1, 1}, {1, 3, 17}, {3, 1, 16}, {37, 45, 80}, {5, 7, 83}, {64, 3, 1040}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
        run_shape(shapes[i][0], shapes[i][1], shapes[i][2], 17u + (unsigned)i);
    printf("ok\n");
    return 0;
}
