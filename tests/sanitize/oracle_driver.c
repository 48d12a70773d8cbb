/* Test driver for the CPU oracle built with sanitizers (ASan + UBSan, or
 * TSan): every result buffer is allocated at its exact size, the
 * multi-threaded paths run with 3 threads, the full and sampled forms are
 * cross-checked, the exact zero-weight closed form is checked, and every
 * invalid-argument path is exercised.  Exit status 0 = all checks passed. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_conv2d_sizes(long H, long W, long K, long pool, long *Hc, long *Wc, long *PH, long *PW);
int oracle_conv2d_pool_sigmoid_sum(const float *x, long B, long Cin, long H, long W, const float *w, long Cout,
                                   long K, const float *bias, long pool, const long *batch_idx, long nb, double *out,
                                   double *part, double *pooled, int nthreads);
int oracle_conv2d_pooled_at(const float *x, long B, long Cin, long H, long W, const float *w, long Cout, long K,
                            const float *bias, long pool, const long *idx, long n, double *avg);
long oracle_dwsep_tout_ex(long T, long K, long pad, long stride, long dilation);
int oracle_dwsep_conv1d_ex(const float *x, long B, long C, long T, const float *w_dw, long K, const float *w_pw,
                           long O, const float *b_pw, long pad, long stride, long dilation, const long *batch_idx,
                           long nb, double *y, int nthreads);
int oracle_dwsep_conv1d_at_ex(const float *x, long B, long C, long T, const float *w_dw, long K, const float *w_pw,
                              long O, const float *b_pw, long pad, long stride, long dilation, const long *idx, long n,
                              double *y);

static unsigned long long rng_state = 88172645463325252ULL;
static float urand(void) { /* xorshift64, uniform in [-1, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (float)((double)(rng_state >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}
static float *fill(long n) {
    float *p = malloc((size_t)n * sizeof(float));
    for (long i = 0; i < n; ++i) p[i] = urand();
    return p;
}
static int failures = 0;
static void check(int ok, const char *what) {
    if (!ok) {
        fprintf(stderr, "FAIL: %s\n", what);
        ++failures;
    }
}

static void conv2d_checks(void) {
    const long B = 2, Cin = 3, H = 11, W = 13, Cout = 4, K = 3, pool = 2;
    long Hc, Wc, PH, PW;
    check(oracle_conv2d_sizes(H, W, K, pool, &Hc, &Wc, &PH, &PW) == 0 && PH == 4 && PW == 5, "conv2d sizes");
    float *x = fill(B * Cin * H * W), *w = fill(Cout * Cin * K * K), *b = fill(Cout);
    double *out = malloc(B * sizeof(double)), *part = malloc(B * Cout * sizeof(double));
    double *pooled = malloc(B * Cout * PH * PW * sizeof(double));
    check(oracle_conv2d_pool_sigmoid_sum(x, B, Cin, H, W, w, Cout, K, b, pool, NULL, B, out, part, pooled, 3) == 0,
          "conv2d full");
    /* the sampled form at every pooled position agrees with the full form */
    const long n = B * Cout * PH * PW;
    long *idx = malloc((size_t)n * 4 * sizeof(long));
    double *avg = malloc((size_t)n * sizeof(double));
    long i = 0;
    for (long bb = 0; bb < B; ++bb)
        for (long co = 0; co < Cout; ++co)
            for (long ph = 0; ph < PH; ++ph)
                for (long pw = 0; pw < PW; ++pw, ++i) {
                    idx[4 * i] = bb, idx[4 * i + 1] = co, idx[4 * i + 2] = ph, idx[4 * i + 3] = pw;
                }
    check(oracle_conv2d_pooled_at(x, B, Cin, H, W, w, Cout, K, b, pool, idx, n, avg) == 0, "conv2d pooled_at");
    double worst = 0;
    for (i = 0; i < n; ++i) worst = fmax(worst, fabs(avg[i] - pooled[i]));
    check(worst < 1e-12, "pooled_at equals the full form");
    /* one batch item through batch_idx */
    const long one = 1;
    double out1;
    check(oracle_conv2d_pool_sigmoid_sum(x, B, Cin, H, W, w, Cout, K, b, pool, &one, 1, &out1, NULL, NULL, 3) == 0 &&
              out1 == out[1],
          "conv2d batch_idx");
    /* zero weights and bias: out = Cout * PH * PW / 2 exactly */
    float *w0 = calloc((size_t)(Cout * Cin * K * K), sizeof(float));
    check(oracle_conv2d_pool_sigmoid_sum(x, B, Cin, H, W, w0, Cout, K, NULL, pool, NULL, B, out, NULL, NULL, 2) == 0 &&
              out[0] == Cout * PH * PW / 2.0 && out[1] == Cout * PH * PW / 2.0,
          "conv2d zero-weight closed form");
    /* invalid arguments */
    check(oracle_conv2d_pool_sigmoid_sum(NULL, B, Cin, H, W, w, Cout, K, b, pool, NULL, B, out, NULL, NULL, 1) != 0,
          "conv2d NULL x");
    check(oracle_conv2d_pool_sigmoid_sum(x, B, Cin, 2, W, w, Cout, K, b, pool, NULL, B, out, NULL, NULL, 1) != 0,
          "conv2d H < K");
    check(oracle_conv2d_pooled_at(x, B, Cin, H, W, w, Cout, K, b, 0, idx, n, avg) != 0, "conv2d pool 0");
    free(x), free(w), free(b), free(out), free(part), free(pooled), free(idx), free(avg), free(w0);
}

static void dwsep_checks(long stride, long dil) {
    const long B = 2, C = 5, T = 17, K = 4, O = 3, pad = 2;
    const long Tout = oracle_dwsep_tout_ex(T, K, pad, stride, dil);
    check(Tout >= 1, "dwsep Tout");
    float *x = fill(B * C * T), *wd = fill(C * K), *wp = fill(O * C), *bp = fill(O);
    double *y = malloc((size_t)(B * O * Tout) * sizeof(double));
    check(oracle_dwsep_conv1d_ex(x, B, C, T, wd, K, wp, O, bp, pad, stride, dil, NULL, B, y, 3) == 0, "dwsep full");
    const long n = B * O * Tout;
    long *idx = malloc((size_t)n * 3 * sizeof(long));
    double *ys = malloc((size_t)n * sizeof(double));
    long i = 0;
    for (long bb = 0; bb < B; ++bb)
        for (long o = 0; o < O; ++o)
            for (long t = 0; t < Tout; ++t, ++i) idx[3 * i] = bb, idx[3 * i + 1] = o, idx[3 * i + 2] = t;
    check(oracle_dwsep_conv1d_at_ex(x, B, C, T, wd, K, wp, O, bp, pad, stride, dil, idx, n, ys) == 0, "dwsep at");
    double worst = 0;
    for (i = 0; i < n; ++i) worst = fmax(worst, fabs(ys[i] - y[i]));
    check(worst < 1e-12, "dwsep at equals the full form");
    check(oracle_dwsep_conv1d_ex(x, B, C, T, wd, K, wp, O, bp, -1, stride, dil, NULL, B, y, 1) != 0, "dwsep pad < 0");
    check(oracle_dwsep_conv1d_ex(x, B, C, T, wd, K, wp, O, bp, pad, 0, dil, NULL, B, y, 1) != 0, "dwsep stride 0");
    check(oracle_dwsep_tout_ex(3, 9, 0, 1, 1) < 0, "dwsep empty output");
    free(x), free(wd), free(wp), free(bp), free(y), free(idx), free(ys);
}

int main(void) {
    conv2d_checks();
    dwsep_checks(1, 1);
    dwsep_checks(2, 3);
    if (failures) return 1;
    printf("oracle sanitizer driver: all checks passed\n");
    return 0;
}
