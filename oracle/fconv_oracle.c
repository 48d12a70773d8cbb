/*
 * fconv_oracle.c -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.
 *
 * A slow, plainly written CPU reference for the two fused fp32 convolutions,
 * in double precision.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code with the HIP library and
 * includes none of its headers.
 *
 * Sources (the method is defined on these pages; citations name the page and
 * the part of it):
 *   [P65] POPCORNBENCH reasoning trace "Kimi-K2.6 l2_p65" (Conv2d -> AvgPool2d
 *         -> Sigmoid -> Sum): the opening problem statement and dimension
 *         walk-through, the fused per-pooled-output formula that follows it,
 *         and the later boundary discussion of which conv rows the floor pool
 *         keeps.
 *   [P7]  POPCORNBENCH reasoning trace "Kimi-K2.6 l2_p7" (depthwise-separable
 *         Conv1d): the opening problem statement (output length formula) and
 *         the per-output formula out[b,o,t] = sum_c (sum_k in*dw) * pw + bias.
 *   [NEWS] the 新智元 article on the Stanford CRFM kernels: its list of fused
 *         operators includes Conv2D + ReLU + MaxPool, the model for the
 *         pooling generalisation (optional ReLU after the conv, max pooling).
 *
 * Readings taken where the pages leave a step open (listed again in the
 * design notes): AvgPool2d uses stride = kernel, padding 0 and floor mode,
 * divisor s*s; Conv2d is PyTorch's cross-correlation (no flip), stride 1, no
 * padding; sigmoid is the logistic 1/(1+exp(-a)); the depthwise stage has no
 * bias of its own; padding is zero padding; stride and dilation are 1.
 * The pooling generalisation follows PyTorch's AvgPool2d / MaxPool2d with
 * kernel = stride = s and no padding: ceil mode adds a last, partial window
 * when the conv map does not divide evenly (it must start inside the map);
 * a partial window averages over the conv outputs it covers, and takes
 * their maximum for max pooling; ReLU, when asked for, acts on the conv
 * outputs (bias included) before pooling.
 *
 * Every function here is a literal transcription of the definition: the
 * conv map is materialised in full, then pooled, then passed through the
 * sigmoid, then summed.  No blocking, fusion or re-association beyond the
 * loop order needed to walk the arrays.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL -1
#define ORACLE_ENOMEM -2

/* ---------------------------------------------------------------- threads */

typedef void (*work_fn)(void *ctx, long item, double *scratch);

typedef struct {
    work_fn fn;
    void *ctx;
    long n_items;
    long next;
    size_t scratch_doubles;
    int failed;
    pthread_mutex_t lock;
} pool_t;

static void *pool_worker(void *arg) {
    pool_t *p = (pool_t *)arg;
    double *scratch = NULL;
    if (p->scratch_doubles) {
        scratch = (double *)malloc(p->scratch_doubles * sizeof(double));
        if (!scratch) {
            pthread_mutex_lock(&p->lock);
            p->failed = 1;
            pthread_mutex_unlock(&p->lock);
            return NULL;
        }
    }
    for (;;) {
        pthread_mutex_lock(&p->lock);
        long item = p->next++;
        pthread_mutex_unlock(&p->lock);
        if (item >= p->n_items) break;
        p->fn(p->ctx, item, scratch);
    }
    free(scratch);
    return NULL;
}

/* Runs fn(ctx, item, scratch) for item in [0, n_items) on nthreads threads;
 * each thread owns a scratch buffer of scratch_doubles doubles. */
static int parallel_for(long n_items, int nthreads, size_t scratch_doubles, work_fn fn, void *ctx) {
    pool_t p;
    p.fn = fn;
    p.ctx = ctx;
    p.n_items = n_items;
    p.next = 0;
    p.scratch_doubles = scratch_doubles;
    p.failed = 0;
    pthread_mutex_init(&p.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((long)nthreads > n_items) nthreads = (int)(n_items > 0 ? n_items : 1);
    pthread_t tid[256];
    int started = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&tid[i], NULL, pool_worker, &p) != 0) break;
        ++started;
    }
    if (started == 0) pool_worker(&p);
    for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
    pthread_mutex_destroy(&p.lock);
    return p.failed ? ORACLE_ENOMEM : ORACLE_OK;
}

static double logistic(double a) { return 1.0 / (1.0 + exp(-a)); }

/* ------------------------------------------------ Conv2d -> AvgPool2d -> sigmoid -> sum */

/* Output sizes.  [P65] opening dimension walk-through: a valid (unpadded)
 * stride-1 Conv2d of kernel K gives H-K+1; AvgPool2d(s) with its default
 * stride s and floor mode gives floor((H-K+1)/s).  In ceil mode the count is
 * rounded up instead (PyTorch's pooling output size; with no padding the
 * last window always starts inside the conv map, so none is dropped). */
static long pooled_len(long n, long s, int ceil_mode) { return ceil_mode ? (n + s - 1) / s : n / s; }

int oracle_conv2d_sizes_ex(long H, long W, long K, long pool, int ceil_mode, long *Hc, long *Wc, long *PH,
                           long *PW) {
    if (H < 1 || W < 1 || K < 1 || pool < 1 || H < K || W < K) return ORACLE_EINVAL;
    *Hc = H - K + 1;
    *Wc = W - K + 1;
    *PH = pooled_len(*Hc, pool, ceil_mode);
    *PW = pooled_len(*Wc, pool, ceil_mode);
    return ORACLE_OK;
}

int oracle_conv2d_sizes(long H, long W, long K, long pool, long *Hc, long *Wc, long *PH, long *PW) {
    return oracle_conv2d_sizes_ex(H, W, K, pool, 0, Hc, Wc, PH, PW);
}

typedef struct {
    const float *x, *w, *bias;
    long B, Cin, H, W, Cout, K, pool, Hc, Wc, PH, PW;
    int pool_mode, relu; /* pool_mode 0: average, 1: maximum */
    const long *batch_idx;
    double *part;   /* [nb*Cout] */
    double *pooled; /* [nb*Cout*PH*PW] or NULL */
} conv2d_ctx;

/* One (batch item, output channel): the full conv map M, then the pool A,
 * then the sum of sigmoid(A).  [P65] problem statement: conv output
 * [i,j] = bias[oc] + sum over (c, ky, kx) of input[b,c,i+ky,j+kx] *
 * weight[oc,c,ky,kx]; the pool averages each non-overlapping s x s block;
 * the floor drops the conv rows/columns at or beyond PH*s. */
static void conv2d_item(void *vctx, long item, double *M) {
    conv2d_ctx *c = (conv2d_ctx *)vctx;
    const long bi = item / c->Cout, co = item % c->Cout;
    const long b = c->batch_idx ? c->batch_idx[bi] : bi;
    const long Hc = c->Hc, Wc = c->Wc, H = c->H, W = c->W, K = c->K, s = c->pool;

    /* step 1: conv map M[y][x] for 0 <= y < Hc, 0 <= x < Wc */
    const double beta = c->bias ? (double)c->bias[co] : 0.0;
    for (long i = 0; i < Hc * Wc; ++i) M[i] = 0.0;
    for (long ic = 0; ic < c->Cin; ++ic) {
        const float *xp = c->x + ((b * c->Cin + ic) * H) * W;
        const float *wp = c->w + ((co * c->Cin + ic) * K) * K;
        for (long ky = 0; ky < K; ++ky)
            for (long kx = 0; kx < K; ++kx) {
                const double wv = (double)wp[ky * K + kx];
                for (long y = 0; y < Hc; ++y) {
                    const float *row = xp + (y + ky) * W + kx;
                    double *mrow = M + y * Wc;
                    for (long xx = 0; xx < Wc; ++xx) mrow[xx] += (double)row[xx] * wv;
                }
            }
    }
    for (long i = 0; i < Hc * Wc; ++i) M[i] += beta;
    if (c->relu)
        for (long i = 0; i < Hc * Wc; ++i) M[i] = M[i] > 0.0 ? M[i] : 0.0;

    /* steps 2-3: pool (each window clipped to the conv map), sigmoid, sum */
    double total = 0.0;
    for (long ph = 0; ph < c->PH; ++ph)
        for (long pw = 0; pw < c->PW; ++pw) {
            const long ny = (ph * s + s <= Hc) ? s : Hc - ph * s;
            const long nx = (pw * s + s <= Wc) ? s : Wc - pw * s;
            double a;
            if (c->pool_mode == 1) {
                a = -INFINITY;
                for (long dy = 0; dy < ny; ++dy)
                    for (long dx = 0; dx < nx; ++dx) {
                        const double v = M[(ph * s + dy) * Wc + (pw * s + dx)];
                        a = v > a ? v : a;
                    }
            } else {
                double acc = 0.0;
                for (long dy = 0; dy < ny; ++dy)
                    for (long dx = 0; dx < nx; ++dx) acc += M[(ph * s + dy) * Wc + (pw * s + dx)];
                a = acc / (double)(ny * nx);
            }
            if (c->pooled) c->pooled[((bi * c->Cout + co) * c->PH + ph) * c->PW + pw] = a;
            total += logistic(a);
        }
    c->part[bi * c->Cout + co] = total;
}

/*
 * out[i] = sum over co, ph, pw of sigmoid(pool(relu?(conv2d(x[b_i], w) + bias)))
 * for the batch items b_i = batch_idx[i] (batch_idx NULL: i = 0..nb-1);
 * pool_mode 0 averages, 1 takes the maximum; relu 1 applies ReLU to the conv
 * outputs first; ceil_mode 1 keeps the last, partial windows.
 * part[i*Cout+co] (optional) receives the per-channel sums, pooled (optional)
 * the pre-sigmoid pooled map [nb, Cout, PH, PW].  bias may be NULL (zero).
 * The per-channel sums are added in increasing co, so out is deterministic.
 */
int oracle_conv2d_pool_sigmoid_sum_ex(const float *x, long B, long Cin, long H, long W, const float *w, long Cout,
                                      long K, const float *bias, long pool, int pool_mode, int relu, int ceil_mode,
                                      const long *batch_idx, long nb, double *out, double *part, double *pooled,
                                      int nthreads) {
    conv2d_ctx c;
    if (!x || !w || !out || B < 1 || Cin < 1 || Cout < 1 || nb < 0) return ORACLE_EINVAL;
    if (pool_mode < 0 || pool_mode > 1 || relu < 0 || relu > 1 || ceil_mode < 0 || ceil_mode > 1)
        return ORACLE_EINVAL;
    if (oracle_conv2d_sizes_ex(H, W, K, pool, ceil_mode, &c.Hc, &c.Wc, &c.PH, &c.PW) != ORACLE_OK)
        return ORACLE_EINVAL;
    c.pool_mode = pool_mode;
    c.relu = relu;
    if (batch_idx) {
        for (long i = 0; i < nb; ++i)
            if (batch_idx[i] < 0 || batch_idx[i] >= B) return ORACLE_EINVAL;
    } else if (nb > B) {
        return ORACLE_EINVAL;
    }
    c.x = x; c.w = w; c.bias = bias;
    c.B = B; c.Cin = Cin; c.H = H; c.W = W; c.Cout = Cout; c.K = K; c.pool = pool;
    c.batch_idx = batch_idx;
    c.pooled = pooled;
    double *own = NULL;
    c.part = part;
    if (!c.part) {
        own = (double *)malloc((size_t)(nb * Cout > 0 ? nb * Cout : 1) * sizeof(double));
        if (!own) return ORACLE_ENOMEM;
        c.part = own;
    }
    int rc = parallel_for(nb * Cout, nthreads, (size_t)(c.Hc * c.Wc), conv2d_item, &c);
    if (rc == ORACLE_OK)
        for (long i = 0; i < nb; ++i) {
            double s = 0.0;
            for (long co = 0; co < Cout; ++co) s += c.part[i * Cout + co];
            out[i] = s;
        }
    free(own);
    return rc;
}

int oracle_conv2d_pool_sigmoid_sum(const float *x, long B, long Cin, long H, long W, const float *w,
                                   long Cout, long K, const float *bias, long pool, const long *batch_idx,
                                   long nb, double *out, double *part, double *pooled, int nthreads) {
    return oracle_conv2d_pool_sigmoid_sum_ex(x, B, Cin, H, W, w, Cout, K, bias, pool, 0, 0, 0, batch_idx, nb, out,
                                             part, pooled, nthreads);
}

/*
 * Pre-sigmoid pooled values at n chosen positions idx[4*i..4*i+3] =
 * (b, co, ph, pw): avg = (1/s^2) * sum over the s x s window of the conv map,
 * each conv output computed from its definition.  [P65] fused
 * per-pooled-output formula.
 */
int oracle_conv2d_pooled_at_ex(const float *x, long B, long Cin, long H, long W, const float *w, long Cout, long K,
                               const float *bias, long pool, int pool_mode, int relu, int ceil_mode, const long *idx,
                               long n, double *val) {
    long Hc, Wc, PH, PW;
    if (!x || !w || !val || (n > 0 && !idx)) return ORACLE_EINVAL;
    if (pool_mode < 0 || pool_mode > 1 || relu < 0 || relu > 1 || ceil_mode < 0 || ceil_mode > 1)
        return ORACLE_EINVAL;
    if (oracle_conv2d_sizes_ex(H, W, K, pool, ceil_mode, &Hc, &Wc, &PH, &PW) != ORACLE_OK) return ORACLE_EINVAL;
    for (long i = 0; i < n; ++i) {
        const long b = idx[4 * i], co = idx[4 * i + 1], ph = idx[4 * i + 2], pw = idx[4 * i + 3];
        if (b < 0 || b >= B || co < 0 || co >= Cout || ph < 0 || ph >= PH || pw < 0 || pw >= PW)
            return ORACLE_EINVAL;
        double acc = 0.0, mx = -INFINITY;
        long count = 0;
        for (long dy = 0; dy < pool; ++dy)
            for (long dx = 0; dx < pool; ++dx) {
                const long y = ph * pool + dy, xx = pw * pool + dx;
                if (y >= Hc || xx >= Wc) continue; /* outside a partial (ceil-mode) window */
                double conv = bias ? (double)bias[co] : 0.0;
                for (long ic = 0; ic < Cin; ++ic)
                    for (long ky = 0; ky < K; ++ky)
                        for (long kx = 0; kx < K; ++kx)
                            conv += (double)x[((b * Cin + ic) * H + y + ky) * W + xx + kx] *
                                    (double)w[((co * Cin + ic) * K + ky) * K + kx];
                if (relu && conv < 0.0) conv = 0.0;
                acc += conv;
                mx = conv > mx ? conv : mx;
                ++count;
            }
        val[i] = pool_mode == 1 ? mx : acc / (double)count;
    }
    return ORACLE_OK;
}

int oracle_conv2d_pooled_at(const float *x, long B, long Cin, long H, long W, const float *w, long Cout,
                            long K, const float *bias, long pool, const long *idx, long n, double *avg) {
    return oracle_conv2d_pooled_at_ex(x, B, Cin, H, W, w, Cout, K, bias, pool, 0, 0, 0, idx, n, avg);
}

/* ------------------------------------ depthwise Conv1d -> pointwise 1x1 Conv1d + bias */

/* [P7] opening problem statement: T_out = (T + 2*pad - K)/stride + 1.  With
 * a dilation d the filter spans d*(K-1)+1 steps (PyTorch's Conv1d), so
 * T_out = floor((T + 2*pad - d*(K-1) - 1)/stride) + 1; -1 if that is < 1. */
long oracle_dwsep_tout_ex(long T, long K, long pad, long stride, long dilation) {
    if (T < 1 || K < 1 || pad < 0 || stride < 1 || dilation < 1) return -1;
    const long span = T + 2 * pad - dilation * (K - 1) - 1;
    if (span < 0) return -1;
    return span / stride + 1;
}

long oracle_dwsep_tout(long T, long K, long pad) { return oracle_dwsep_tout_ex(T, K, pad, 1, 1); }

typedef struct {
    const float *x, *w_dw, *w_pw, *b_pw;
    long B, C, T, K, O, pad, stride, dilation, Tout;
    long b;
    double *D; /* [C][Tout] */
    double *y; /* [O][Tout] for the current batch item */
} dwsep_ctx;

/* Depthwise stage, one channel: D[c,t] = sum_k w_dw[c,k] * x[b,c,t*stride+k*dilation-pad],
 * reading 0 outside [0, T).  [P7] per-output formula, inner sum (its
 * in[b, c, t*stride + k - padding]; the dilation spaces the taps). */
static void dw_channel(void *vctx, long c, double *unused) {
    (void)unused;
    dwsep_ctx *d = (dwsep_ctx *)vctx;
    const float *xr = d->x + (d->b * d->C + c) * d->T;
    const float *wr = d->w_dw + c * d->K;
    double *Dr = d->D + c * d->Tout;
    for (long t = 0; t < d->Tout; ++t) {
        double acc = 0.0;
        for (long k = 0; k < d->K; ++k) {
            const long src = t * d->stride + k * d->dilation - d->pad;
            const double xv = (src >= 0 && src < d->T) ? (double)xr[src] : 0.0;
            acc += (double)wr[k] * xv;
        }
        Dr[t] = acc;
    }
}

/* Pointwise stage, one output channel: y[b,o,t] = b_pw[o] + sum_c w_pw[o,c] * D[c,t].
 * [P7] per-output formula, outer sum plus bias.  The sum runs over c in
 * increasing order for every t. */
static void pw_channel(void *vctx, long o, double *unused) {
    (void)unused;
    dwsep_ctx *d = (dwsep_ctx *)vctx;
    double *yr = d->y + o * d->Tout;
    for (long t = 0; t < d->Tout; ++t) yr[t] = 0.0;
    for (long c = 0; c < d->C; ++c) {
        const double wv = (double)d->w_pw[o * d->C + c];
        const double *Dr = d->D + c * d->Tout;
        for (long t = 0; t < d->Tout; ++t) yr[t] += wv * Dr[t];
    }
    const double beta = d->b_pw ? (double)d->b_pw[o] : 0.0;
    for (long t = 0; t < d->Tout; ++t) yr[t] += beta;
}

/*
 * y[i] = pointwise(depthwise(x[b_i])) + b_pw for the batch items b_i =
 * batch_idx[i] (NULL: i = 0..nb-1); y is [nb, O, Tout] doubles.  b_pw may
 * be NULL (zero).
 */
int oracle_dwsep_conv1d_ex(const float *x, long B, long C, long T, const float *w_dw, long K, const float *w_pw,
                           long O, const float *b_pw, long pad, long stride, long dilation, const long *batch_idx,
                           long nb, double *y, int nthreads) {
    dwsep_ctx d;
    if (!x || !w_dw || !w_pw || !y || B < 1 || C < 1 || O < 1 || nb < 0) return ORACLE_EINVAL;
    d.Tout = oracle_dwsep_tout_ex(T, K, pad, stride, dilation);
    if (d.Tout < 1) return ORACLE_EINVAL;
    if (batch_idx) {
        for (long i = 0; i < nb; ++i)
            if (batch_idx[i] < 0 || batch_idx[i] >= B) return ORACLE_EINVAL;
    } else if (nb > B) {
        return ORACLE_EINVAL;
    }
    d.x = x; d.w_dw = w_dw; d.w_pw = w_pw; d.b_pw = b_pw;
    d.B = B; d.C = C; d.T = T; d.K = K; d.O = O; d.pad = pad; d.stride = stride; d.dilation = dilation;
    d.D = (double *)malloc((size_t)(C * d.Tout) * sizeof(double));
    if (!d.D) return ORACLE_ENOMEM;
    int rc = ORACLE_OK;
    for (long i = 0; i < nb && rc == ORACLE_OK; ++i) {
        d.b = batch_idx ? batch_idx[i] : i;
        d.y = y + i * O * d.Tout;
        rc = parallel_for(C, nthreads, 0, dw_channel, &d);
        if (rc == ORACLE_OK) rc = parallel_for(O, nthreads, 0, pw_channel, &d);
    }
    free(d.D);
    return rc;
}

int oracle_dwsep_conv1d(const float *x, long B, long C, long T, const float *w_dw, long K, const float *w_pw,
                        long O, const float *b_pw, long pad, const long *batch_idx, long nb, double *y,
                        int nthreads) {
    return oracle_dwsep_conv1d_ex(x, B, C, T, w_dw, K, w_pw, O, b_pw, pad, 1, 1, batch_idx, nb, y, nthreads);
}

/* y at n chosen positions idx[3*i..3*i+2] = (b, o, t), each from the
 * definition (the depthwise values are recomputed per position). */
int oracle_dwsep_conv1d_at_ex(const float *x, long B, long C, long T, const float *w_dw, long K,
                              const float *w_pw, long O, const float *b_pw, long pad, long stride, long dilation,
                              const long *idx, long n, double *y) {
    const long Tout = oracle_dwsep_tout_ex(T, K, pad, stride, dilation);
    if (!x || !w_dw || !w_pw || !y || (n > 0 && !idx) || Tout < 1) return ORACLE_EINVAL;
    for (long i = 0; i < n; ++i) {
        const long b = idx[3 * i], o = idx[3 * i + 1], t = idx[3 * i + 2];
        if (b < 0 || b >= B || o < 0 || o >= O || t < 0 || t >= Tout) return ORACLE_EINVAL;
        double acc = 0.0;
        for (long c = 0; c < C; ++c) {
            double dv = 0.0;
            for (long k = 0; k < K; ++k) {
                const long src = t * stride + k * dilation - pad;
                const double xv = (src >= 0 && src < T) ? (double)x[(b * C + c) * T + src] : 0.0;
                dv += (double)w_dw[c * K + k] * xv;
            }
            acc += (double)w_pw[o * C + c] * dv;
        }
        y[i] = acc + (b_pw ? (double)b_pw[o] : 0.0);
    }
    return ORACLE_OK;
}

int oracle_dwsep_conv1d_at(const float *x, long B, long C, long T, const float *w_dw, long K,
                           const float *w_pw, long O, const float *b_pw, long pad, const long *idx, long n,
                           double *y) {
    return oracle_dwsep_conv1d_at_ex(x, B, C, T, w_dw, K, w_pw, O, b_pw, pad, 1, 1, idx, n, y);
}
