/*
 * fconv.h -- C ABI of libfconv: fused fp32 convolutions for AMD MI355X (gfx950).
 *
 * Two operations, each one call that keeps its intermediate out of HBM:
 *
 *   fconv2d_pool_sigmoid_sum   Conv2d (stride 1, no padding) -> AvgPool2d
 *                              (kernel = stride = pool, floor) -> sigmoid ->
 *                              sum over channels and space: one scalar per
 *                              batch item.  Defined by the POPCORNBENCH
 *                              reasoning trace "Kimi-K2.6 l2_p65"
 *                              (Conv2d -> AvgPool2d -> Sigmoid -> Sum): its
 *                              opening problem statement and the fused
 *                              per-pooled-output formula that follows it.
 *
 *   dwsep_conv1d               depthwise Conv1d (kernel K, zero padding pad,
 *                              stride 1) -> pointwise 1x1 Conv1d + bias.
 *                              Defined by the POPCORNBENCH reasoning trace
 *                              "Kimi-K2.6 l2_p7" (depthwise-separable Conv1d):
 *                              its opening problem statement (output length)
 *                              and the per-output formula
 *                              out[b,o,t] = sum_c (sum_k in[b,c,t+k-pad] *
 *                              dw[c,k]) * pw[o,c] + bias[o].
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, contiguous, row-major fp32 in DEVICE memory
 *     (hipMalloc'd or equivalent), owned by the caller.  Only 4-byte
 *     alignment is required.  Input buffers are never written.
 *   - The library is reentrant.  Calls on different streams may run
 *     concurrently as long as their output buffers do not overlap.  The
 *     fused sums (fconv2d_pool_sigmoid_sum, _algo, _ex) take their partial
 *     sums' scratch (at most 4 KiB per batch item) from a memory pool the
 *     library creates per device on first use and keeps until the process
 *     ends, allocated in stream order on the call's stream
 *     (hipMallocFromPoolAsync).  Up to 8 streams per device keep a buffer
 *     of up to 1 MiB between calls, guarded by an event the library records
 *     after each use and waits on (on the GPU) before the next; other calls,
 *     and calls on a stream being captured into a graph, allocate per call
 *     and free in stream order (hipFreeAsync).  Concurrent calls never share
 *     scratch, and `stream` must belong to the current device.  No other
 *     entry point allocates device memory.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Every call is asynchronous with respect to the host: it enqueues its
 *     kernels on `stream` and returns.  Outputs are valid once the stream
 *     has reached that point.
 *   - Sizes are int64_t.  Argument checks happen on the host before any
 *     device work; a failed check returns FCONV_EINVAL and enqueues nothing.
 *   - A HIP launch error is returned as FCONV_EHIP (from hipGetLastError).
 *   - The sums inside a call are fp32.  Every fused sum writes one partial
 *     sum per workgroup and a second kernel adds each batch item's partials
 *     in a fixed order, so repeated calls with the same inputs, algorithm
 *     and device give identical bits.  A call never uses more than 1024
 *     workgroups per batch item (larger maps have each workgroup walk
 *     several tiles, summing in fp64 between them): 96 partials per item
 *     for x[128,8,384,384] (box-sum), 1024 for an item of 5e8 input
 *     elements.  Every partial is positive (a sum of sigmoids) and no chain
 *     of additions in that reduction is longer than 12, so it rounds by at
 *     most 12 x 2^-24 = 7.2e-7 |out[b]| at every shape the ABI accepts.
 */
#ifndef FCONV_H
#define FCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned (as int) by every entry point. */
typedef enum fconv_status {
    FCONV_OK = 0,
    FCONV_EINVAL = -1,       /* an argument failed a check; nothing was enqueued */
    FCONV_EUNSUPPORTED = -2, /* the requested algorithm cannot run this shape   */
    FCONV_EHIP = -3,         /* the HIP runtime reported an error              */
    FCONV_ESCRATCH = -4      /* more partial sums than the fixed scratch holds (see
                                fconv2d_pool_sigmoid_sum_det_noalloc); nothing was enqueued */
} fconv_status;

/* Algorithms for the Conv2d path.  All compute the same result up to fp32
 * rounding.  AUTO picks the fastest one that supports the shape: BOXSUM,
 * else DIRECT_MFMA, else DIRECT_SIMPLE. */
#define FCONV_ALGO_AUTO 0
#define FCONV_ALGO_DIRECT_MFMA 1   /* direct conv on fp32 matrix cores: s*s*Cin*K*K MACs per
                                      (co, pooled output); K=3 with pool 2,3,4 and K=5 with
                                      pool 3, any Cin: a workgroup stages all of its tile's
                                      channels in LDS while they fit (up to Cin 32-68 by
                                      shape), else 16 channels at a time */
#define FCONV_ALGO_DIRECT_SIMPLE 2 /* direct conv, one thread per pooled output, any shape */
#define FCONV_ALGO_BOXSUM 3        /* pool-then-convolve: s x s box sums of the input, then
                                      Cin*K*K MACs per (co, pooled output) on matrix cores;
                                      K=3 with pool 2,3,4 and K=5 with pool 3, any Cin (the box
                                      sums pass through LDS 8 or 16 channels at a time).
                                      Pooling commutes with the convolution (both are linear),
                                      so the result is the same function of the inputs. */

/*
 * fconv2d_pool_sigmoid_sum
 *
 *   out[b] = sum_{co < Cout} sum_{ph < PH} sum_{pw < PW}
 *              sigmoid( (1/pool^2) * sum_{dy,dx < pool} conv[b,co,ph*pool+dy,pw*pool+dx] )
 *   conv[b,co,y,x] = bias[co] + sum_{ic,ky,kx} x[b,ic,y+ky,x+kx] * w[co,ic,ky,kx]
 *   Hc = H-K+1, Wc = W-K+1, PH = floor(Hc/pool), PW = floor(Wc/pool);
 *   sigmoid(a) = 1/(1+exp(-a)).  Conv rows/columns at or beyond PH*pool
 *   (PW*pool) feed no pooled output (floor mode).
 *
 *   x    [B, Cin, H, W]
 *   w    [Cout, Cin, K, K]   (cross-correlation, as PyTorch's Conv2d)
 *   bias [Cout], or NULL for no bias
 *   out  [B], fully overwritten
 *
 * FCONV_EINVAL when: x, w or out is NULL; any of B, Cin, Cout, H, W, K, pool
 * is < 1; H < K or W < K; an element count overflows int64.  A shape with
 * PH = 0 or PW = 0 is valid and gives out = 0.
 * FCONV_EUNSUPPORTED when one batch item's input (Cin*H*W) or the weight
 * (Cout*Cin*K*K) has 2^29 elements or more, one batch item's pooled map
 * (Cout*PH*PW) exceeds 2^31-1 elements, B > 65535, Cout > 2^20, or K or
 * pool > 4096.
 * FCONV_EHIP also if the partial sums' scratch cannot be allocated.
 */
int fconv2d_pool_sigmoid_sum(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W,
                             const float* w, int64_t Cout, int64_t K, const float* bias,
                             int64_t pool, float* out, void* stream);

/* As fconv2d_pool_sigmoid_sum, with an explicit algorithm (FCONV_ALGO_*).
 * FCONV_EUNSUPPORTED if that algorithm has no instance for (K, pool). */
int fconv2d_pool_sigmoid_sum_algo(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W,
                                  const float* w, int64_t Cout, int64_t K, const float* bias,
                                  int64_t pool, int algo, float* out, void* stream);

/*
 * fconv2d_pool_sigmoid_sum_det -- fconv2d_pool_sigmoid_sum_algo with the
 *   partial sums in a caller-owned workspace instead of the library's pool:
 *   each workgroup writes its partial sum to its own slot of `workspace`; a
 *   second kernel then adds each batch item's slots in a fixed order into
 *   out[b].  Same kernels, so the same bits as the pooled call with the same
 *   algorithm.  This is the workspace two-pass that the l2_p65 trace weighs
 *   against per-block atomics in its atomic-contention discussion; on
 *   MI355X it is also the faster of the two (12,288 same-address float
 *   atomics for x[128,8,384,384] cost 13 % of the kernel's time).
 *   workspace        device memory of at least the size that
 *                    fconv2d_pool_sigmoid_sum_det_workspace reports, owned by
 *                    the caller; its contents on entry are ignored and on
 *                    return are unspecified.  Calls that share a workspace
 *                    must be ordered (same stream).
 *   workspace_bytes  its size; FCONV_EINVAL if too small (or NULL with a
 *                    non-empty pooled map).
 * Other arguments and errors as fconv2d_pool_sigmoid_sum_algo.
 */
int fconv2d_pool_sigmoid_sum_det(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W,
                                 const float* w, int64_t Cout, int64_t K, const float* bias,
                                 int64_t pool, int algo, void* workspace, size_t workspace_bytes,
                                 float* out, void* stream);

/*
 * fconv2d_pool_sigmoid_sum_det_noalloc -- fconv2d_pool_sigmoid_sum_det with no
 *   workspace argument, for callers that cannot allocate device memory: code
 *   under HIP graph capture, tight serving loops, harnesses that forbid
 *   hipMalloc.  The call allocates nothing (no hipMalloc, no allocating
 *   library routine); its partial sums go to a fixed device array of
 *   FCONV_NOALLOC_MAX_PARTIALS floats (1 MiB) inside the library, one per GPU,
 *   held until the process ends.  Same kernels, same fixed-order reduction
 *   and so the same bits as fconv2d_pool_sigmoid_sum_det.
 *   Limit: B * (workgroups per batch item) <= FCONV_NOALLOC_MAX_PARTIALS
 *   (the workspace query of fconv2d_pool_sigmoid_sum_det / 4 gives that
 *   product; at most 1024 workgroups per item, so any shape with B <= 256
 *   fits); beyond it the call returns FCONV_ESCRATCH and enqueues nothing.
 *   Every call on one GPU shares that GPU's array: calls that overlap in
 *   time on one GPU (different streams, or different host threads without
 *   ordering) race and give undefined results.  Calls ordered on one stream
 *   are safe.  `stream` must belong to the current device.
 *   FCONV_EHIP also if the array's device address cannot be obtained.
 * Other arguments and errors as fconv2d_pool_sigmoid_sum_det.
 */
#define FCONV_NOALLOC_MAX_PARTIALS (1 << 18)
int fconv2d_pool_sigmoid_sum_det_noalloc(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W,
                                         const float* w, int64_t Cout, int64_t K, const float* bias,
                                         int64_t pool, int algo, float* out, void* stream);

/* Workspace bytes fconv2d_pool_sigmoid_sum_det needs for this shape and
 * algorithm (B * workgroups per batch item * 4, with at most 1024 workgroups
 * per item: at most 4 KiB per batch item; 0 if the pooled map is empty).
 * Host only.  Errors as the call itself (NULL bytes: EINVAL). */
int fconv2d_pool_sigmoid_sum_det_workspace(int64_t B, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                                           int64_t K, int64_t pool, int algo, size_t* bytes);

/*
 * fconv2d_pool_map -- the pre-sigmoid pooled map of the same computation,
 *   pooled[b,co,ph,pw] = bias[co] + (1/pool^2) * sum_{dy,dx} (conv - bias)
 * written for every (b, co, ph, pw) of [B, Cout, PH, PW], computed by the
 * same kernels (same tiling and accumulation order) as the fused call.
 * This is the elementwise view the fused scalar hides; it exists for
 * verification and costs an extra HBM write of B*Cout*PH*PW floats.
 * Errors as fconv2d_pool_sigmoid_sum_algo; with PH or PW = 0 nothing is
 * written and `pooled` may be NULL (it must not be NULL otherwise).
 */
int fconv2d_pool_map(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W,
                     const float* w, int64_t Cout, int64_t K, const float* bias, int64_t pool,
                     int algo, float* pooled, void* stream);

/* fconv2d_pool_debug_map -- fconv2d_pool_map with algo = FCONV_ALGO_AUTO:
 * the pooled map the default fconv2d_pool_sigmoid_sum call sums, with that
 * call's arguments (pooled [B, Cout, PH, PW] in place of out).  Same errors. */
int fconv2d_pool_debug_map(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W,
                           const float* w, int64_t Cout, int64_t K, const float* bias, int64_t pool,
                           float* pooled, void* stream);

/* Output size of the pooled map: PH, PW (either may be 0).  Pure host
 * arithmetic, no device access.  FCONV_EINVAL on sizes < 1, H < K, W < K. */
int fconv2d_pool_out_size(int64_t H, int64_t W, int64_t K, int64_t pool, int64_t* PH, int64_t* PW);

/* The algorithm FCONV_ALGO_AUTO would run for this shape (a FCONV_ALGO_*
 * value), or FCONV_EINVAL.  Pure host logic, no device access. */
int fconv2d_select_algo(int64_t Cin, int64_t Cout, int64_t K, int64_t pool);

/*
 * Generalised pool (the Conv2D + ReLU + MaxPool fused operator that the
 * 新智元 article on the KernelBench / POPCORNBENCH results lists, on top of
 * the l2_p65 chain):
 *
 *   out[b] = sum_{co,ph,pw} sigmoid( POOL_{(y,x) in window(ph,pw)} act(conv[b,co,y,x]) )
 *   conv   as in fconv2d_pool_sigmoid_sum (bias included before act)
 *   act    = max(., 0) with FCONV_RELU, else the identity
 *   POOL   = mean over the window's elements (FCONV_POOL_AVG) or their
 *            maximum (FCONV_POOL_MAX)
 *   window(ph,pw) = rows [ph*pool, min(ph*pool+pool, Hc)) x columns
 *            [pw*pool, min(pw*pool+pool, Wc))
 *   PH = floor(Hc/pool), or ceil(Hc/pool) with FCONV_CEIL_MODE (PW alike).
 *
 * This is PyTorch's AvgPool2d / MaxPool2d with kernel = stride = pool, no
 * padding, ceil_mode as flagged: in ceil mode the last window of a row or
 * column is clipped to the map and a clipped window averages over its
 * valid elements only (no padding means every window starts inside the map).
 * FCONV_POOL_AVG with flags 0 is exactly fconv2d_pool_sigmoid_sum.
 * NaN inputs: the maximum of a window that holds a NaN is unspecified.
 */
#define FCONV_POOL_AVG 0
#define FCONV_POOL_MAX 1
#define FCONV_RELU 1      /* flag: ReLU after the conv + bias, before the pool */
#define FCONV_CEIL_MODE 2 /* flag: ceil output size, clipped last windows      */

/*
 * fconv2d_pool_sigmoid_sum_ex -- the fused sum with the generalised pool.
 *   pool_mode  FCONV_POOL_AVG or FCONV_POOL_MAX
 *   flags      0 or an OR of FCONV_RELU, FCONV_CEIL_MODE
 *   algo       FCONV_ALGO_AUTO, DIRECT_MFMA (K = 3 with pool 2, 3, 4 and
 *              K = 5 with pool 3, any Cin; whole-tile LDS staging up to
 *              Cin 32 (K3, pool 4), 56 (pool 2), 40 (pool 3), 68 (K5,
 *              pool 3), 16 channels at a time beyond),
 *              DIRECT_SIMPLE (any shape) or, only for
 *              FCONV_POOL_AVG with flags 0, BOXSUM.  AUTO picks DIRECT_MFMA
 *              where it has an instance, else DIRECT_SIMPLE (for the plain
 *              average pool it picks as fconv2d_pool_sigmoid_sum does).
 * Other arguments, layouts and errors as fconv2d_pool_sigmoid_sum_algo;
 * additionally FCONV_EINVAL for an unknown pool_mode or flag bit, and
 * FCONV_EUNSUPPORTED for BOXSUM with a max pool, ReLU or ceil mode (the
 * box-sum identity needs a linear pool over full windows).
 */
int fconv2d_pool_sigmoid_sum_ex(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W,
                                const float* w, int64_t Cout, int64_t K, const float* bias,
                                int64_t pool, int pool_mode, int flags, int algo, float* out,
                                void* stream);

/* The pre-sigmoid pooled map [B, Cout, PH, PW] of fconv2d_pool_sigmoid_sum_ex
 * (PH, PW as fconv2d_pool_out_size_ex reports), computed by the same kernels.
 * Arguments and errors as fconv2d_pool_sigmoid_sum_ex; `pooled` may be NULL
 * when the map has no elements. */
int fconv2d_pool_map_ex(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W,
                        const float* w, int64_t Cout, int64_t K, const float* bias, int64_t pool,
                        int pool_mode, int flags, int algo, float* pooled, void* stream);

/* The bitwise-reproducible form of fconv2d_pool_sigmoid_sum_ex: per-workgroup
 * partial sums into `workspace`, then a fixed-order reduction, as
 * fconv2d_pool_sigmoid_sum_det (same workspace rules; its size from
 * fconv2d_pool_sigmoid_sum_det_workspace_ex).  Arguments and errors as
 * fconv2d_pool_sigmoid_sum_ex, plus FCONV_EINVAL for a workspace that is too
 * small (or NULL with a non-empty pooled map). */
int fconv2d_pool_sigmoid_sum_det_ex(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W,
                                    const float* w, int64_t Cout, int64_t K, const float* bias,
                                    int64_t pool, int pool_mode, int flags, int algo, void* workspace,
                                    size_t workspace_bytes, float* out, void* stream);

/* Workspace bytes fconv2d_pool_sigmoid_sum_det_ex needs (0 for an empty
 * pooled map).  Host only; errors as the call itself (NULL bytes: EINVAL). */
int fconv2d_pool_sigmoid_sum_det_workspace_ex(int64_t B, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                                              int64_t K, int64_t pool, int pool_mode, int flags, int algo,
                                              size_t* bytes);

/* PH, PW of the generalised pool (FCONV_CEIL_MODE in flags selects ceil;
 * FCONV_RELU is accepted and ignored).  Host only.  FCONV_EINVAL on sizes
 * < 1, H < K, W < K or an unknown flag bit. */
int fconv2d_pool_out_size_ex(int64_t H, int64_t W, int64_t K, int64_t pool, int flags, int64_t* PH,
                             int64_t* PW);

/*
 * dwsep_conv1d
 *
 *   y[b,o,t] = b_pw[o] + sum_{c < C} w_pw[o,c] * D[b,c,t]
 *   D[b,c,t] = sum_{k < K} w_dw[c,k] * x[b,c,t+k-pad]   (x read as 0 outside [0,T))
 *   Tout = T + 2*pad - K + 1, t < Tout.  No depthwise bias.
 *
 *   x     [B, C, T]
 *   w_dw  [C, K]     (PyTorch's depthwise weight [C,1,K])
 *   w_pw  [O, C]     (PyTorch's pointwise weight [O,C,1])
 *   b_pw  [O], or NULL for no bias
 *   y     [B, O, Tout], fully overwritten
 *
 * FCONV_EINVAL when: x, w_dw, w_pw or y is NULL; any of B, C, T, O, K is
 * < 1; pad < 0; Tout < 1; an element count overflows int64.
 * FCONV_EUNSUPPORTED when C*T, O*Tout or C*K exceeds 2^31-1, O*C or T is
 * 2^29 or more, B > 65535, O > 2^20, or K is so wide that the depthwise
 * window does not fit the kernel's LDS tile (K above roughly 500).
 */
int dwsep_conv1d(const float* x, int64_t B, int64_t C, int64_t T, const float* w_dw, int64_t K,
                 const float* w_pw, int64_t O, const float* b_pw, int64_t pad, float* y,
                 void* stream);

/* Tout for dwsep_conv1d, or -1 if the arguments are invalid.  Host only. */
int64_t dwsep_conv1d_out_len(int64_t T, int64_t K, int64_t pad);

/*
 * dwsep_conv1d_ex -- dwsep_conv1d with a depthwise stride and dilation
 * (PyTorch Conv1d semantics; the l2_p7 trace parametrises the stride):
 *   D[b,c,t] = sum_{k < K} w_dw[c,k] * x[b,c, t*stride + k*dilation - pad]
 *   Tout = floor((T + 2*pad - dilation*(K-1) - 1) / stride) + 1
 * The pointwise stage and the bias are as in dwsep_conv1d.  stride = dilation
 * = 1 is exactly dwsep_conv1d.  FCONV_EINVAL additionally for stride < 1 or
 * dilation < 1; FCONV_EUNSUPPORTED additionally when pad, stride or
 * dilation*(K-1) is 2^29 or more, or the strided input window of even the
 * narrowest time tile does not fit in LDS.
 */
int dwsep_conv1d_ex(const float* x, int64_t B, int64_t C, int64_t T, const float* w_dw, int64_t K,
                    const float* w_pw, int64_t O, const float* b_pw, int64_t pad, int64_t stride,
                    int64_t dilation, float* y, void* stream);

/* Tout for dwsep_conv1d_ex, or -1 if the arguments are invalid.  Host only. */
int64_t dwsep_conv1d_out_len_ex(int64_t T, int64_t K, int64_t pad, int64_t stride, int64_t dilation);

/* Algorithms for the depthwise-separable path (same result up to rounding). */
#define FCONV_DWSEP_AUTO 0      /* = SEPARABLE */
#define FCONV_DWSEP_SEPARABLE 1 /* depthwise into LDS, pointwise GEMM: C*(K+O) MACs per step */
#define FCONV_DWSEP_DENSE 2     /* one convolution with the combined weight
                                   W[o,c,k] = w_pw[o,c]*w_dw[c,k] (the l2_p7 trace's dense-fused
                                   form): C*K*O MACs per step; a comparison path */

/* dwsep_conv1d_ex with an explicit algorithm (FCONV_DWSEP_*).  FCONV_EINVAL
 * for an unknown algorithm; otherwise as dwsep_conv1d_ex. */
int dwsep_conv1d_algo(const float* x, int64_t B, int64_t C, int64_t T, const float* w_dw, int64_t K,
                      const float* w_pw, int64_t O, const float* b_pw, int64_t pad, int64_t stride,
                      int64_t dilation, int algo, float* y, void* stream);

/* Static description of a status code (never NULL). */
const char* fconv_strerror(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fconv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FCONV_H */
