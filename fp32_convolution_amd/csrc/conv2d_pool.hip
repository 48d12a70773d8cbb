// conv2d_pool.hip -- Conv2d (stride 1, no pad) -> AvgPool2d(k = s, floor) -> sigmoid -> sum,
// fused so that neither the conv map nor the pooled map reaches HBM.
//
// Method: POPCORNBENCH reasoning trace "Kimi-K2.6 l2_p65" (Conv2d -> AvgPool2d ->
// Sigmoid -> Sum).  Its fused per-pooled-output formula is used as written:
// a pooled output of channel co is
//     bias[co] + (1/s^2) * sum_{dy,dx < s} sum_{ic,ky,kx} x[ic, ph*s+dy+ky, pw*s+dx+kx] * w[co,ic,ky,kx]
// (the bias factors out of the window average, as the trace notes when it
// accumulates all s*s conv outputs into one running sum).  Because the pool's
// stride equals its kernel, windows do not overlap and every conv output that
// feeds the pool is computed exactly once: s*s*Cin*K*K multiply-adds per
// (co, pooled output).
//
// gfx950 design (not the trace's H100 tiling):
//  * The whole (dy, dx, ic, ky, kx) reduction is one fp32 matrix-core
//    contraction: M = output channels, N = pooled positions,
//    k = Cin*K*K*s*s.  The pool is folded into the reduction, so the
//    accumulators hold window sums directly and no conv value is ever
//    materialised, not even in registers.
//  * v_mfma_f32_16x16x4_f32: the 4 k-slots of an instruction are 4 channel
//    groups (lane group g = l/16 reads channel g*CINQ + q), so every operand
//    address is a per-lane base plus a compile-time immediate: no address
//    arithmetic in the inner loop.
//  * The input tile (all channels, tile + K-1 halo) sits in LDS with its
//    columns split by phase (column c stored at phase c%s, slot c/s), so the
//    16 lanes of a group that read 16 horizontally adjacent pooled positions
//    (stride s in x) hit 16 consecutive LDS words.
//  * Weights stream from L2/L1 straight into registers (they are 18-200 KB).
//  * Epilogue: scale by 1/s^2, add bias, sigmoid, lane sum, wave + LDS
//    reduction, one partial sum per workgroup (added in a fixed order into
//    out[b] by reduce_partials).
// Instances: K5/s3, K3/s2, K3/s3.  K3/s4, and K3/s2 up to 16 channels, run
// on conv2d_pool_elem_kernel (conv2d_pool_ex.hip), which keeps each conv
// output in an accumulator and pools in registers: the same multiply-adds,
// measured faster there.
#include "fconv_device.hpp"
#include "fconv_internal.hpp"

namespace fconv {

// ---------------------------------------------------------------- MFMA direct conv

// Compile-time tiling of one instance.
//   K, S      conv kernel and pool size
//   CB        16-channel output blocks per wave
//   P         16-position pooled blocks per wave
//   WCO,WPOS  waves along output channels / along pooled positions
//   TPH,TPW   pooled tile of the workgroup (TPH*TPW = 16*P*WPOS)
template <int K_, int S_, int CB_, int P_, int WCO_, int WPOS_, int TPH_, int TPW_>
struct DirectCfg {
    static constexpr int K = K_, S = S_, CB = CB_, P = P_, WCO = WCO_, WPOS = WPOS_, TPH = TPH_, TPW = TPW_;
    static constexpr int NW = WCO * WPOS;
    static constexpr int NT = 64 * NW;
    static constexpr int IH = TPH * S + K - 1;  // input rows of the tile
    static constexpr int IW = TPW * S + K - 1;  // input columns of the tile
    static constexpr int QP = (IW + S - 1) / S; // LDS slots per phase
    static constexpr int RP = S * QP;           // LDS floats per input row
    static constexpr int NBV = S + K - 1;       // distinct input offsets per axis inside a window
    static constexpr int CO_RANGE = 16 * CB * WCO;
    static_assert(TPH * TPW == 16 * P * WPOS, "tile must hold the waves' position blocks");
};

template <class Cfg, int MODE, bool WALK>
__global__ __launch_bounds__(Cfg::NT) void conv2d_pool_mfma_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ dst, int Cin, int H, int W, int Cout, int PH, int PW, int CINQ, int plane,
    int tiles_w, int tiles, int units, int parts) {
    constexpr int K = Cfg::K, S = Cfg::S, CB = Cfg::CB, P = Cfg::P, WCO = Cfg::WCO;
    constexpr int TPH = Cfg::TPH, TPW = Cfg::TPW, IH = Cfg::IH, IW = Cfg::IW;
    constexpr int QP = Cfg::QP, RP = Cfg::RP, NBV = Cfg::NBV;
    constexpr int NR = S + K - 1;  // input rows a pooled row's windows touch

    extern __shared__ float lds[];
    __shared__ float red[Cfg::NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wco = wave % WCO;
    const int wpos = wave / WCO;
    const int g = lane >> 4;   // k-slot of the MFMA: channel group
    const int l16 = lane & 15; // row of A / column of B
    // Workgroup `part` of batch item b walks units part, part + parts, ...
    // of the item (unit = channel range * tiles + tile), so that a fused sum
    // adds at most `parts` partials into out[b].
    const int b = blockIdx.x / parts;
    const int part = blockIdx.x - b * parts;
    walk_sum_t<WALK> dsum = 0;  // this lane's sigmoids over all its units
    for (int u = part;; u += parts) {
        if (WALK && u != part) __syncthreads();  // every wave is done with the last unit's tile
        const int cr = u / tiles, tile = u - (u / tiles) * tiles;
        const int tile_y = tile / tiles_w;
        const int tile_x = tile - tile_y * tiles_w;
        const int y0 = tile_y * TPH * S, x0 = tile_x * TPW * S;
        const int co0 = cr * Cfg::CO_RANGE + wco * 16 * CB;

        const buf_rsrc rw = make_rsrc(w, Cout * Cin * K * K * 4);

        // Weights of channel quad q for this lane: a[ky][cb][kx] =
        // w[co0 + cb*16 + l16, g*CINQ + q, ky, kx], 0 where co or ic is out of range.
        auto load_a = [&](float (&a)[K][CB][K], int q) {
            const int ic = g * CINQ + q;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int co = co0 + cb * 16 + l16;
                const bool ok = (co < Cout) && (ic < Cin) && (q < CINQ);
                const int base = ok ? (co * Cin + ic) * (K * K * 4) : kBufOOB;
#pragma unroll
                for (int ky = 0; ky < K; ++ky)
#pragma unroll
                    for (int kx = 0; kx < K; ++kx) a[ky][cb][kx] = buf_load_f32(rw, base + (ky * K + kx) * 4);
            }
        };
        float a_cur[K][CB][K], a_nxt[K][CB][K];
        load_a(a_cur, 0);  // in flight while the tile is staged

        // Biases of this lane's output channels co0 + cb*16 + 4g + r (0 where
        // co >= Cout or bias is NULL: the resource is then empty).
        const buf_rsrc rb = make_rsrc(bias, bias ? Cout * 4 : 0);
        float bco[CB][4];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = co0 + cb * 16 + 4 * g + r;
                bco[cb][r] = buf_load_f32(rb, co < Cout ? co * 4 : kBufOOB);
            }

        // Stage the input tile: channel ic at ic*plane, row r at r*RP, column c at
        // phase (c % S)*QP + slot c/S.  Each wave copies whole rows: the row's
        // address and bounds live in a buffer resource built in scalar registers
        // (empty for rows outside the image and channels >= Cin, so they load
        // as 0), and each lane's column offset is fixed for the whole tile, so a
        // row costs its loads, one address add and its LDS writes.
        {
            constexpr int NCH = (IW + 63) / 64;  // 64-column chunks per row
            constexpr int UR = 4;                // rows in flight per wave
            int voff[NCH], loff[NCH];
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                const int c = lane + 64 * k;
                voff[k] = (c < IW && x0 + c < W) ? (x0 + c) * 4 : kBufOOB;
                loff[k] = (c < IW) ? (c % S) * QP + c / S : -1;
            }
            const int wave_s = __builtin_amdgcn_readfirstlane(wave);
            const int nrows = 4 * CINQ * IH;
            const float* xb = x + (size_t)b * Cin * H * W;
            for (int row0 = wave_s; row0 < nrows; row0 += Cfg::NW * UR) {
                float v[UR][NCH];
#pragma unroll
                for (int u = 0; u < UR; ++u) {
                    const int row = row0 + u * Cfg::NW;
                    const int ic = row / IH, r = row - (row / IH) * IH;
                    const bool ok = (row < nrows) && (ic < Cin) && (y0 + r < H);
                    const buf_rsrc rrow = make_rsrc(xb + (ok ? (ic * H + y0 + r) * W : 0), ok ? W * 4 : 0);
#pragma unroll
                    for (int k = 0; k < NCH; ++k) v[u][k] = buf_load_f32(rrow, voff[k]);
                }
#pragma unroll
                for (int u = 0; u < UR; ++u) {
                    const int row = row0 + u * Cfg::NW;
                    if (row < nrows) {
                        const int ic = row / IH, r = row - (row / IH) * IH;
                        float* lrow = lds + ic * plane + r * RP;
#pragma unroll
                        for (int k = 0; k < NCH; ++k)
                            if (loff[k] >= 0) lrow[loff[k]] = v[u][k];
                    }
                }
            }
        }
        __syncthreads();

        int pbase[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int j = (wpos * P + p) * 16 + l16;
            const int py = j / TPW, px = j - (j / TPW) * TPW;
            pbase[p] = g * CINQ * plane + py * S * RP + px;
        }

        floatx4 acc[CB][P];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int p = 0; p < P; ++p) acc[cb][p] = floatx4{0.f, 0.f, 0.f, 0.f};

        // Input row rr of a window (0 <= rr < S+K-1) is shared by every (ky, dy)
        // with ky + dy = rr: it is read from LDS once and multiplied by each of
        // those weight rows.  The next row (and the next quad's weights) load
        // while the current row's matrix instructions run.
        auto load_row = [&](float (&bv)[P][NBV], int lq, int rr) {
#pragma unroll
            for (int p = 0; p < P; ++p)
#pragma unroll
                for (int cc = 0; cc < NBV; ++cc) bv[p][cc] = lds[pbase[p] + lq + rr * RP + (cc % S) * QP + cc / S];
        };

        for (int q = 0; q < CINQ; ++q) {
            const int lq = q * plane;
            load_a(a_nxt, q + 1);  // zeros past the last quad
            float bcur[P][NBV], bnxt[P][NBV];
            load_row(bcur, lq, 0);
#pragma unroll
            for (int rr = 0; rr < NR; ++rr) {
                if (rr + 1 < NR) load_row(bnxt, lq, rr + 1);
#pragma unroll
                for (int ky = 0; ky < K; ++ky) {
                    const int dy = rr - ky;
                    if (dy < 0 || dy >= S) continue;
#pragma unroll
                    for (int kx = 0; kx < K; ++kx)
#pragma unroll
                        for (int dx = 0; dx < S; ++dx)
#pragma unroll
                            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                                for (int p = 0; p < P; ++p)
                                    acc[cb][p] = mfma_16x16x4(a_cur[ky][cb][kx], bcur[p][dx + kx], acc[cb][p]);
                }
                if (rr + 1 < NR) {
#pragma unroll
                    for (int p = 0; p < P; ++p)
#pragma unroll
                        for (int cc = 0; cc < NBV; ++cc) bcur[p][cc] = bnxt[p][cc];
                }
            }
#pragma unroll
            for (int ky = 0; ky < K; ++ky)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int kx = 0; kx < K; ++kx) a_cur[ky][cb][kx] = a_nxt[ky][cb][kx];
        }

        // Epilogue.  Lane (g, l16) holds, for block (cb, p) and r = 0..3, the
        // window sum of output channel co0 + cb*16 + 4g + r at pooled position
        // j = (wpos*P + p)*16 + l16 of the tile.
        const float inv = 1.0f / (float)(S * S);
        const int ph0 = tile_y * TPH, pw0 = tile_x * TPW;
        float lsum = 0.f;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = co0 + cb * 16 + 4 * g + r;
                const bool cok = co < Cout;
#pragma unroll
                for (int p = 0; p < P; ++p) {
                    const int j = (wpos * P + p) * 16 + l16;
                    const int ph = ph0 + j / TPW, pw = pw0 + (j - (j / TPW) * TPW);
                    if (cok && ph < PH && pw < PW) {
                        const float avg = acc[cb][p][r] * inv + bco[cb][r];
                        if constexpr (MODE == OUT_MAP)
                            dst[(((size_t)b * Cout + co) * PH + ph) * PW + pw] = avg;
                        else
                            lsum += logistic(avg);
                    }
                }
            }
        dsum += lsum;
        if (!WALK || u + parts >= units) break;
    }  // units
    if constexpr (MODE != OUT_MAP) {
        const float s = block_sum<Cfg::NW>((float)dsum, red);
        if (tid == 0) dst[(size_t)b * parts + part] = s;
    }
}

// Instances (tilings measured on MI355X).  K3/s2 and K3/s3: a 4x16 pooled
// tile, 4 waves each owning 16 output channels of a 64-channel range and all
// 64 positions.  K5/s3: a 4x12 tile (84 = 21*4 = 7*12, so an 84x84 map has no
// ragged tiles), 8 waves of 16 channels each.  K3/s4 runs on the
// per-conv-output kernel of conv2d_pool_ex.hip (same multiply-adds; it
// measured 4 % faster than this kernel's 4x16 instance: it skips the padded
// pooled rows of a ragged tile and its row-major tile has no bank conflicts).
// The FCONV_CFG_* macros let a build override an instance's tiling.
#ifndef FCONV_CFG_K5S3
#define FCONV_CFG_K5S3 5, 3, 1, 3, 8, 1, 4, 12
#endif
using CfgK5S3 = DirectCfg<FCONV_CFG_K5S3>;
using CfgK3S2 = DirectCfg<3, 2, 1, 4, 4, 1, 4, 16>;
using CfgK3S3 = DirectCfg<3, 3, 1, 4, 4, 1, 4, 16>;

template <class Cfg>
static int plane_floats(int CINQ) {
    // Pad each channel plane so that the 4 lane groups (which read planes
    // g*CINQ*plane apart) fall on different LDS banks where possible.
    const int base = Cfg::IH * Cfg::RP;
    for (int pad = 0; pad < 32; ++pad)
        if (((long)CINQ * (base + pad)) % 32 == 16) return base + pad;
    return base;
}

template <class Cfg>
static size_t lds_bytes_for(int Cin) {
    const int CINQ = (Cin + 3) / 4;
    return (size_t)4 * CINQ * plane_floats<Cfg>(CINQ) * sizeof(float);
}

static constexpr size_t kMaxLds = 160 * 1024 - 256;  // dynamic share; the rest holds the reduction slots

// The pool-folded direct kernel takes (Cin, K, S): its instance exists, one
// workgroup's tile of all Cin channels fits LDS, and it is the faster of the
// two direct kernels there.  For K3/s2 up to 16 channels the per-conv-output
// kernel's 4 x 32 tiles (its own folded average pool) ran faster: 1.2552
// against 1.4481 ms on x[128,8,384,384] -> 64 and 1.1337 against 1.2006 ms on
// x[64,16,257,257] -> 128, but 0.7845 against 0.6578 ms with Cin = 32
// (interleaved A/B); for K3/s3 it was slower at every Cin tried.
static bool direct_fits(int Cin, int K, int S) {
    size_t bytes = 0;
    if (K == 5 && S == 3) bytes = lds_bytes_for<CfgK5S3>(Cin);
    else if (K == 3 && S == 2) {
        if (Cin <= 16) return false;
        bytes = lds_bytes_for<CfgK3S2>(Cin);
    }
    else if (K == 3 && S == 3) bytes = lds_bytes_for<CfgK3S3>(Cin);
    else return false;
    return bytes <= kMaxLds;
}

// Direct MFMA: K3/s4, and K3/s2 up to 16 channels, run on the
// per-conv-output kernel; K5/s3, K3/s2 and K3/s3 otherwise on the pool-folded
// kernel while its tile fits, else on the per-conv-output kernel's
// channel-chunked tiling (any Cin).
bool conv2d_mfma_supported(int Cin, int K, int S) {
    return direct_fits(Cin, K, S) || conv2d_elem_supported(Cin, K, S);
}

// Instantiates a kernel template for the three output modes and launches
// the one `mode` asks for, raising the dynamic LDS limit first.
#define FCONV_LAUNCH_MODES(KERNEL, GRID, BLOCK, LDS, STREAM, ...)                                            \
    do {                                                                                                 \
        const void* fn = mode == OUT_MAP ? (const void*)KERNEL<OUT_MAP> : (const void*)KERNEL<OUT_PARTIAL>; \
        if ((LDS) > 0) {                                                                                 \
            hipError_t ea = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)(LDS)); \
            if (ea != hipSuccess) return ea;                                                             \
        }                                                                                                \
        if (mode == OUT_MAP)                                                                             \
            hipLaunchKernelGGL((KERNEL<OUT_MAP>), GRID, BLOCK, LDS, STREAM, __VA_ARGS__);                \
        else                                                                                             \
            hipLaunchKernelGGL((KERNEL<OUT_PARTIAL>), GRID, BLOCK, LDS, STREAM, __VA_ARGS__);            \
        return hipGetLastError();                                                                        \
    } while (0)

// The same for a kernel template KERNEL<MODE, WALK>: the WALK instance (each
// workgroup walks several units) when there are more units than workgroups.
#define FCONV_LAUNCH_WALK(KERNEL, WALK, GRID, BLOCK, LDS, STREAM, ...)                                      \
    do {                                                                                                 \
        if (WALK) {                                                                                      \
            FCONV_LAUNCH_MODES(KERNEL##_walk, GRID, BLOCK, LDS, STREAM, __VA_ARGS__);                    \
        } else {                                                                                         \
            FCONV_LAUNCH_MODES(KERNEL##_once, GRID, BLOCK, LDS, STREAM, __VA_ARGS__);                    \
        }                                                                                                \
    } while (0)

template <class Cfg>
struct DirectLaunch {
    template <int MODE>
    static constexpr auto kernel_once = conv2d_pool_mfma_kernel<Cfg, MODE, false>;
    template <int MODE>
    static constexpr auto kernel_walk = conv2d_pool_mfma_kernel<Cfg, MODE, true>;
};

// Units of work of one batch item: pooled tiles x output-channel ranges.
// A tile's pooled count fits int32 and so does the item's pooled map, which
// holds at least one output per unit.
struct Walk {
    int tiles_w, tiles, co_ranges, units, parts;
};

template <int TPH, int TPW, int CO_RANGE>
static Walk make_walk(const Conv2dShape& s) {
    Walk k;
    k.tiles_w = (s.PW + TPW - 1) / TPW;
    k.tiles = ((s.PH + TPH - 1) / TPH) * k.tiles_w;
    k.co_ranges = (s.Cout + CO_RANGE - 1) / CO_RANGE;
    k.units = k.tiles * k.co_ranges;
    k.parts = walk_parts(k.units);
    return k;
}

template <class Cfg>
static Walk direct_walk(const Conv2dShape& s) {
    return make_walk<Cfg::TPH, Cfg::TPW, Cfg::CO_RANGE>(s);
}

template <class Cfg>
static hipError_t launch_direct(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                                float* dst, int mode, hipStream_t stream) {
    const int CINQ = (s.Cin + 3) / 4;
    const int plane = plane_floats<Cfg>(CINQ);
    const size_t lds = (size_t)4 * CINQ * plane * sizeof(float);
    const Walk k = direct_walk<Cfg>(s);
    // at most 65535 * 1024 workgroups
    const dim3 grid((unsigned)k.parts * (unsigned)s.B);
    FCONV_LAUNCH_WALK(DirectLaunch<Cfg>::template kernel, k.units > k.parts, grid, dim3(Cfg::NT), lds, stream, x, w, bias, dst, s.Cin,
                       s.H, s.W, s.Cout, s.PH, s.PW, CINQ, plane, k.tiles_w, k.tiles, k.units, k.parts);
}

hipError_t conv2d_mfma_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                              float* dst, int mode, hipStream_t stream) {
    if (!direct_fits(s.Cin, s.K, s.S))
        return conv2d_elem_launch(s, x, w, bias, dst, mode, PoolOpts{false, false, false}, stream);
    if (s.K == 5 && s.S == 3) return launch_direct<CfgK5S3>(s, x, w, bias, dst, mode, stream);
    if (s.K == 3 && s.S == 2) return launch_direct<CfgK3S2>(s, x, w, bias, dst, mode, stream);
    if (s.K == 3 && s.S == 3) return launch_direct<CfgK3S3>(s, x, w, bias, dst, mode, stream);
    return hipErrorInvalidValue;
}

int64_t conv2d_mfma_parts(const Conv2dShape& s) {
    if (!direct_fits(s.Cin, s.K, s.S)) return conv2d_elem_parts(s, PoolOpts{false, false, false});
    if (s.K == 5 && s.S == 3) return direct_walk<CfgK5S3>(s).parts;
    if (s.K == 3 && s.S == 2) return direct_walk<CfgK3S2>(s).parts;
    if (s.K == 3 && s.S == 3) return direct_walk<CfgK3S3>(s).parts;
    return -1;
}

// ---------------------------------------------------------------- box-sum variant

// Pooling commutes with the convolution: the window sum of conv outputs is
//     sum_{dy,dx<s} conv[ph*s+dy, pw*s+dx] - s^2*bias
//   = sum_{ic,ky,kx} w[co,ic,ky,kx] * Sx[ic, ph*s+ky, pw*s+kx],
//     Sx[ic,y,x] = sum_{dy,dx<s} x[ic, y+dy, x+dx],
// (the linearity behind the trace's bias factoring, applied to the whole
// sum), so after s x s box sums of the input each (co, pooled output) needs
// Cin*K*K multiply-adds instead of s^2*Cin*K*K.  The result equals the
// direct form up to rounding.
//
// Workgroup: one batch item, a TPH x TPW pooled tile, all WCO*16*CB output
// channels of a range, every wave covering all positions (WPOS must be 1).
//  1. Each wave loads all IH rows of a channel's tile into registers (many
//     loads in flight: the kernel is HBM-bound), adds s consecutive rows in
//     registers and writes those vertical sums V[ic][r][c] to LDS.
//  2. Sx[ic][r][c] = sum_{dx<s} V[ic][r][c+dx] into a phase-split buffer
//     (column c at phase c % s, slot c/s, as the direct kernel's tile).
//  3. MFMA contraction over (ic, ky, kx) with the direct kernel's channel
//     grouping of the 4 k-slots.  Same epilogue.
// Blocks are numbered so that consecutive tiles land on the same XCD (blocks
// are dealt to the 8 XCDs round-robin), where they share halo lines in L2.
template <class Cfg>
struct BoxLayout {
    static constexpr int K = Cfg::K, S = Cfg::S;
    static constexpr int RS = (Cfg::TPH - 1) * S + K;  // rows of Sx the tile needs
    static constexpr int CS = (Cfg::TPW - 1) * S + K;  // columns of Sx the tile needs
    static constexpr int NCH = (Cfg::IW + 63) / 64;     // 64-column chunks of an input row
    static constexpr int NCS = (CS + 63) / 64;          // 64-column chunks of an Sx row
    static constexpr int QS = (CS + S - 1) / S;         // Sx slots per phase
    // Lanes and banks.  With PATCH, block p's 16 lanes (l = 0..15) read the
    // 4 x 4 patch of pooled positions (l / 4, 4p + l % 4) of the 4-row tile,
    // and the Sx row stride RSS satisfies S * RSS = 4 (mod 64): the 16 lanes
    // then read 16 consecutive LDS banks, and channel planes padded to 16
    // (mod 64) put the four lane groups (four channels) on disjoint banks.
    // PATCH needs a 4-row tile, a width that is a multiple of 4, and at most
    // 16 floats of row padding; otherwise block p holds positions
    // 16p .. 16p+15 in row order and RSS = S * QS.
    static constexpr int rss_patch() {
        for (int r = S * QS; r < S * QS + 64; ++r)
            if ((S * r) % 64 == 4) return r;
        return -1;
    }
    static constexpr bool PATCH = Cfg::TPH == 4 && Cfg::TPW % 4 == 0 && rss_patch() >= 0 && rss_patch() - S * QS <= 16;
    static constexpr int RSS = PATCH ? rss_patch() : S * QS;  // Sx floats per row
    // channel planes 16 or 48 (mod 64) apart: either puts the four lane
    // groups on four disjoint 16-bank sets; the nearer one is taken (in row
    // order too, where a block's 16 lanes read 16 consecutive words: K3/s3's
    // unpadded 576-word planes put all four groups on the same banks)
    static constexpr int pad_to(int n, int m) { return (m - n % 64 + 64) % 64; }
    static constexpr int SPLANE =
        RS * RSS + (pad_to(RS * RSS, 16) < pad_to(RS * RSS, 48) ? pad_to(RS * RSS, 16) : pad_to(RS * RSS, 48));
    // horizontal sums by DPP wave shifts (one 64-column chunk per row, s = 2
    // or 3), else through one vertical-sum row of LDS per wave
    static constexpr bool DPP_H = NCH == 1 && (S == 2 || S == 3);
    static constexpr int SCRATCH = DPP_H ? 0 : NCH * 64;
    static constexpr int CC = 2 * Cfg::NW;              // channels per LDS chunk: two per wave
    static constexpr int QC = CC / 4;                   // channel quads per chunk
    static_assert(Cfg::WPOS == 1, "box-sum waves split output channels only");
    static_assert(QC % 2 == 0, "a chunk's quads run in weight-buffer pairs");
};

// Waves per SIMD the register budget must allow.  The K = 5, s = 3 instance
// (8-wave workgroups, 37 KB of LDS) is held to 80 VGPRs so that 3 workgroups
// fit a CU instead of 2: 0.398 against 0.434 ms on x[64,16,257,257] (0.412
// with 73 VGPRs when its weight buffers were copied rather than alternated);
// at 64 VGPRs (4 workgroups) its spills made it 0.467 ms.
#ifndef FCONV_BOX_K5S3_MIN_WAVES
#define FCONV_BOX_K5S3_MIN_WAVES 6
#endif
// The 4-wave K3/s2 and K3/s3 instances are held to 8 waves per SIMD (64
// VGPRs: 58-61 used, no VGPR spills; 5-9 SGPRs kept in VGPR lanes):
// unbounded, the compiler took 100
// registers (accumulators in AGPRs) and 4 waves per SIMD, and these short
// workgroups (36 MFMAs per channel quad and wave) had too few waves to hide
// their loads and barriers: 0.4384 against 0.4538 ms for K3/s2 and 0.2422
// against 0.2517 ms for K3/s3 on x[128,8,384,384] -> 64 channels, 0.0998
// against 0.1081 ms for K3/s3 on x[32,32,256,256] (interleaved A/B).
template <class Cfg>
constexpr int box_min_waves() {
    if (Cfg::K == 3 && (Cfg::S == 2 || Cfg::S == 3) && Cfg::NW == 4) return 8;
    return Cfg::K == 5 && Cfg::S == 3 ? FCONV_BOX_K5S3_MIN_WAVES : 1;
}

template <class Cfg, int MODE, bool WALK>
__global__ __launch_bounds__(Cfg::NT, box_min_waves<Cfg>()) void conv2d_pool_boxsum_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ dst, int Cin, int H, int W, int Cout, int PH, int PW, int CINQ, int tiles_w,
    int tiles, int units, int parts, int nblocks) {
    using L = BoxLayout<Cfg>;
    constexpr int K = Cfg::K, S = Cfg::S, CB = Cfg::CB, P = Cfg::P, NW = Cfg::NW;
    constexpr int TPH = Cfg::TPH, TPW = Cfg::TPW, IH = Cfg::IH, IW = Cfg::IW;
    constexpr int RS = L::RS, CS = L::CS, QS = L::QS, RSS = L::RSS;

    constexpr int CC = L::CC, QC = L::QC;
    extern __shared__ float lds[];
    __shared__ float red[NW];
    float* Sb = lds;                                        // [CC][RS][RSS] phase-split
    float* scratch = lds + CC * L::SPLANE;                  // [NW][SCRATCH]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    // The tile position (row py, column px) lane l16 holds in block p.
    auto tile_pos = [&](int p, int& py, int& px) {
        if constexpr (L::PATCH) {
            py = l16 >> 2;
            px = 4 * p + (l16 & 3);
        } else {
            const int j = p * 16 + l16;
            py = j / TPW;
            px = j - (j / TPW) * TPW;
        }
    };
    // Workgroup `part` of batch item b walks units part, part + parts, ...
    // (unit = channel range * tiles + tile).
    const int lid = xcd_spread(blockIdx.x, nblocks);
    const int b = lid / parts;
    const int part = lid - b * parts;
    walk_sum_t<WALK> dsum = 0;  // this lane's sigmoids over all its units
    for (int u = part;; u += parts) {
        if (WALK && u != part) __syncthreads();  // every wave is done with the last unit's box sums
        const int cr = u / tiles, tile = u - (u / tiles) * tiles;
        const int tile_y = tile / tiles_w, tile_x = tile - (tile / tiles_w) * tiles_w;
        const int y0 = tile_y * TPH * S, x0 = tile_x * TPW * S;
        const int co0 = cr * Cfg::CO_RANGE + wave * 16 * CB;

        const buf_rsrc rw = make_rsrc(w, Cout * Cin * K * K * 4);
        // Weights of quad q for lane (g, l16): channel 4q + g (0 past Cin,
        // Cout and CINQ).
        auto load_a = [&](float (&a)[K * K][CB], int q) {
            const int ic = 4 * q + g;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const int co = co0 + cb * 16 + l16;
                const bool ok = (co < Cout) && (ic < Cin) && (q < CINQ);
                const int base = ok ? (co * Cin + ic) * (K * K * 4) : kBufOOB;
#pragma unroll
                for (int kk = 0; kk < K * K; ++kk) a[kk][cb] = buf_load_f32(rw, base + kk * 4);
            }
        };
        float a_cur[K * K][CB], a_nxt[K * K][CB];
        load_a(a_cur, 0);
        const buf_rsrc rb = make_rsrc(bias, bias ? Cout * 4 : 0);
        float bco[CB][4];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = co0 + cb * 16 + 4 * g + r;
                bco[cb][r] = buf_load_f32(rb, co < Cout ? co * 4 : kBufOOB);
            }

        // 1-2. Box sums, one channel per wave at a time, CC = 2*NW channels
        //      (QC quads) per LDS chunk: wave w makes those of the chunk's
        //      channels w and w + NW.  All IH rows of the channel's tile are
        //      loaded into registers (the second channel's rows load while the
        //      first one is summed); s rows are added in registers; each
        //      vertical-sum row goes through the wave's own LDS scratch row and
        //      comes back shifted by 0..s-1 columns for the horizontal sum.
        //      LDS operations of one wave complete in order, so the scratch row
        //      needs no workgroup barrier, only compiler fences.
        constexpr int NCH = L::NCH, NCS = L::NCS;
        int voff[NCH];
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int c = lane + 64 * k;
            voff[k] = (c < IW && x0 + c < W) ? (x0 + c) * 4 : kBufOOB;
        }
        int soff[NCS];
#pragma unroll
        for (int k = 0; k < NCS; ++k) {
            const int c = lane + 64 * k;
            soff[k] = c < CS ? (c % S) * QS + c / S : -1;
        }
        const float* xb = x + (size_t)b * Cin * H * W;
        float* srow = scratch + wave * L::SCRATCH;
        // Row r of channel ic: rows past the image and channels past Cin get
        // an empty resource (their loads return 0 and touch no memory), so
        // the row pointer needs no condition: one scalar add per row.
        auto load_rows = [&](float (&vv)[IH][NCH], int ic) {
            const bool cok = ic < Cin;
            const float* prow = xb + ((size_t)(cok ? ic : 0) * H + y0) * W;
#pragma unroll
            for (int r = 0; r < IH; ++r, prow += W) {
                const bool ok = cok && (y0 + r < H);
                const buf_rsrc rrow = make_rsrc(prow, ok ? W * 4 : 0);
#pragma unroll
                for (int k = 0; k < NCH; ++k) vv[r][k] = buf_load_f32(rrow, voff[k]);
            }
        };
        // into LDS slot `slot` of the chunk
        // With one 64-column chunk per row (NCH = 1) and s = 2 or 3, lane c
        // takes its neighbours' vertical sums with DPP wave shifts, which fold
        // into the adds: h = v + shl(v) for s = 2, h = v + shl(v + shl(v))
        // for s = 3.  Otherwise they go through the wave's LDS scratch row.
        constexpr bool DPP_H = L::DPP_H;
        auto sum_rows = [&](float (&vv)[IH][NCH], int slot) {
            float* splane = Sb + slot * L::SPLANE;
            if constexpr (DPP_H) {
                // All rows first, then one store branch: with a branch per
                // row the compiler sank each row's last add into it, where
                // the shift's source lane may be inactive, so every shift
                // stayed a move of its own (with its hazard wait) and every
                // row paid an exec-mask save and restore.  The empty register
                // constraint keeps the sums ahead of the branch.
                float hv[RS];
#pragma unroll
                for (int r = 0; r < RS; ++r) {
                    float v = vv[r][0];
#pragma unroll
                    for (int dy = 1; dy < S; ++dy) v += vv[r + dy][0];
                    hv[r] = S == 2 ? v + wave_shl1(v) : v + wave_shl1(v + wave_shl1(v));
                }
#pragma unroll
                for (int r = 0; r < RS; ++r) asm volatile("" : "+v"(hv[r]));
                if (lane < CS) {
#pragma unroll
                    for (int r = 0; r < RS; ++r) splane[r * RSS + soff[0]] = hv[r];
                }
                return;
            }
#pragma unroll
            for (int r = 0; r < RS; ++r) {
                // The fences keep the compiler from moving this row's reads
                // above its writes (or the next row's writes above these
                // reads): other lanes' values are exchanged through srow.
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int k = 0; k < NCH; ++k) {
                    float sum = vv[r][k];
#pragma unroll
                    for (int dy = 1; dy < S; ++dy) sum += vv[r + dy][k];
                    srow[lane + 64 * k] = sum;
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int k = 0; k < NCS; ++k) {
                    const int c = lane + 64 * k;
                    if (c < CS) {
                        float sum = srow[c];
#pragma unroll
                        for (int dx = 1; dx < S; ++dx) sum += srow[c + dx];
                        splane[r * RSS + soff[k]] = sum;
                    }
                }
            }
        };

        // 3. contraction: B for lane (g, l16), block p, tap (ky, kx) and the
        //    chunk's quad j is Sx[slot 4j + g][py*S + ky][px*S + kx] for the
        //    lane's position (py, px) of block p.
        int pbase[P];
#pragma unroll
        for (int p = 0; p < P; ++p) {
            int py, px;
            tile_pos(p, py, px);
            pbase[p] = g * L::SPLANE + py * S * RSS + px;
        }
        floatx4 acc[CB][P];
        // Each quad's reads come off base registers the compiler cannot
        // relate to one another, so that paired LDS reads take their taps
        // and blocks as immediate offsets (with PATCH one base: block p is 4p
        // words on, and a quad's reads span under 256 words) instead of an
        // address add per pair.
        auto contract = [&](const float (&a)[K * K][CB], int jq) {
            const int lq = 4 * jq * L::SPLANE;
            lds_fptr qb[P];
#pragma unroll
            for (int p = 0; p < P; ++p)
                qb[p] = L::PATCH ? (p == 0 ? lds_opaque((lds_fptr)lds + pbase[0] + lq) : qb[0] + 4 * p)
                                 : lds_opaque((lds_fptr)lds + pbase[p] + lq);
#pragma unroll
            for (int ky = 0; ky < K; ++ky)
#pragma unroll
                for (int kx = 0; kx < K; ++kx) {
                    float bv[P];
#pragma unroll
                    for (int p = 0; p < P; ++p) bv[p] = qb[p][ky * RSS + (kx % S) * QS + kx / S];
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                        for (int p = 0; p < P; ++p) acc[cb][p] = mfma_16x16x4(a[ky * K + kx][cb], bv[p], acc[cb][p]);
                }
        };

        float va[IH][NCH], vb[IH][NCH];
        // box sums of chunk c (va holds the rows of its first channel)
        auto box_chunk = [&](int c) {
            load_rows(vb, c * CC + wave + NW);
            sum_rows(va, wave);
            sum_rows(vb, wave + NW);
            __syncthreads();
        };
        // the chunk's quads in pairs, so that the two weight buffers
        // alternate without copies (one copy per weight and group cost 25
        // moves per group); a_cur holds the chunk's first quad on entry and
        // the next chunk's on exit (QC is even)
        auto contract_chunk = [&](int c) {
            const int q0 = c * QC, qend = min(q0 + QC, CINQ);
            for (int q = q0; q < qend; q += 2) {
                load_a(a_nxt, q + 1);
                contract(a_cur, q - q0);
                if (q + 1 < qend) {
                    load_a(a_cur, q + 2);
                    contract(a_nxt, q + 1 - q0);
                }
            }
        };
        // the first chunk on its own, so that the accumulators start after
        // its box sums
        load_rows(va, wave);
        box_chunk(0);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
            for (int p = 0; p < P; ++p) acc[cb][p] = floatx4{0.f, 0.f, 0.f, 0.f};
        contract_chunk(0);
        // Further chunks: the accumulators stay live through the box sums,
        // so those use one row buffer (no prefetch of the second channel).
        const int nchunks = (CINQ + QC - 1) / QC;
        for (int c = 1; c < nchunks; ++c) {
            __syncthreads();  // the last chunk's box sums are read
            load_rows(va, c * CC + wave);
            sum_rows(va, wave);
            load_rows(va, c * CC + wave + NW);
            sum_rows(va, wave + NW);
            __syncthreads();
            contract_chunk(c);
        }

        // Epilogue (as the direct kernel): window sum / s^2 + bias.
        const float inv = 1.0f / (float)(S * S);
        const int ph0 = tile_y * TPH, pw0 = tile_x * TPW;
        float lsum = 0.f;
        static_assert(P * 16 == TPH * TPW, "every lane of every block holds a tile position");
        if (MODE != OUT_MAP && co0 + 16 * CB <= Cout && ph0 + TPH <= PH && pw0 + TPW <= PW) {
            // the whole tile is in range: no per-output tests, and the scale, the
            // bias and -log2(e) of the sigmoid's argument in one multiply-add
            constexpr float kNegLog2e = -1.4426950408889634f;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float c0 = bco[cb][r] * kNegLog2e;
#pragma unroll
                    for (int p = 0; p < P; ++p)
                        lsum += __builtin_amdgcn_rcpf(
                            1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(acc[cb][p][r], inv * kNegLog2e, c0)));
                }
        } else {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int co = co0 + cb * 16 + 4 * g + r;
                    const bool cok = co < Cout;
#pragma unroll
                    for (int p = 0; p < P; ++p) {
                        int py, px;
                        tile_pos(p, py, px);
                        const int ph = ph0 + py, pw = pw0 + px;
                        if (cok && ph < PH && pw < PW) {
                            const float avg = acc[cb][p][r] * inv + bco[cb][r];
                            if constexpr (MODE == OUT_MAP)
                                dst[(((size_t)b * Cout + co) * PH + ph) * PW + pw] = avg;
                            else
                                lsum += logistic(avg);
                        }
                    }
                }
        }
        dsum += lsum;
        if (!WALK || u + parts >= units) break;
    }  // units
    if constexpr (MODE != OUT_MAP) {
        const float s = block_sum<NW>((float)dsum, red);
        if (tid == 0) dst[(size_t)b * parts + part] = s;
    }
}

// ---------------------------------------------------------------- box-sum, K = 3, s = 4, one pooled column per lane

// The box-sum identity above, arranged for K = 3 < s = 4.  The 6 x 6 input
// windows of neighbouring pooled outputs overlap by two rows and columns,
// and each pooled output needs exactly 9 box sums per channel:
//     Sx[ic][ky][kx] at (4ph + ky, 4pw + kx), ky, kx < 3.
// Lane l owns pooled column pw0 + l.  One 16-byte load gives it input
// columns 4pw .. 4pw+3 of a row; the next two columns are the next lane's
// first two, read through DPP wave_shl:1 (lane TPW only supplies them).
// The vertical 4-sums come first, per column: 9 sums of adjacent rows, then
// each window of rows 4ph+ky .. +3 as two of them (15 adds per column for
// both pooled rows).  Then per (ph, ky) 7 adds give the horizontal 4-sums:
//     h0 = (u0+u1) + (u2+u3),  h1 = (u1+u2) + (u3+n0),  h2 = (u2+u3) + (n0+n1).
// That is 114 adds per channel, 12 of which read the next lane's operand
// through a DPP modifier (no move of their own); summing each row across
// first took 138 adds and 20 moves.  The 9 values go to LDS tap-major,
// Sx[ic][ph][tap][pw] (consecutive lanes write and read consecutive words), which the
// contraction reads as B operands, one word per MFMA step.  Each channel's
// plane is padded by 16 words so that the four lane groups, which read four
// channels, start 16 banks apart.  For Cin = 8 that is 28 KB per workgroup,
// and 5 workgroups fit a CU; a position-major [pw][12] layout (three 16-byte
// reads per 9 steps) took 37 KB, 4 per CU, and ran 2 % slower.  Compared
// with the general box-sum kernel this computes only the box sums the pooled
// outputs use (9 of every 16) and issues about half the vector instructions
// per output.
// Workgroup: one batch item, TPH = 2 pooled rows x TPW = 48 pooled columns,
// 64 output channels (4 waves x 16).  k-slot g of contraction step (m, tap)
// is channel 4m + g at tap (ky, kx) = (tap / 3, tap % 3), so lane group g
// reads one channel's 9 taps.  The channels go through LDS in chunks of CQ
// quads (4*CQ channels: 28 KB for CQ = 2), so any channel count fits: wave w
// makes the box sums of channel 4m + w of each quad m of the chunk, then the
// workgroup contracts the chunk's quads, then the next chunk's box sums
// overwrite them.  The next channel's rows load during the current one's
// sums and, across a chunk boundary, during the contraction.  Requires
// W % 4 == 0 (a 16-byte column group is all in or all out of the row); VEC
// selects 16-byte loads (x 16-byte aligned) or four 4-byte loads.
struct Box4 {
    static constexpr int K = 3, S = 4, TPH = 2, TPW = 48, NW = 4, NT = 256;
    static constexpr int IR = TPH * S + K - 1;  // input rows a tile reads: 10
    static constexpr int CO_RANGE = NW * 16;
    // tap-major layout: a channel's [TPH][9][TPW] values plus 16 floats, so
    // that the four lane groups' channels start 16 banks apart
    static constexpr int CPLANE = TPH * 9 * TPW + 16;
};

// Channel quads per LDS chunk: one for a single-quad input, else two.
constexpr int box4_chunk_quads(int NQ) { return NQ == 1 ? 1 : 2; }

// NQ: CINQ when it is 1 or 2 (one chunk, the channel loop unrolled, each
// channel's rows in registers of their own), else 0 (chunks in a run-time
// loop).
template <int MODE, bool VEC, int NQ, bool WALK>
__global__ __launch_bounds__(Box4::NT, 4) void conv2d_pool_boxsum4_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ dst, int Cin, int H, int W, int Cout, int PH, int PW, int CINQ, int tiles_w,
    int tiles, int units, int parts, int nblocks) {
    constexpr int S = Box4::S, TPH = Box4::TPH, TPW = Box4::TPW, NW = Box4::NW, IR = Box4::IR;
    constexpr int CQ = box4_chunk_quads(NQ);
    constexpr int NB = TPH * TPW / 16;  // 16-position blocks of the tile
    extern __shared__ float lds[];      // Sx [4*CQ][CPLANE]: [TPH][9][TPW] + 16 per channel
    __shared__ float red[NW];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, l16 = lane & 15;
    // Workgroup `part` of batch item b walks units part, part + parts, ...
    // (unit = channel range * tiles + tile).
    const int lid = xcd_spread(blockIdx.x, nblocks);
    const int b = lid / parts;
    const int part = lid - b * parts;
    const float* xb = x + (size_t)b * Cin * H * W;
    const buf_rsrc rw = make_rsrc(w, Cout * Cin * 9 * 4);
    const buf_rsrc rb = make_rsrc(bias, bias ? Cout * 4 : 0);
    const int nq = NQ > 0 ? NQ : CINQ;
    walk_sum_t<WALK> dsum = 0;  // this lane's sigmoids over all its units

    for (int u = part;; u += parts) {
        if (WALK && u != part) __syncthreads();  // every wave is done with the last unit's box sums
        const int cr = u / tiles, tile = u - (u / tiles) * tiles;
        const int tile_y = tile / tiles_w, tile_x = tile - (tile / tiles_w) * tiles_w;
        const int ph0 = tile_y * TPH, pw0 = tile_x * TPW;
        const int y0 = ph0 * S, x0 = pw0 * S;
        const int co_w = cr * Box4::CO_RANGE + wave * 16;  // this wave's first output channel

        float bco[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int co = co_w + 4 * g + r;
            bco[r] = buf_load_f32(rb, co < Cout ? co * 4 : kBufOOB);
        }

        const int xc = x0 + 4 * lane;
        const int coff = (lane <= TPW && xc < W) ? xc * 4 : kBufOOB;
        // rows past the image and channels past Cin get an empty resource
        // (their loads return 0), so the row pointer needs no condition
        auto load_rows = [&](floatx4 (&v)[IR], int ic) {
            const bool cok = ic < Cin;
            const float* prow = xb + ((size_t)(cok ? ic : 0) * H + y0) * W;
#pragma unroll
            for (int r = 0; r < IR; ++r, prow += W) {
                const bool ok = cok && y0 + r < H;
                const buf_rsrc rr = make_rsrc(prow, ok ? W * 4 : 0);
                if constexpr (VEC) {
                    v[r] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rr, coff, 0, 0));
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[r][j] = buf_load_f32(rr, coff + 4 * j);
                }
            }
        };
        // the value of lane + 1 (lane 63, whose value no stored sum uses,
        // reads 0)
        auto next_lane = [](float v) { return wave_shl1(v); };
        // A of step (m, tap) for lane (g, l16) is w[co][4m + g][tap], co = this
        // wave's channel l16; 0 past Cin, past Cout and for m >= CINQ.
        const int co_a = co_w + l16;
        auto load_a = [&](float (&a)[9], int m) {
            const int ic = 4 * m + g;
            const int base = (co_a < Cout && ic < Cin && m < CINQ) ? (co_a * Cin + ic) * 36 : kBufOOB;
#pragma unroll
            for (int t = 0; t < 9; ++t) a[t] = buf_load_f32(rw, base + 4 * t);
        };

        floatx4 v[IR];
        load_rows(v, wave);
        float a[CQ][9];
        floatx4 acc[NB];

        // Box sums of this wave's channel of quad c*CQ + j into LDS slot
        // 4j + wave.  The chunk's weights load after its box sums.
        auto load_chunk_a = [&](int c) {
#pragma unroll
            for (int jj = 0; jj < CQ; ++jj) load_a(a[jj], c * CQ + jj);
        };
        auto box_sums = [&](int c, int j) {
            const int i = c * CQ + j;
            const int ic = 4 * i + wave;
            // vertical 4-sums first: column c of the lane's four, window rows
            // 4ph+ky .. 4ph+ky+3 = pair (4ph+ky, +1) + pair (4ph+ky+2, +3)
            float vs[TPH][3][4];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                float p[IR - 1];
#pragma unroll
                for (int r = 0; r + 1 < IR; ++r) p[r] = v[r][cc] + v[r + 1][cc];
#pragma unroll
                for (int ph = 0; ph < TPH; ++ph)
#pragma unroll
                    for (int ky = 0; ky < 3; ++ky) vs[ph][ky][cc] = p[ph * S + ky] + p[ph * S + ky + 2];
            }
            // within a chunk the next channel's rows load now, under this
            // channel's sums; the next chunk's first rows load when that chunk
            // starts (a prefetch across the contraction kept them live
            // together with the accumulators and spilled registers)
            if (j < CQ - 1 && i + 1 < nq) load_rows(v, ic + NW);
            float* sp = lds + (size_t)(4 * j + wave) * Box4::CPLANE + lane;
#pragma unroll
            for (int ph = 0; ph < TPH; ++ph) {
                // then the horizontal 4-sums at kx = 0, 1, 2 (columns 4 and 5
                // are the next lane's 0 and 1)
                float sx[9];
#pragma unroll
                for (int ky = 0; ky < 3; ++ky) {
                    const float* uu = vs[ph][ky];
                    const float p01 = uu[0] + uu[1], p23 = uu[2] + uu[3];
                    sx[3 * ky] = p01 + p23;
                    sx[3 * ky + 1] = (uu[1] + uu[2]) + (next_lane(uu[0]) + uu[3]);
                    sx[3 * ky + 2] = next_lane(p01) + p23;
                }
                // The sums stay ahead of the store branch: sunk into it, an add
                // whose operand comes from lane TPW (inactive there) cannot
                // take its DPP move as a modifier, and each of the 12 moves
                // became an instruction of its own.
#pragma unroll
                for (int k = 0; k < 9; ++k) asm volatile("" : "+v"(sx[k]));
                if (lane < TPW) {
                    float* q = sp + ph * 9 * TPW;
#pragma unroll
                    for (int k = 0; k < 9; ++k) q[k * TPW] = sx[k];
                }
            }
        };
        // Contraction of LDS slot quad j (channels 4j .. 4j+3) with weights aq:
        // 6 blocks of 16 positions x 9 taps.  The unit's first quad starts the
        // accumulators from 0 inside its first MFMA.
        auto quad = [&](const float (&aq)[9], int j, auto first_tag) {
            constexpr bool FIRST = decltype(first_tag)::value;
            const float* cb = lds + (size_t)(4 * j + g) * Box4::CPLANE;
#pragma unroll
            for (int p = 0; p < NB; ++p) {
                const float* q = cb + (p / 3) * 9 * TPW + (p % 3) * 16 + l16;
                float t[9];
#pragma unroll
                for (int k = 0; k < 9; ++k) t[k] = q[k * TPW];
                acc[p] = mfma_16x16x4(aq[0], t[0], FIRST ? floatx4{0.f, 0.f, 0.f, 0.f} : acc[p]);
#pragma unroll
                for (int k = 1; k < 9; ++k) acc[p] = mfma_16x16x4(aq[k], t[k], acc[p]);
            }
        };
        auto chunk = [&](int c, auto first_tag) {
#pragma unroll
            for (int j = 0; j < CQ; ++j) box_sums(c, j);
            load_chunk_a(c);
            __syncthreads();
            quad(a[0], 0, first_tag);
#pragma unroll
            for (int j = 1; j < CQ; ++j)
                if (c * CQ + j < nq) quad(a[j], j, std::false_type{});
        };
        chunk(0, std::true_type{});
        if constexpr (NQ == 0) {
            const int nchunks = (nq + CQ - 1) / CQ;
            for (int c = 1; c < nchunks; ++c) {
                __syncthreads();  // the last chunk's box sums are read
                load_rows(v, 4 * c * CQ + wave);
                chunk(c, std::false_type{});
            }
        }

        // Epilogue: lane (g, l16) of block p holds the window sum of channel
        // co = ... + 4g + r at pooled position (p / 3, (p % 3) * 16 + l16).
        // sigma(sum / s^2 + bias) = 1 / (1 + 2^(sum * c1 + c0[r])), with the
        // scale, the bias and -log2(e) folded into one multiply-add.
        const float inv = 1.0f / (float)(S * S);
        constexpr float kNegLog2e = -1.4426950408889634f;
        float lsum = 0.f;
        if constexpr (MODE != OUT_MAP) {
            if (co_w + 16 <= Cout && ph0 + TPH <= PH && pw0 + TPW <= PW) {
                // every output of the wave is in range
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float c0 = bco[r] * kNegLog2e;
#pragma unroll
                    for (int p = 0; p < NB; ++p)
                        lsum += __builtin_amdgcn_rcpf(
                            1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(acc[p][r], inv * kNegLog2e, c0)));
                }
            } else if (co_w + 16 <= Cout) {
                // a tile at the bottom or right edge: every channel of the wave
                // is in range, so one select per position block adds the
                // block's four sums or nothing (positions past the map hold
                // finite values of the zero-padded or dropped input, but a
                // select keeps a non-finite one out of the sum too)
                bool colok[3];
#pragma unroll
                for (int c = 0; c < 3; ++c) colok[c] = pw0 + c * 16 + l16 < PW;
#pragma unroll
                for (int p = 0; p < NB; ++p) {
                    float sp = 0.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sp += __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(
                                                               acc[p][r], inv * kNegLog2e, bco[r] * kNegLog2e)));
                    lsum += (ph0 + p / 3 < PH && colok[p % 3]) ? sp : 0.f;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int co = co_w + 4 * g + r;
                    const float c0 = bco[r] * kNegLog2e;
#pragma unroll
                    for (int p = 0; p < NB; ++p) {
                        const int ph = ph0 + p / 3, pw = pw0 + (p % 3) * 16 + l16;
                        const float v =
                            __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(acc[p][r], inv * kNegLog2e, c0)));
                        lsum += (co < Cout && ph < PH && pw < PW) ? v : 0.f;
                    }
                }
            }
            dsum += lsum;
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = co_w + 4 * g + r;
#pragma unroll
                for (int p = 0; p < NB; ++p) {
                    const int ph = ph0 + p / 3, pw = pw0 + (p % 3) * 16 + l16;
                    if (co < Cout && ph < PH && pw < PW)
                        dst[(((size_t)b * Cout + co) * PH + ph) * PW + pw] = acc[p][r] * inv + bco[r];
                }
            }
        }
        if (!WALK || u + parts >= units) break;
    }  // units
    if constexpr (MODE != OUT_MAP) {
        const float sum = block_sum<NW>((float)dsum, red);
        if (tid == 0) dst[(size_t)b * parts + part] = sum;
    }
}

static size_t box4_lds_bytes(int NQ) {
    return (size_t)4 * box4_chunk_quads(NQ) * Box4::CPLANE * sizeof(float);
}

// The K = 3, s = 4 shapes the one-column-per-lane kernel takes (by shape
// alone, so that the deterministic form's workspace size does not depend on
// pointer alignment).  Any channel count: the box sums go through LDS in
// chunks of at most 8 channels.
static bool box4_fits(const Conv2dShape& s) { return s.K == 3 && s.S == 4 && s.W % 4 == 0; }

template <bool VEC, int NQ>
struct Box4Launch {
    template <int MODE>
    static constexpr auto kernel_once = conv2d_pool_boxsum4_kernel<MODE, VEC, NQ, false>;
    template <int MODE>
    static constexpr auto kernel_walk = conv2d_pool_boxsum4_kernel<MODE, VEC, NQ, true>;
};

static Walk box4_walk(const Conv2dShape& s) { return make_walk<Box4::TPH, Box4::TPW, Box4::CO_RANGE>(s); }

static int64_t box4_parts(const Conv2dShape& s) { return box4_walk(s).parts; }

template <bool VEC, int NQ>
static hipError_t launch_box4_q(const Conv2dShape& s, const float* x, const float* w, const float* bias, float* dst,
                                int mode, hipStream_t stream) {
    const int CINQ = (s.Cin + 3) / 4;
    const size_t lds = box4_lds_bytes(NQ);
    const Walk k = box4_walk(s);
    const int nblocks = k.parts * s.B;  // at most 1024 * 65535
    using L = Box4Launch<VEC, NQ>;
    FCONV_LAUNCH_WALK(L::template kernel, k.units > k.parts, dim3(nblocks), dim3(Box4::NT), lds, stream, x, w, bias, dst, s.Cin, s.H,
                       s.W, s.Cout, s.PH, s.PW, CINQ, k.tiles_w, k.tiles, k.units, k.parts, nblocks);
}

// One or two channels per wave at compile time, more at run time.
template <bool VEC>
static hipError_t launch_box4_v(const Conv2dShape& s, const float* x, const float* w, const float* bias, float* dst,
                                int mode, hipStream_t stream) {
    const int CINQ = (s.Cin + 3) / 4;
    if (CINQ == 1) return launch_box4_q<VEC, 1>(s, x, w, bias, dst, mode, stream);
    if (CINQ == 2) return launch_box4_q<VEC, 2>(s, x, w, bias, dst, mode, stream);
    return launch_box4_q<VEC, 0>(s, x, w, bias, dst, mode, stream);
}

static hipError_t launch_box4(const Conv2dShape& s, const float* x, const float* w, const float* bias, float* dst,
                              int mode, hipStream_t stream) {
    if ((uintptr_t)x % 16 == 0) return launch_box4_v<true>(s, x, w, bias, dst, mode, stream);
    return launch_box4_v<false>(s, x, w, bias, dst, mode, stream);
}

// Instances: K3/s4 4x16 tile with 4 waves x 16 channels; K5/s3 4x12 tile
// with 8 waves x 16 channels; K3/s2 and K3/s3 4x16 tiles with 4 waves x 16
// channels, or 8 waves x 16 where Cout > 64: with 64-channel ranges two
// workgroups made the same box sums for each tile of a 128-channel map
// (x[64,16,257,257] -> 128: 0.1875 against 0.2045 ms for K3/s3, 0.3411
// against 0.3481 ms for K3/s2, interleaved A/B).
#ifndef FCONV_CFG_BOX_K3S4
#define FCONV_CFG_BOX_K3S4 3, 4, 1, 4, 4, 1, 4, 16
#endif
#ifndef FCONV_CFG_BOX_K5S3
#define FCONV_CFG_BOX_K5S3 5, 3, 1, 3, 8, 1, 4, 12
#endif
using BoxK3S4 = DirectCfg<FCONV_CFG_BOX_K3S4>;
using BoxK5S3 = DirectCfg<FCONV_CFG_BOX_K5S3>;
using BoxK3S2 = DirectCfg<3, 2, 1, 4, 4, 1, 4, 16>;
using BoxK3S3 = DirectCfg<3, 3, 1, 4, 4, 1, 4, 16>;
using BoxK3S2W8 = DirectCfg<3, 2, 1, 4, 8, 1, 4, 16>;
using BoxK3S3W8 = DirectCfg<3, 3, 1, 4, 8, 1, 4, 16>;

// LDS of one workgroup: a chunk of CC channels' box sums plus the waves'
// scratch rows, whatever Cin is.
template <class Cfg>
static constexpr size_t box_lds_bytes() {
    using L = BoxLayout<Cfg>;
    return ((size_t)L::CC * L::SPLANE + (size_t)Cfg::NW * L::SCRATCH) * sizeof(float);
}

// Every channel count: the box sums go through LDS in chunks.
bool conv2d_boxsum_supported(int Cin, int K, int S) {
    return Cin >= 1 && ((K == 3 && (S == 2 || S == 3 || S == 4)) || (K == 5 && S == 3));
}

template <class Cfg>
struct BoxLaunch {
    template <int MODE>
    static constexpr auto kernel_once = conv2d_pool_boxsum_kernel<Cfg, MODE, false>;
    template <int MODE>
    static constexpr auto kernel_walk = conv2d_pool_boxsum_kernel<Cfg, MODE, true>;
};

template <class Cfg>
static int64_t box_parts(const Conv2dShape& s) {
    return direct_walk<Cfg>(s).parts;
}

template <class Cfg>
static hipError_t launch_box(const Conv2dShape& s, const float* x, const float* w, const float* bias, float* dst,
                             int mode, hipStream_t stream) {
    const int CINQ = (s.Cin + 3) / 4;
    constexpr size_t lds = box_lds_bytes<Cfg>();
    static_assert(lds <= kMaxLds, "box-sum chunk fits LDS");
    const Walk k = direct_walk<Cfg>(s);
    const int nblocks = k.parts * s.B;  // at most 1024 * 65535
    FCONV_LAUNCH_WALK(BoxLaunch<Cfg>::template kernel, k.units > k.parts, dim3(nblocks), dim3(Cfg::NT), lds, stream, x, w, bias, dst,
                       s.Cin, s.H, s.W, s.Cout, s.PH, s.PW, CINQ, k.tiles_w, k.tiles, k.units, k.parts, nblocks);
}

hipError_t conv2d_boxsum_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                                float* dst, int mode, hipStream_t stream) {
#ifndef FCONV_NO_BOX4
    if (box4_fits(s)) return launch_box4(s, x, w, bias, dst, mode, stream);
#endif
    if (s.K == 3 && s.S == 4) return launch_box<BoxK3S4>(s, x, w, bias, dst, mode, stream);
    if (s.K == 5 && s.S == 3) return launch_box<BoxK5S3>(s, x, w, bias, dst, mode, stream);
    if (s.K == 3 && s.S == 2)
        return s.Cout > 64 ? launch_box<BoxK3S2W8>(s, x, w, bias, dst, mode, stream)
                           : launch_box<BoxK3S2>(s, x, w, bias, dst, mode, stream);
    if (s.K == 3 && s.S == 3)
        return s.Cout > 64 ? launch_box<BoxK3S3W8>(s, x, w, bias, dst, mode, stream)
                           : launch_box<BoxK3S3>(s, x, w, bias, dst, mode, stream);
    return hipErrorInvalidValue;
}

int64_t conv2d_boxsum_parts(const Conv2dShape& s) {
#ifndef FCONV_NO_BOX4
    if (box4_fits(s)) return box4_parts(s);
#endif
    if (s.K == 3 && s.S == 4) return box_parts<BoxK3S4>(s);
    if (s.K == 5 && s.S == 3) return box_parts<BoxK5S3>(s);
    if (s.K == 3 && s.S == 2) return s.Cout > 64 ? box_parts<BoxK3S2W8>(s) : box_parts<BoxK3S2>(s);
    if (s.K == 3 && s.S == 3) return s.Cout > 64 ? box_parts<BoxK3S3W8>(s) : box_parts<BoxK3S3>(s);
    return -1;
}

// ---------------------------------------------------------------- simple direct conv (any K, s)

// One thread per (co, ph, pw) of one batch item: the window's s*s conv
// outputs are summed straight from global memory.  The general fallback.
// Workgroup (part, b) walks the item's 256-output blocks part, part + parts,
// ... (parts = gridDim.x).
template <int MODE>
__global__ __launch_bounds__(256) void conv2d_pool_simple_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ dst, int Cin, int H, int W, int Cout, int K, int S, int PH, int PW, int units) {
    __shared__ float red[4];
    const int b = blockIdx.y;
    const int parts = gridDim.x;
    const int n = Cout * PH * PW;
    double dsum = 0.0;
    for (int blk = blockIdx.x; blk < units; blk += parts) {
        const int64_t idx64 = (int64_t)blk * 256 + threadIdx.x;
        if (idx64 < n) {
            const int idx = (int)idx64;
            const int co = idx / (PH * PW);
            const int rem = idx - co * (PH * PW);
            const int ph = rem / PW, pw = rem - (rem / PW) * PW;
            const float* xb = x + (size_t)b * Cin * H * W;
            const float* wc = w + (size_t)co * Cin * K * K;
            float acc = 0.f;
            for (int dy = 0; dy < S; ++dy)
                for (int dx = 0; dx < S; ++dx)
                    for (int ic = 0; ic < Cin; ++ic)
                        for (int ky = 0; ky < K; ++ky) {
                            const float* xr = xb + ((size_t)ic * H + ph * S + dy + ky) * W + pw * S + dx;
                            const float* wr = wc + (ic * K + ky) * K;
                            for (int kx = 0; kx < K; ++kx) acc += xr[kx] * wr[kx];
                        }
            const float avg = acc / (float)(S * S) + (bias ? bias[co] : 0.f);
            if constexpr (MODE == OUT_MAP)
                dst[(size_t)b * n + idx] = avg;
            else
                dsum += (double)logistic(avg);
        }
    }
    if constexpr (MODE != OUT_MAP) {
        const float s = block_sum<4>((float)dsum, red);
        if (threadIdx.x == 0) dst[(size_t)b * parts + blockIdx.x] = s;
    }
}

struct SimpleLaunch {
    template <int MODE>
    static constexpr auto kernel = conv2d_pool_simple_kernel<MODE>;
};

static int simple_units(const Conv2dShape& s) { return (int)(((int64_t)s.Cout * s.PH * s.PW + 255) / 256); }

int64_t conv2d_simple_parts(const Conv2dShape& s) { return walk_parts(simple_units(s)); }

hipError_t conv2d_simple_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                                float* dst, int mode, hipStream_t stream) {
    const dim3 grid((unsigned)conv2d_simple_parts(s), s.B);
    FCONV_LAUNCH_MODES(SimpleLaunch::template kernel, grid, dim3(256), 0, stream, x, w, bias, dst, s.Cin, s.H, s.W,
                       s.Cout, s.K, s.S, s.PH, s.PW, simple_units(s));
}

// ---------------------------------------------------------------- fixed-order reduction of partial sums

// out[b] = sum over p of ws[b*parts + p]: thread t adds p = t, t+256, ... in
// order, then the workgroup tree (fixed shuffle pattern, fixed wave order).
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ ws, int64_t parts,
                                                              float* __restrict__ out) {
    __shared__ float red[4];
    const float* row = ws + (size_t)blockIdx.x * parts;
    float v = 0.f;
    for (int64_t p = threadIdx.x; p < parts; p += 256) v += row[p];
    const float s = block_sum<4>(v, red);
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

hipError_t reduce_partials(const float* ws, int64_t parts, int B, float* out, hipStream_t stream) {
    hipLaunchKernelGGL(reduce_partials_kernel, dim3(B), dim3(256), 0, stream, ws, parts, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------- zero fill

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

hipError_t fill_zero(float* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace fconv
