// conv2d_pool_ex.hip -- the Conv2d path with the pool generalised: average or
// max pooling, an optional ReLU between the convolution and the pool, and
// PyTorch's floor or ceil output size.
//
//   pooled[co,ph,pw] = POOL_{y,x in window(ph,pw)} act(conv[co,y,x])
//   conv[co,y,x]     = bias[co] + sum_{ic,ky,kx} x[ic,y+ky,x+kx] * w[co,ic,ky,kx]
//   act              = ReLU or identity;  POOL = mean or max
//   window(ph,pw)    = rows [ph*s, min(ph*s+s, Hc)) x columns [pw*s, min(pw*s+s, Wc))
//   out[b]           = sum_{co,ph,pw} sigmoid(pooled[co,ph,pw])
//
// Sources: the base chain is the one of POPCORNBENCH reasoning trace
// "Kimi-K2.6 l2_p65" (Conv2d -> AvgPool2d -> Sigmoid -> Sum); the 新智元
// article on the same benchmark lists a fused Conv2D + ReLU + MaxPool
// operator, which is where the ReLU-before-the-pool order and the max pool
// come from.  Ceil mode follows PyTorch's pooling: ceil(Hc/s) rows, the last
// window clipped to the map, a partial window averaging over its valid
// elements only (there is no padding, so every window starts inside the map).
//
// Neither ReLU nor max is linear, so the pool can no longer be folded into
// the contraction (as the AvgPool kernels do): each conv output must exist
// on its own, if only in a register.  Two kernels:
//  * conv2d_pool_elem_kernel (K = 3, s = 4, fp32 matrix cores): the MFMA N
//    dimension runs over 16 consecutive conv columns (four windows) of one
//    conv row, and each wave keeps four accumulator blocks, one per window
//    row dy, for each of its 16-column blocks.  The bias is the
//    accumulators' starting value, so every accumulator element is a finished
//    conv output.  The pool then reduces over dy inside each lane's
//    registers and over dx across the 4 lanes of a window with two DPP quad
//    steps, arranged as a transposing reduction that leaves lane dx holding
//    the pooled value of output channel 4g+dx: one sigmoid per lane per
//    block, none wasted.  The multiply-adds are those of the direct AvgPool
//    kernel (s^2*Cin*K*K per pooled output), only grouped by conv output.
//  * conv2d_pool_general_kernel: one thread per pooled output, any shape.
#include <limits.h>
#include <math.h>

#include <type_traits>

#include "fconv_device.hpp"
#include "fconv_internal.hpp"

namespace fconv {

// ---------------------------------------------------------------- any shape

// One thread per pooled output; workgroup (part, b) walks the item's
// 256-output blocks part, part + parts, ... (parts = gridDim.x).
template <int MODE>
__global__ __launch_bounds__(256) void conv2d_pool_general_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ dst, int Cin, int H, int W, int Cout, int K, int S, int PH, int PW, int pool_max,
    int relu, int units) {
    __shared__ float red[4];
    const int b = blockIdx.y;
    const int parts = gridDim.x;
    const int n = Cout * PH * PW;
    const int Hc = H - K + 1, Wc = W - K + 1;
    double dsum = 0.0;
    for (int blk = blockIdx.x; blk < units; blk += parts) {
        const int64_t idx64 = (int64_t)blk * 256 + threadIdx.x;
        if (idx64 < n) {
            const int idx = (int)idx64;
            const int co = idx / (PH * PW);
            const int rem = idx - co * (PH * PW);
            const int ph = rem / PW, pw = rem - (rem / PW) * PW;
            const int ny = min(S, Hc - ph * S), nx = min(S, Wc - pw * S);
            const float* xb = x + (size_t)b * Cin * H * W;
            const float* wc = w + (size_t)co * Cin * K * K;
            const float bc = bias ? bias[co] : 0.f;
            float pooled = pool_max ? -INFINITY : 0.f;
            for (int dy = 0; dy < ny; ++dy)
                for (int dx = 0; dx < nx; ++dx) {
                    float c = 0.f;
                    for (int ic = 0; ic < Cin; ++ic)
                        for (int ky = 0; ky < K; ++ky) {
                            const float* xr = xb + ((size_t)ic * H + ph * S + dy + ky) * W + pw * S + dx;
                            const float* wr = wc + (ic * K + ky) * K;
                            for (int kx = 0; kx < K; ++kx) c += xr[kx] * wr[kx];
                        }
                    c += bc;
                    if (relu) c = fmaxf(c, 0.f);
                    pooled = pool_max ? fmaxf(pooled, c) : pooled + c;
                }
            if (!pool_max) pooled /= (float)(ny * nx);
            if constexpr (MODE == OUT_MAP)
                dst[(size_t)b * n + idx] = pooled;
            else
                dsum += (double)logistic(pooled);
        }
    }
    if constexpr (MODE != OUT_MAP) {
        const float s = block_sum<4>((float)dsum, red);
        if (threadIdx.x == 0) dst[(size_t)b * parts + blockIdx.x] = s;
    }
}

static int general_units(const Conv2dShape& s) { return (int)(((int64_t)s.Cout * s.PH * s.PW + 255) / 256); }

int64_t conv2d_general_parts(const Conv2dShape& s) { return walk_parts(general_units(s)); }

// ---------------------------------------------------------------- on matrix cores

// Tiling: a workgroup of 4 waves covers 64 output channels (16 per wave) and
// a TPH x TPW pooled tile; each wave walks the tile's pooled rows one at a
// time, holding NCB column blocks x S window rows of accumulators.  A column
// block is the MFMA's 16 lanes of N: WPB = 16/S whole windows, CPB = WPB*S
// conv columns (for s = 3 the 16th lane's column belongs to no window of its
// block and is ignored).
template <int K_, int S_, int NCB_, int TPH_, bool CHUNK_ = false>
struct ElemCfg {
    static constexpr int K = K_, S = S_, NCB = NCB_, TPH = TPH_;
    // CHUNK: the channels pass through LDS CQ quads at a time (any Cin);
    // otherwise all of a tile's channels are staged at once
    static constexpr bool CHUNK = CHUNK_;
    static constexpr int CQ = 4;
    static constexpr int WPB = 16 / S;                 // windows per column block
    static constexpr int CPB = WPB * S;                // conv columns per column block
    static constexpr int TPW = NCB * WPB;              // pooled columns per tile
    static constexpr int NW = 4, NT = 64 * NW;
    static constexpr int CO_RANGE = 16 * NW;
    static constexpr int IH = TPH * S + K - 1;         // input rows per tile
    static constexpr int IW = (NCB - 1) * CPB + 16 + K - 1;  // input columns the lanes read
    static constexpr int RP = IW;                      // LDS floats per row
    static constexpr int NR = S + K - 1;               // input rows one pooled row reads
    static_assert(S == 2 || S == 3 || S == 4, "window reduction implemented for s = 2, 3, 4");
};

// Instances: K = 3 with s = 2, 3, 4; K = 5 with s = 3.
using ElemK3S4 = ElemCfg<3, 4, 4, 4>;  // 4 x 16 pooled tile, 18 x 66 input
// The folded average pool needs 60 instead of 115 VGPRs, so LDS decides its
// occupancy: 3-row tiles (5 workgroups per CU) measured 0.7 % faster there,
// while the 115-VGPR variants are fastest with 4-row tiles.
using ElemK3S4Fold = ElemCfg<3, 4, 4, 3>;  // 3 x 16 pooled tile, 14 x 66 input
using ElemK3S2 = ElemCfg<3, 2, 4, 4>;  // 4 x 32 pooled tile, 10 x 66 input
using ElemK3S3 = ElemCfg<3, 3, 4, 4>;  // 4 x 20 pooled tile, 14 x 63 input
using ElemK5S3 = ElemCfg<5, 3, 2, 4>;  // 4 x 10 pooled tile, 16 x 35 input
// Channel-chunked instances for Cin beyond the staged tiles above: one pooled
// row per tile, so that one row's accumulators carry over the chunks, and 16
// channels per LDS chunk (17-26 KB).
using ElemK3S4C = ElemCfg<3, 4, 4, 1, true>;
using ElemK3S2C = ElemCfg<3, 2, 4, 1, true>;
using ElemK3S3C = ElemCfg<3, 3, 4, 1, true>;
using ElemK5S3C = ElemCfg<5, 3, 2, 1, true>;

// POOL: kPoolMean (each conv output kept, then averaged), kPoolMax, or
// kPoolMeanFolded: the average pool of a plain conv (no ReLU, floor mode),
// where the pool's linearity lets the MFMAs add a window's rows into one
// accumulator block per column block (which starts at s * bias), so only the
// window's columns are summed afterwards.
constexpr int kPoolMean = 0, kPoolMax = 1, kPoolMeanFolded = 2;

// NQ: 0, or the number of channel quads CINQ (1 or 2) when all of them fit
// in registers.  Then the block's weights load once; otherwise quad q's
// weights stream in under quad q-1's matrix instructions.
// Occupancy: the whole-tile instances are held to 3 workgroups per CU (up
// to 170 VGPRs); the channel-chunked ones to 4, which fits the max-pool
// instance's 64 accumulators in 128 VGPRs without spills in its sum path
// (x[16,64,384,384], ReLU + max pool: 1.316 -> 1.260 ms).
template <class C, int POOL, int MODE, int NQ, bool WALK>
__global__ __launch_bounds__(C::NT, C::CHUNK ? 4 : 3) void conv2d_pool_elem_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ bias,
    float* __restrict__ dst, int Cin, int H, int W, int Cout, int PH, int PW, int CINQ, int plane, int tiles_w,
    int tiles, int co_ranges, int units, int parts, int nblocks, int relu, int ceil_mode) {
    constexpr int K = C::K, S = C::S, NCB = C::NCB, TPH = C::TPH, TPW = C::TPW;
    constexpr int IH = C::IH, IW = C::IW, RP = C::RP, NR = C::NR, WPB = C::WPB, CPB = C::CPB;
    constexpr bool POOL_MAX = POOL == kPoolMax, FOLD = POOL == kPoolMeanFolded;
    constexpr int NACC = FOLD ? 1 : S;  // accumulator blocks per column block
    // TF: with s = 4 or 2 the MFMA operands are swapped (input as A,
    // weights as B), so a lane's four accumulator elements are four adjacent
    // conv columns of one channel, and a window's columns pool inside the
    // lane instead of through the cross-lane exchange (6 selects and 3 DPP
    // operations per 16-column block).  Interleaved A/B on x[128,8,384,384]
    // -> 64, ms: folded average pool 1.1966 against 1.2090 (K3/s2: 1.2467
    // against 1.2646); ReLU + max pool 1.2159 against 1.2286 (K3/s2: 1.2659
    // against 1.2910; ceil mode 1.2497 against 1.2556).  The unfolded average
    // pool (ReLU before it) measured 1.2745 against 1.2554 and keeps the
    // exchange; so do s = 3 windows, which do not align with a lane's four
    // columns.
    constexpr bool TF = (S == 4 || S == 2) && POOL != kPoolMean;
    static_assert(NQ >= 0 && NQ <= 2, "resident weights for one or two channel quads");

    extern __shared__ float lds[];
    __shared__ float red[C::NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;    // MFMA k-slot: channel group
    const int l16 = lane & 15;  // row of A / column of B
    const int Hc = H - K + 1, Wc = W - K + 1;
    // Block order: the hardware deals block ids to the 8 XCDs round-robin;
    // xcd_spread gives each XCD one contiguous run of logical ids, ordered
    // (batch item, tile row, tile column, channel range) with the channel
    // range fastest.  Tiles that share input (the channel ranges of one tile,
    // its right and lower neighbours with their halo lines) then run close
    // together in time on one XCD and find that input in its L2.  Workgroup
    // `part` of batch item b walks the item's units part, part + parts, ...
    // (unit = tile * co_ranges + channel range).
    const int lid = xcd_spread(blockIdx.x, nblocks);
    const int b = lid / parts;
    const int part = lid - b * parts;
    walk_sum_t<WALK> dsum = 0;  // this lane's sigmoids over all its units
    for (int u = part;; u += parts) {
        if (WALK && u != part) __syncthreads();  // every wave is done with the last unit's tile
        const int cor = u % co_ranges;
        const int tile = u / co_ranges;
        const int tile_y = tile / tiles_w;
        const int tile_x = tile - tile_y * tiles_w;
        const int y0 = tile_y * TPH * S, x0 = tile_x * TPW * S;
        const int ph0 = tile_y * TPH, pw0 = tile_x * TPW;
        const int co0 = cor * C::CO_RANGE + wave * 16;

        // Weights of channel quad q: a[ky][kx] = w[co0 + l16, ic, ky, kx] with
        // ic = g*CINQ + q (whole tiles staged: lane group g walks its own
        // channel range) or ic = 4q + g (chunked: a quad is 4 consecutive
        // channels); 0 where co or ic is out of range.
        const buf_rsrc rw = make_rsrc(w, Cout * Cin * K * K * 4);
        auto load_a = [&](float (&a)[K][K], int q) {
            const int ic = C::CHUNK ? 4 * q + g : g * CINQ + q;
            const int co = co0 + l16;
            const bool ok = (co < Cout) && (ic < Cin) && (q < CINQ);
            const int base = ok ? (co * Cin + ic) * (K * K * 4) : kBufOOB;
#pragma unroll
            for (int ky = 0; ky < K; ++ky)
#pragma unroll
                for (int kx = 0; kx < K; ++kx) a[ky][kx] = buf_load_f32(rw, base + (ky * K + kx) * 4);
        };
        // Streaming: a[0] holds the current quad's weights, a[1] the next one's.
        // Resident: a[q] holds quad q's.
        float a[2][K][K];
        load_a(a[0], 0);
        if constexpr (NQ == 2) load_a(a[1], 1);

        // Bias of the channels this lane's accumulator elements hold: co0 + 4g + r
        // (TF: co0 + l16 for all four).
        const buf_rsrc rb = make_rsrc(bias, bias ? Cout * 4 : 0);
        floatx4 bco;
        if constexpr (TF) {
            const int co = co0 + l16;
            const float bl = buf_load_f32(rb, co < Cout ? co * 4 : kBufOOB);
            bco = floatx4{bl, bl, bl, bl};
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = co0 + 4 * g + r;
                bco[r] = buf_load_f32(rb, co < Cout ? co * 4 : kBufOOB);
            }
        }

        // Stage the input tile: channels chan0 .. chan0+nchan-1 (slot s =
        // ic - chan0 at s*plane), row r at r*RP, column c at c.  Whole rows per
        // wave through a per-row buffer resource (empty for rows outside the
        // image and channels >= Cin, which therefore read 0).
        auto stage = [&](int chan0, int nchan) {
            constexpr int NCH = (IW + 63) / 64;
            constexpr int UR = C::CHUNK ? 6 : 14;  // rows in flight per wave
            int voff[NCH];
            bool inr[NCH];
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                const int c = lane + 64 * k;
                inr[k] = c < IW;
                voff[k] = (c < IW && x0 + c < W) ? (x0 + c) * 4 : kBufOOB;
            }
            const int wave_s = __builtin_amdgcn_readfirstlane(wave);
            const int nrows = nchan * IH;
            const float* xb = x + (size_t)b * Cin * H * W;
            for (int row0 = wave_s; row0 < nrows; row0 += C::NW * UR) {
                float v[UR][NCH];
#pragma unroll
                for (int uu = 0; uu < UR; ++uu) {
                    const int row = row0 + uu * C::NW;
                    const int ic = chan0 + row / IH, r = row - (row / IH) * IH;
                    const bool ok = (row < nrows) && (ic < Cin) && (y0 + r < H);
                    const buf_rsrc rrow = make_rsrc(xb + (ok ? (ic * H + y0 + r) * W : 0), ok ? W * 4 : 0);
#pragma unroll
                    for (int k = 0; k < NCH; ++k) v[uu][k] = buf_load_f32(rrow, voff[k]);
                }
#pragma unroll
                for (int uu = 0; uu < UR; ++uu) {
                    const int row = row0 + uu * C::NW;
                    if (row < nrows) {
                        const int sl = row / IH, r = row - (row / IH) * IH;
                        float* lrow = lds + sl * plane + r * RP;
#pragma unroll
                        for (int k = 0; k < NCH; ++k)
                            if (inr[k]) lrow[lane + 64 * k] = v[uu][k];
                    }
                }
            }
        };
        if constexpr (C::CHUNK)
            stage(0, 4 * min(C::CQ, CINQ));
        else
            stage(0, 4 * CINQ);
        __syncthreads();

        // A column block's lanes read 16 consecutive words; the 4 channel groups
        // sit plane*CINQ (chunked: plane) words apart (padded onto different
        // banks).  Rows of one
        // pooled row read from two base registers: rows 0 .. RG-1 from the
        // first, the rest from a second one RG rows further on, so that every
        // read keeps within the 8-bit dword offsets of paired LDS reads.
        constexpr int RG = (255 - (NCB - 1) * CPB - (K - 1)) / RP + 1;
        static_assert(RG >= 1 && NR <= 2 * RG, "two base registers reach every row");
        const lds_fptr lbase = (lds_fptr)lds + g * (C::CHUNK ? 1 : CINQ) * plane + l16;
        // NBA (a compile-time tag): the column blocks the tile computes.
        auto load_row = [&](float (&bv)[NCB][K], lds_fptr row, auto nba) {
#pragma unroll
            for (int nb = 0; nb < decltype(nba)::value; ++nb)
#pragma unroll
                for (int kx = 0; kx < K; ++kx) bv[nb][kx] = row[nb * CPB + kx];
        };

        const bool odd1 = (l16 & 1) != 0, odd2 = (l16 & 2) != 0;
        auto pool2 = [](float a, float c) { return POOL_MAX ? fmaxf(a, c) : a + c; };

        // One channel quad of one pooled row with weights aq.  In the first quad
        // the first MFMA into each accumulator block takes the bias as its C
        // operand, so the accumulators never need a separate initialisation.
        // Folded rows: each column accumulator sums S conv outputs, so it starts
        // at S * bias.
        if constexpr (FOLD) bco = bco * (float)S;
        floatx4 acc[NCB][NACC];
        auto mma_quad = [&](const float (&aq)[K][K], int q, int pr, auto first_tag, auto nba) {
            constexpr bool FIRST = decltype(first_tag)::value;
            constexpr int NBA = decltype(nba)::value;
            // quad q's channels: slot q (whole tile) or 4 (q % CQ) (chunked)
            const lds_fptr p0 = lbase + (C::CHUNK ? 4 * (q % C::CQ) : q) * plane + pr * S * RP;
            const lds_fptr p1 = NR > RG ? lds_opaque(p0 + RG * RP) : p0;
            auto row = [&](int rr) { return rr < RG ? p0 + rr * RP : p1 + (rr - RG) * RP; };
            float bcur[NCB][K], bnxt[NCB][K];
            load_row(bcur, row(0), nba);
#pragma unroll
            for (int rr = 0; rr < NR; ++rr) {
                if (rr + 1 < NR) load_row(bnxt, row(rr + 1), nba);
#pragma unroll
                for (int ky = 0; ky < K; ++ky) {
                    const int dy = rr - ky;
                    if (dy < 0 || dy >= S) continue;
#pragma unroll
                    for (int kx = 0; kx < K; ++kx)
#pragma unroll
                        for (int nb = 0; nb < NBA; ++nb) {
                            const floatx4 cin =
                                (FIRST && ky == 0 && kx == 0 && (!FOLD || dy == 0)) ? bco : acc[nb][FOLD ? 0 : dy];
                            acc[nb][FOLD ? 0 : dy] = TF ? mfma_16x16x4(bcur[nb][kx], aq[ky][kx], cin)
                                                        : mfma_16x16x4(aq[ky][kx], bcur[nb][kx], cin);
                        }
                }
                if (rr + 1 < NR) {
#pragma unroll
                    for (int nb = 0; nb < NBA; ++nb)
#pragma unroll
                        for (int kx = 0; kx < K; ++kx) bcur[nb][kx] = bnxt[nb][kx];
                }
            }
        };
        // Streaming weights: the next quad's (quad 0 again after the last: the
        // next pooled row starts there) load under this quad's MFMAs.
        auto quad_stream = [&](int q, int pr, auto first_tag, auto nba) {
            load_a(a[1], q + 1 < CINQ ? q + 1 : 0);
            mma_quad(a[0], q, pr, first_tag, nba);
#pragma unroll
            for (int ky = 0; ky < K; ++ky)
#pragma unroll
                for (int kx = 0; kx < K; ++kx) a[0][ky][kx] = a[1][ky][kx];
        };

        float lsum = 0.f;
        // FULL: every column of the tile and every channel of the wave lies
        // inside the pooled map, so no lane needs a range check.
        auto pool_row = [&](const floatx4 (&ac)[NCB][NACC], int ph, int yr, auto edge_tag, auto full_tag, auto nba) {
            constexpr bool EDGE = decltype(edge_tag)::value, FULL = decltype(full_tag)::value;
            const float fill = POOL_MAX ? -INFINITY : 0.f;
            if constexpr (TF) {
                // Lane (g, l16) holds, for channel co0 + l16, conv columns
                // x0 + nb*16 + 4g + r (r = 0..3) of each conv row dy of the
                // window (folded: the rows' sum), so its 4 / S windows pool
                // over its own elements.
                constexpr int NV = 4 / S;
                const int co = co0 + l16;
#pragma unroll
                for (int nb = 0; nb < decltype(nba)::value; ++nb)
#pragma unroll
                    for (int i = 0; i < NV; ++i) {
                        float o;
                        if constexpr (FOLD) {
                            const floatx4 v = ac[nb][0];
                            o = S == 4 ? (v[0] + v[1]) + (v[2] + v[3]) : v[2 * i] + v[2 * i + 1];
                        } else {
                            float e[S * S];
#pragma unroll
                            for (int dy = 0; dy < S; ++dy)
#pragma unroll
                                for (int j = 0; j < S; ++j) {
                                    float t = ac[nb][dy][S * i + j];
                                    if (!POOL_MAX && relu) t = fmaxf(t, 0.f);
                                    if constexpr (EDGE) {
                                        const bool ok = (yr + dy < Hc) && (x0 + nb * CPB + 4 * g + S * i + j < Wc);
                                        t = ok ? t : fill;
                                    }
                                    e[dy * S + j] = t;
                                }
                            // pairwise over the window's S*S conv outputs
#pragma unroll
                            for (int w2 = S * S / 2; w2 >= 1; w2 /= 2)
#pragma unroll
                                for (int k = 0; k < w2; ++k) e[k] = pool2(e[k], e[k + w2]);
                            o = e[0];
                        }
                        const int pw = pw0 + nb * WPB + NV * g + i;
                        if (FULL || (pw < PW && co < Cout)) {
                            const float inv = EDGE ? 1.0f / (float)(min(S, Hc - ph * S) * min(S, Wc - pw * S))
                                                   : 1.0f / (float)(S * S);
                            if (POOL_MAX) {
                                if (relu) o = fmaxf(o, 0.f);  // ReLU commutes with max
                            } else if (EDGE || MODE == OUT_MAP) {
                                o = o * inv;
                            }
                            if constexpr (MODE == OUT_MAP)
                                dst[(((size_t)b * Cout + co) * PH + ph) * PW + pw] = o;
                            else if (POOL_MAX || EDGE)
                                lsum += logistic(o);
                            else
                                lsum += logistic_scaled(o, inv);
                        }
                    }
                return;
            }
#pragma unroll
            for (int nb = 0; nb < decltype(nba)::value; ++nb) {
                float m[4];
                if constexpr (FOLD) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[r] = ac[nb][0][r];
                } else {
                    float v[S][4];
#pragma unroll
                    for (int dy = 0; dy < S; ++dy)
#pragma unroll
                        for (int r = 0; r < 4; ++r) v[dy][r] = ac[nb][dy][r];
                    if (!POOL_MAX && relu) {
#pragma unroll
                        for (int dy = 0; dy < S; ++dy)
#pragma unroll
                            for (int r = 0; r < 4; ++r) v[dy][r] = fmaxf(v[dy][r], 0.f);
                    }
                    if constexpr (EDGE) {
                        const bool col_ok = x0 + nb * CPB + l16 < Wc;
#pragma unroll
                        for (int dy = 0; dy < S; ++dy) {
                            const bool ok = col_ok && (yr + dy < Hc);
#pragma unroll
                            for (int r = 0; r < 4; ++r) v[dy][r] = ok ? v[dy][r] : fill;
                        }
                    }
                    // Over the window's rows, inside the lane.
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        m[r] = v[0][r];
#pragma unroll
                        for (int dy = 1; dy < S; ++dy) m[r] = pool2(m[r], v[dy][r]);
                    }
                }
                // Over the window's columns, across lanes.  Each case leaves NV
                // finished pooled values per lane, value i for channel
                // co0 + 4g + chan[i] at window win of the block, valid where the
                // lane finishes a window (fin).
                constexpr int NV = S == 4 ? 1 : S == 2 ? 2 : 4;
                float pv[NV];
                int chan[NV];
                int win;
                bool fin;
                if constexpr (S == 4) {
                    // Lanes 4j..4j+3 hold window j.  Step 1 pairs lanes l, l^1:
                    // the even lane keeps channels r = 0, 2 and sends r = 1, 3;
                    // the odd lane the reverse.  Step 2 pairs l, l^2 the same way
                    // over the two kept values.  Lane dx ends with channel r = dx
                    // over all four columns.
                    const float k01 = odd1 ? m[1] : m[0], s01 = odd1 ? m[0] : m[1];
                    const float k23 = odd1 ? m[3] : m[2], s23 = odd1 ? m[2] : m[3];
                    const float p01 = pool2(k01, quad_xor1(s01));
                    const float p23 = pool2(k23, quad_xor1(s23));
                    const float kk = odd2 ? p23 : p01, ss = odd2 ? p01 : p23;
                    pv[0] = pool2(kk, quad_xor2(ss));
                    chan[0] = l16 & 3;
                    win = l16 >> 2;
                    fin = true;
                } else if constexpr (S == 2) {
                    // Lanes 2j, 2j+1 hold window j.  One pairing step as above:
                    // lane dx ends with channels dx and 2 + dx.
                    const float k01 = odd1 ? m[1] : m[0], s01 = odd1 ? m[0] : m[1];
                    const float k23 = odd1 ? m[3] : m[2], s23 = odd1 ? m[2] : m[3];
                    pv[0] = pool2(k01, quad_xor1(s01));
                    pv[1] = pool2(k23, quad_xor1(s23));
                    chan[0] = l16 & 1;
                    chan[1] = 2 + (l16 & 1);
                    win = l16 >> 1;
                    fin = true;
                } else {
                    // Lanes 3j..3j+2 (j < 5) hold window j: the window's last lane
                    // gathers its two left neighbours (DPP row shifts) and
                    // finishes all four channels.
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pv[r] = pool2(pool2(m[r], row_shr1(m[r])), row_shr2(m[r]));
                        chan[r] = r;
                    }
                    win = l16 / 3;
                    fin = (l16 % 3 == 2) && l16 < 15;
                }

                const int pw = pw0 + nb * WPB + win;
                if (fin && (FULL || pw < PW)) {
                    const float inv = EDGE ? 1.0f / (float)(min(S, Hc - ph * S) * min(S, Wc - pw * S))
                                           : 1.0f / (float)(S * S);
#pragma unroll
                    for (int i = 0; i < NV; ++i) {
                        const int co = co0 + 4 * g + chan[i];
                        if (FULL || co < Cout) {
                            float o = pv[i];
                            if (POOL_MAX) {
                                if (relu) o = fmaxf(o, 0.f);  // ReLU commutes with max
                            } else if (EDGE || MODE == OUT_MAP) {
                                o = o * inv;
                            }
                            if constexpr (MODE == OUT_MAP)
                                dst[(((size_t)b * Cout + co) * PH + ph) * PW + pw] = o;
                            else if (POOL_MAX || EDGE)
                                lsum += logistic(o);
                            else
                                lsum += logistic_scaled(o, inv);
                        }
                    }
                }
            }
        };

        const int nrow_tile = min(TPH, PH - ph0);
        const bool full = pw0 + TPW <= PW && co0 + 16 <= Cout;
        auto row_pass = [&](int pr, auto nba) {
            if constexpr (NQ > 0) {
                mma_quad(a[0], 0, pr, std::true_type{}, nba);
                if constexpr (NQ == 2) mma_quad(a[1], 1, pr, std::false_type{}, nba);
            } else if constexpr (C::CHUNK) {
                // one pooled row per tile: every CQ quads, the next chunk of
                // channels replaces the last one in LDS
                static_assert(TPH == 1, "a chunked tile is one pooled row");
                quad_stream(0, pr, std::true_type{}, nba);
                for (int q = 1; q < CINQ; ++q) {
                    if (q % C::CQ == 0) {
                        __syncthreads();  // every wave is done with the last chunk
                        stage(4 * q, 4 * min(C::CQ, CINQ - q));
                        __syncthreads();
                    }
                    quad_stream(q, pr, std::false_type{}, nba);
                }
            } else {
                quad_stream(0, pr, std::true_type{}, nba);
                for (int q = 1; q < CINQ; ++q) quad_stream(q, pr, std::false_type{}, nba);
            }

            // Epilogue of pooled row ph.  Lane (g, l16) holds in acc[nb][dy][r]
            // the conv output of channel co0 + 4g + r at conv row ph*S + dy,
            // column x0 + nb*16 + l16 (TF: channel co0 + l16, column
            // x0 + nb*16 + 4g + r; folded: the window's rows summed in
            // acc[nb][0]).  The pool works on register copies.
            // Conv outputs outside the map exist only in partial (ceil-mode)
            // windows at the bottom and right edges; those rows take a separate
            // copy of the epilogue that masks them.
            const int ph = ph0 + pr;
            const int yr = y0 + pr * S;
            if (!FOLD && ceil_mode && (yr + S > Hc || x0 + TPW * S > Wc))
                pool_row(acc, ph, yr, std::true_type{}, std::false_type{}, nba);  // (the folded pool has floor mode only)
            else if (full)
                pool_row(acc, ph, yr, std::false_type{}, std::true_type{}, nba);
            else
                pool_row(acc, ph, yr, std::false_type{}, std::false_type{}, nba);
        };
        // A tile of two column blocks whose second block lies wholly past the
        // map (the last tile column when the map's width is not a multiple of
        // the tile's) computes the first block only.
        const int nbv = min(NCB, (PW - pw0 + WPB - 1) / WPB);
        for (int pr = 0; pr < nrow_tile; ++pr) {
            if constexpr (NCB == 2) {
                if (nbv == 1)
                    row_pass(pr, std::integral_constant<int, 1>{});
                else
                    row_pass(pr, std::integral_constant<int, 2>{});
            } else {
                row_pass(pr, std::integral_constant<int, NCB>{});
            }
        }

        dsum += lsum;
        if (!WALK || u + parts >= units) break;
    }  // units
    if constexpr (MODE != OUT_MAP) {
        const float s = block_sum<C::NW>((float)dsum, red);
        if (tid == 0) dst[(size_t)b * parts + part] = s;
    }
}

namespace {

constexpr size_t kMaxLdsEx = 160 * 1024 - 256;

// Channel planes padded so that the 4 channel groups (plane*CINQ words
// apart; chunked: plane words) start 16 banks apart.
template <class C>
int elem_plane(int CINQ) {
    if (C::CHUNK) CINQ = 1;
    const int base = C::IH * C::RP;
    for (int pad = 0; pad < 64; ++pad)
        if (((long)CINQ * (base + pad)) % 64 == 16) return base + pad;
    for (int pad = 0; pad < 32; ++pad)
        if (((long)CINQ * (base + pad)) % 32 == 16) return base + pad;
    return base;
}

// The channel slots a workgroup stages at once: all quads, or one chunk.
template <class C>
int elem_slots(int CINQ) {
    return 4 * (C::CHUNK ? (CINQ < C::CQ ? CINQ : C::CQ) : CINQ);
}

template <class C>
size_t elem_lds_bytes(int Cin) {
    const int CINQ = (Cin + 3) / 4;
    return (size_t)elem_slots<C>(CINQ) * elem_plane<C>(CINQ) * sizeof(float);
}

// The plain average pool (no ReLU, floor mode) runs folded.
bool folds(const PoolOpts& o) { return !o.pool_max && !o.relu && !o.ceil_mode; }

// Units of one batch item (tiles x channel ranges: at most its pooled-map
// size, which fits int32) and workgroups per item.
struct ElemGrid {
    int tiles_w, tiles, co_ranges, units, parts;
};

template <class C>
ElemGrid elem_grid(const Conv2dShape& s) {
    const int tiles_h = (s.PH + C::TPH - 1) / C::TPH;
    const int tiles_w = (s.PW + C::TPW - 1) / C::TPW;
    const int co_ranges = (s.Cout + C::CO_RANGE - 1) / C::CO_RANGE;
    const int units = tiles_h * tiles_w * co_ranges;
    return {tiles_w, tiles_h * tiles_w, co_ranges, units, walk_parts(units)};
}

template <class C, int POOL, int MODE, int NQ, bool WALK>
hipError_t launch_elem_w(const Conv2dShape& s, const float* x, const float* w, const float* bias, float* dst,
                         const PoolOpts& o, hipStream_t stream) {
    const int CINQ = (s.Cin + 3) / 4;
    const int plane = elem_plane<C>(CINQ);
    const size_t lds = (size_t)elem_slots<C>(CINQ) * plane * sizeof(float);
    const ElemGrid g = elem_grid<C>(s);
    const int nblocks = g.parts * s.B;  // at most 1024 * 65535
    const void* fn = (const void*)conv2d_pool_elem_kernel<C, POOL, MODE, NQ, WALK>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((conv2d_pool_elem_kernel<C, POOL, MODE, NQ, WALK>), dim3((unsigned)nblocks), dim3(C::NT), lds,
                       stream, x, w, bias, dst, s.Cin, s.H, s.W, s.Cout, s.PH, s.PW, CINQ, plane, g.tiles_w, g.tiles,
                       g.co_ranges, g.units, g.parts, nblocks, o.relu ? 1 : 0, o.ceil_mode ? 1 : 0);
    return hipGetLastError();
}

// The walking instance when there are more units than workgroups.
template <class C, int POOL, int MODE, int NQ>
hipError_t launch_elem_nq(const Conv2dShape& s, const float* x, const float* w, const float* bias, float* dst,
                          const PoolOpts& o, hipStream_t stream) {
    const ElemGrid g = elem_grid<C>(s);
    if (g.units > g.parts) return launch_elem_w<C, POOL, MODE, NQ, true>(s, x, w, bias, dst, o, stream);
    return launch_elem_w<C, POOL, MODE, NQ, false>(s, x, w, bias, dst, o, stream);
}

// One or two channel quads keep their weights in registers.
template <class C, int POOL, int MODE>
hipError_t launch_elem_as(const Conv2dShape& s, const float* x, const float* w, const float* bias, float* dst,
                          const PoolOpts& o, hipStream_t stream) {
    const int CINQ = (s.Cin + 3) / 4;
    if constexpr (!C::CHUNK) {
        if (CINQ == 1) return launch_elem_nq<C, POOL, MODE, 1>(s, x, w, bias, dst, o, stream);
        if (CINQ == 2) return launch_elem_nq<C, POOL, MODE, 2>(s, x, w, bias, dst, o, stream);
    }
    return launch_elem_nq<C, POOL, MODE, 0>(s, x, w, bias, dst, o, stream);
}

// The K = 3, s = 4 tiling has a folded-pool config and one for the other
// pools; each is only launched for its own.
template <class C>
hipError_t launch_elem_cfg(const Conv2dShape& s, const float* x, const float* w, const float* bias, float* dst,
                           int mode, const PoolOpts& o, hipStream_t stream) {
    constexpr bool fold_only = std::is_same<C, ElemK3S4Fold>::value, no_fold = std::is_same<C, ElemK3S4>::value;
    if constexpr (!fold_only) {
        if (o.pool_max) {
            if (mode == OUT_MAP) return launch_elem_as<C, kPoolMax, OUT_MAP>(s, x, w, bias, dst, o, stream);
            return launch_elem_as<C, kPoolMax, OUT_PARTIAL>(s, x, w, bias, dst, o, stream);
        }
    }
    if constexpr (!no_fold) {
        if (folds(o)) {
            if (mode == OUT_MAP) return launch_elem_as<C, kPoolMeanFolded, OUT_MAP>(s, x, w, bias, dst, o, stream);
            return launch_elem_as<C, kPoolMeanFolded, OUT_PARTIAL>(s, x, w, bias, dst, o, stream);
        }
    }
    if constexpr (!fold_only) {
        if (mode == OUT_MAP) return launch_elem_as<C, kPoolMean, OUT_MAP>(s, x, w, bias, dst, o, stream);
        return launch_elem_as<C, kPoolMean, OUT_PARTIAL>(s, x, w, bias, dst, o, stream);
    }
    return hipErrorInvalidValue;
}

// Calls f with a value of the instance's config type for (K, S), the pool
// variant and Cin: the whole-tile tiling where its LDS tile fits, else the
// channel-chunked one; returns false if there is no instance.
template <class Whole, class Chunked, class F>
bool pick_elem(int Cin, F&& f) {
    if (elem_lds_bytes<Whole>(Cin) <= kMaxLdsEx) return f(Whole{}), true;
    return f(Chunked{}), true;
}

template <class F>
bool with_elem_cfg(int K, int S, bool fold, int Cin, F&& f) {
    if (K == 3 && S == 4)
        return fold ? pick_elem<ElemK3S4Fold, ElemK3S4C>(Cin, f) : pick_elem<ElemK3S4, ElemK3S4C>(Cin, f);
    if (K == 3 && S == 2) return pick_elem<ElemK3S2, ElemK3S2C>(Cin, f);
    if (K == 3 && S == 3) return pick_elem<ElemK3S3, ElemK3S3C>(Cin, f);
    if (K == 5 && S == 3) return pick_elem<ElemK5S3, ElemK5S3C>(Cin, f);
    return false;
}

}  // namespace

// Every channel count: past the whole-tile LDS budget the chunked tiling runs.
bool conv2d_elem_supported(int Cin, int K, int S) {
    return Cin >= 1 && ((K == 3 && (S == 2 || S == 3 || S == 4)) || (K == 5 && S == 3));
}


int64_t conv2d_elem_parts(const Conv2dShape& s, const PoolOpts& o) {
    int64_t parts = -1;
    with_elem_cfg(s.K, s.S, folds(o), s.Cin, [&](auto c) { parts = elem_grid<decltype(c)>(s).parts; });
    return parts;
}

hipError_t conv2d_elem_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias, float* dst,
                              int mode, const PoolOpts& o, hipStream_t stream) {
    if (!conv2d_elem_supported(s.Cin, s.K, s.S)) return hipErrorInvalidValue;
    hipError_t e = hipErrorInvalidValue;
    with_elem_cfg(s.K, s.S, folds(o), s.Cin,
                  [&](auto c) { e = launch_elem_cfg<decltype(c)>(s, x, w, bias, dst, mode, o, stream); });
    return e;
}

hipError_t conv2d_general_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                                 float* dst, int mode, const PoolOpts& o, hipStream_t stream) {
    const dim3 grid((unsigned)conv2d_general_parts(s), s.B);
    const int pm = o.pool_max ? 1 : 0, rl = o.relu ? 1 : 0;
    const int units = general_units(s);
    if (mode == OUT_MAP)
        hipLaunchKernelGGL(conv2d_pool_general_kernel<OUT_MAP>, grid, dim3(256), 0, stream, x, w, bias, dst, s.Cin,
                           s.H, s.W, s.Cout, s.K, s.S, s.PH, s.PW, pm, rl, units);
    else
        hipLaunchKernelGGL(conv2d_pool_general_kernel<OUT_PARTIAL>, grid, dim3(256), 0, stream, x, w, bias, dst,
                           s.Cin, s.H, s.W, s.Cout, s.K, s.S, s.PH, s.PW, pm, rl, units);
    return hipGetLastError();
}

}  // namespace fconv
