// dwsep_conv1d.hip -- depthwise Conv1d(K, zero pad, stride 1) -> pointwise 1x1 Conv1d + bias,
// fused so that the depthwise output never reaches HBM.
//
// Method: POPCORNBENCH reasoning trace "Kimi-K2.6 l2_p7" (depthwise-separable
// Conv1d).  Its per-output formula is computed in the separable order:
//     D[c,t]   = sum_k w_dw[c,k] * x[c, t+k-pad]     (zero outside [0,T))
//     y[o,t]   = b_pw[o] + sum_c w_pw[o,c] * D[c,t]
// i.e. C*K + O*C multiply-adds per time step, not the O*C*K of the dense
// fused 9-tap weight that the trace also considers.  The pointwise stage is a
// real GEMM (M = O, N = time, k = C per batch item) and runs on fp32 matrix
// cores; the depthwise stage (about 2% of the work) runs on the vector ALUs
// and writes its result straight into LDS in the layout the GEMM reads.
//
// Workgroup: one batch item, a tile of OT output channels x TT time steps,
// all C input channels in chunks of CC:
//   1. x[c0:c0+CC, t0-pad : t0+TT+K-1-pad] -> LDS.  Each wave copies whole
//      rows through a per-row buffer resource (scalar registers); the
//      hardware bounds check supplies the zero padding.
//   2. Depthwise stage -> D[t][c] in LDS (row pitch CC+4 floats).  Each wave
//      owns CC/NW channels, so their taps are wave-uniform scalar loads, and
//      lane l makes step t = l (consecutive LDS words, no bank conflicts).
//   3. v_mfma_f32_16x16x4_f32 over the chunk.  Within each group of 16
//      channels, lane group g holds channels 4g..4g+3 for 4 consecutive
//      MFMA steps, so one 16-byte load gives a lane its 4 weights (w_pw rows
//      are contiguous in c) and one 16-byte LDS read its 4 D values.  The
//      weight loads run one 16-channel group ahead of the matrix
//      instructions that use them; the group index is a scalar offset.
//   4. + bias, store.  The output is written with non-temporal stores: it is
//      read by nobody here, and kept out of the caches it does not evict the
//      input the next calls read (x[32,256,4096]: y is twice the size of x,
//      and allocating it in the 256 MB last-level cache pushed x out; the
//      streaming stores took 0.281 to 0.271 ms).
// Out-of-range output rows read a clamped (valid) weight row and are never
// stored.  Channels >= C have D = 0, so whatever weights pair with them
// (the next row's, or 0 past the end of w_pw) add nothing.
#include <type_traits>

#include "fconv_device.hpp"
#include "fconv_internal.hpp"

namespace fconv {

// OB, TB: 16x16 output blocks per wave along o and t; WO, WT: waves along o
// and t; CC: channel chunk; KC: compile-time depthwise taps (0 = runtime K;
// -1 = runtime K with dilation 2, 4 or 8, -2 = runtime K with any dilation,
// tall tile only);
// MINW: waves per SIMD the register budget must allow.
template <int OB_, int TB_, int WO_, int WT_, int CC_, int KC_, int MINW_>
struct DwsepCfg {
    static constexpr int OB = OB_, TB = TB_, WO = WO_, WT = WT_, CC = CC_, KC = KC_, MINW = MINW_;
    static constexpr int NW = WO * WT;
    static constexpr int NT = 64 * NW;
    static constexpr int OT = 16 * OB * WO;
    static constexpr int TT = 16 * TB * WT;
    static constexpr int CCP = CC + 4;  // D row pitch in floats
    static constexpr int CPW = CC / NW; // depthwise channels per wave
    static_assert(CC % 16 == 0, "channel chunk must be whole 16-channel groups");
    static_assert(CC % NW == 0 && CPW % 4 == 0, "each wave makes whole 4-channel groups of D");
};

template <class Cfg, bool VEC>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINW) void dwsep_mfma_kernel(
    const float* __restrict__ x, const float* __restrict__ w_dw, const float* __restrict__ w_pw,
    const float* __restrict__ b_pw, float* __restrict__ y, int C, int T, int Kr, int O, int pad, int Tout,
    int stride, int dil) {
    constexpr int OB = Cfg::OB, TB = Cfg::TB, WO = Cfg::WO, CC = Cfg::CC, CCP = Cfg::CCP, CPW = Cfg::CPW;
    constexpr int TT = Cfg::TT, NW = Cfg::NW;
    const int K = Cfg::KC > 0 ? Cfg::KC : Kr;

    extern __shared__ float lds[];
    float* Ds = lds;             // [TT][CCP]
    float* xs = lds + TT * CCP;  // [CC][XW]
    // input steps a time tile reads; the compile-time-K instances run only
    // with stride = dilation = 1
    const int XW = Cfg::KC > 0 ? TT + K - 1 : (TT - 1) * stride + (K - 1) * dil + 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wo = wave % WO;
    const int wt = wave / WO;
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int t0 = blockIdx.x * TT;
    const int o0 = blockIdx.y * Cfg::OT + wo * 16 * OB;
    const int b = blockIdx.z;
    const float* xb = x + (size_t)b * C * T;
    const int NG = (C + 15) / 16;  // 16-channel groups

    // Pointwise weights: lane (g, l16) of block ob reads row min(o, O-1) at
    // channel 16*grp + 4g.  The group moves the resource's base (scalar
    // arithmetic), so the per-lane offsets stay fixed and the bounds check
    // still covers every byte read: loads past the end of w_pw return 0.
    int woff[OB];
#pragma unroll
    for (int ob = 0; ob < OB; ++ob) woff[ob] = (min(o0 + ob * 16 + l16, O - 1) * C + 4 * g) * 4;
    auto load_pw = [&](floatx4 (&a)[OB], int grp) {
        const buf_rsrc rw = make_rsrc(w_pw + 16 * grp, (O * C - 16 * grp) * 4);
#pragma unroll
        for (int ob = 0; ob < OB; ++ob) {
            if constexpr (VEC) {
                a[ob] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff[ob], 0, 0));
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    a[ob][j] =
                        __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, woff[ob] + 4 * j, 0, 0));
            }
        }
    };

    floatx4 acc[OB][TB];
#pragma unroll
    for (int i = 0; i < OB; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    floatx4 a_next[OB];
    load_pw(a_next, 0);

    // 1. Input rows c0..c0+CC-1, steps t0-pad .. t0-pad+XW-1, copied into
    //    LDS a row per wave at a time through per-row buffer resources.  With
    //    a compile-time K each lane's column offsets are fixed and the next
    //    chunk's rows are loaded into registers while this chunk computes.
    constexpr int UR = 4;  // rows in flight per wave (runtime-K path)
    const int nch = (XW + 63) / 64;
    constexpr int NCHC = Cfg::KC > 0 ? (TT + Cfg::KC - 1 + 63) / 64 : 1;
    constexpr int RPW = CC / NW;  // rows per wave
    int voffc[NCHC];
#pragma unroll
    for (int ch = 0; ch < NCHC; ++ch) {
        const int u = ch * 64 + lane;
        const int src = t0 - pad + u;
        voffc[ch] = (u < XW && src >= 0) ? src * 4 : kBufOOB;  // src >= T: past the row's end
    }
    float xv[Cfg::KC > 0 ? RPW : 1][NCHC];
    auto load_rows = [&](int c0) {
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
            const int row = wave + rr * NW;
            const bool ok = c0 + row < C;
            const buf_rsrc rrow = make_rsrc(xb + (ok ? (size_t)(c0 + row) * T : 0), ok ? T * 4 : 0);
#pragma unroll
            for (int ch = 0; ch < NCHC; ++ch) xv[rr][ch] = buf_load_f32(rrow, voffc[ch]);
        }
    };
    if constexpr (Cfg::KC > 0) load_rows(0);

    for (int c0 = 0; c0 < C; c0 += CC) {
        __syncthreads();  // the previous chunk's LDS data is no longer read
        if constexpr (Cfg::KC > 0) {
#pragma unroll
            for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
                for (int ch = 0; ch < NCHC; ++ch) {
                    const int u = ch * 64 + lane;
                    if (u < XW) xs[(wave + rr * NW) * XW + u] = xv[rr][ch];
                }
            if (c0 + CC < C) load_rows(c0 + CC);
        } else {
            for (int ch = 0; ch < nch; ++ch) {
                const int u = ch * 64 + lane;
                const int src = t0 * stride - pad + u;
                const int voff = (u < XW && src >= 0) ? src * 4 : kBufOOB;
                for (int r0 = wave; r0 < CC; r0 += NW * UR) {
                    float v[UR];
#pragma unroll
                    for (int uu = 0; uu < UR; ++uu) {
                        const int row = r0 + uu * NW;
                        const bool ok = (row < CC) && (c0 + row < C);
                        const buf_rsrc rrow = make_rsrc(xb + (ok ? (size_t)(c0 + row) * T : 0), ok ? T * 4 : 0);
                        v[uu] = buf_load_f32(rrow, voff);
                    }
#pragma unroll
                    for (int uu = 0; uu < UR; ++uu) {
                        const int row = r0 + uu * NW;
                        if (row < CC && u < XW) xs[row * XW + u] = v[uu];
                    }
                }
            }
        }
        __syncthreads();
        // 2. depthwise stage: wave owns channels wave*CPW .. +CPW-1 of the chunk
        for (int t = lane; t < TT; t += 64) {
            float d[CPW];
#pragma unroll
            for (int cc = 0; cc < CPW; ++cc) {
                const int c = wave * CPW + cc;
                const float* wr = w_dw + (size_t)min(c0 + c, C - 1) * K;  // rows >= C: x is 0 there
                const float* xr = xs + c * XW + (Cfg::KC > 0 ? t : t * stride);
                float s = 0.f;
                if constexpr (Cfg::KC > 0) {
#pragma unroll
                    for (int k = 0; k < Cfg::KC; ++k) s += wr[k] * xr[k];
                } else {
                    for (int k = 0; k < K; ++k) s += wr[k] * xr[k * dil];
                }
                d[cc] = s;
            }
#pragma unroll
            for (int c4 = 0; c4 < CPW; c4 += 4)
                *reinterpret_cast<floatx4*>(Ds + t * CCP + wave * CPW + c4) =
                    floatx4{d[c4], d[c4 + 1], d[c4 + 2], d[c4 + 3]};
        }
        __syncthreads();
        // 3. pointwise GEMM over this chunk, weights one group ahead
#pragma unroll
        for (int s16 = 0; s16 < CC; s16 += 16) {
            const int grp = c0 / 16 + s16 / 16;
            if (grp < NG) {
                floatx4 a[OB];
#pragma unroll
                for (int ob = 0; ob < OB; ++ob) a[ob] = a_next[ob];
                if (grp + 1 < NG) load_pw(a_next, grp + 1);
                floatx4 bq[TB];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const int t = (wt * TB + tb) * 16 + l16;
                    bq[tb] = *reinterpret_cast<const floatx4*>(Ds + t * CCP + s16 + 4 * g);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int ob = 0; ob < OB; ++ob)
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb) acc[ob][tb] = mfma_16x16x4(a[ob][j], bq[tb][j], acc[ob][tb]);
            }
        }
    }

    // 4. epilogue: lane (g, l16) holds y[o0 + ob*16 + 4g + r, t0 + (wt*TB + tb)*16 + l16]
    const buf_rsrc rb = make_rsrc(b_pw, b_pw ? O * 4 : 0);
    float* yb = y + (size_t)b * O * Tout;
#pragma unroll
    for (int ob = 0; ob < OB; ++ob)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = o0 + ob * 16 + 4 * g + r;
            const float bo = buf_load_f32(rb, o < O ? o * 4 : kBufOOB);
            if (o >= O) continue;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int t = t0 + (wt * TB + tb) * 16 + l16;
                if (t < Tout) __builtin_nontemporal_store(acc[ob][tb][r] + bo, yb + (size_t)o * Tout + t);
            }
        }
}

// Instances.  Wide (O > 64): 256 x 64 tile, 8 waves of 32 x 64, register
// budget for 4 waves per SIMD.  Small: 32 x 32.  Narrow: 256 x 16, for
// strides/dilations whose 64-step input window would not fit in LDS.
// FCONV_CFG_DW9 lets a build override the K = 9 instance's tiling.
#ifndef FCONV_CFG_DW9
#define FCONV_CFG_DW9 2, 4, 8, 1, 64, 9, 4
#endif
using DwWide9 = DwsepCfg<FCONV_CFG_DW9>;
using DwWideK = DwsepCfg<2, 4, 8, 1, 64, 0, 4>;
using DwNarrowK = DwsepCfg<2, 1, 8, 1, 32, 0, 4>;
using DwSmallK = DwsepCfg<1, 1, 2, 2, 16, 0, 2>;

// ---------------------------------------------------------------- tall-tile variant

// Strides 1 to 5 (any dilation), any C, O > 256: a 512 x 64 tile (8
// waves of 64 x 64), so each depthwise value is made once per time tile
// instead of once per 256 output channels, and the matrix cores see twice
// the work per depthwise instruction.  Smaller O takes the same kernel with
// 256- or 128-row tiles (8 waves of 32 x 64 or 16 x 64) and, at stride 1
// and dilation 1, 64- or 32-row tiles (4 or 2 waves of 16 x 64; with a
// stride or dilation O <= 64 runs the 128-row tile, its waves past O idle).
// The extra accumulator registers are paid for by staging x,
// the depthwise taps and the bias with LDS-direct buffer loads
// (buffer_load_dword ... lds: memory to LDS with no register round trip),
// which also lets the next chunk's rows stream in while the current chunk's
// GEMM runs.
//
// Per chunk of CC channels (every chunk has CC/16 groups; in a last,
// partial chunk the channels >= C are staged as 0, so their depthwise value
// is 0, and their pointwise weights load as 0):
//   wait for this wave's LDS-direct loads; barrier (xs holds chunk i, Ds is free)
//   depthwise xs -> Ds; barrier (Ds ready, xs free)
//   LDS-direct loads of chunk i+1 into xs
//   GEMM over the chunk's 16-channel groups
// The accumulators start at the bias.  Epilogue: each wave transposes its
// 64 x 64 block through LDS, 16 rows at a time, and writes rows of 64 steps
// with 16-byte stores; ragged tiles store element by element.
// Depthwise: lane (dc, dj) = (lane/8, lane%8) makes steps 8dj .. 8dj+7 of
// the wave's channel dc from staged steps (16-byte LDS reads) and the
// channel's K taps (staged in LDS too, so the stage needs no scalar loads,
// whose out-of-order return would serialize the LDS reads): 8 independent
// multiply-add chains per lane.  The K = 9 instance reads 16 steps and 9
// taps once; the runtime-K instance goes over the taps in blocks of 8, 16
// steps per block (8 / dil taps per block with dilation 2, 4 or 8, and tap
// by tap with single-word reads for any other dilation).
// LDS: xs [CC][132], then Ds: [64][CC+4] for the GEMM operand and
// 8 x [16][68] in the epilogue, then the bias [512] and the taps [CC][K]
// (70,656 + 256 K bytes: 72,960 for K = 9, two workgroups per CU up to
// K = 44).  Stride 2: 64 outputs read 127 + K steps, staged as three runs
// (xs [CC][196]); the epilogue then stages through xs and Ds, so the total
// is 69,632 + 256 K bytes (71,936 for K = 9).  Strides 3, 4 and 5 stage
// four, five and six runs (86,016, 102,400 and 118,784 + 256 K bytes): one
// workgroup per CU.
// Row r of xs holds input steps t0-pad .. t0-pad+127 (two 64-lane
// runs; steps past the (K-1)*dil halo or outside [0, T) load as 0); the
// runtime-K blocks read up to step 8*7 + 8*floor((K-1)*dil/8) + 15, so
// (K-1)*dil <= 63.  Dilations other than 1 run on runtime-K instances.
// Pointwise weights: lane (g, l16) of block ob keeps channels 4g..4g+3 of
// the current group; the registers of block ob are refilled with the next
// group's weights as soon as its 16 matrix instructions are issued.
// Tall-tile LDS geometry for stride ST: NRUN 64-step runs staged per input
// row (64 outputs read (TT - 1) * ST + (K - 1) * dil + 1 steps: 2 runs at
// stride 1, ST + 1 above, for windows of at most 64 steps), a row pitch
// of the runs + 4 (rows of consecutive channels start 16 bytes apart on the
// banks), and the float count of the region after xs.  With stride 1 the
// epilogue's [NW][16][68] staging gets a region of its own beside Ds; with
// larger strides the wider xs rows leave no room for it, so the epilogue stages
// through xs and Ds together (both free by then: the last chunk stages no
// next chunk) and the region after xs is Ds alone.
// WX = 1 stages one more run per row, for windows of 65 to 128 steps.
template <class Cfg, int ST, int WX>
struct TallGeom {
    static constexpr int NRUN = (ST + 1 > 2 ? ST + 1 : 2) + WX;
    static constexpr int XP = 64 * NRUN + 4;
    static constexpr int OP = 68;
    static constexpr int EPI = Cfg::NW * 16 * OP;
    static constexpr int DS = Cfg::TT * Cfg::CCP;
    static constexpr int DSF = NRUN == 2 ? (DS > EPI ? DS : EPI) : DS;
    static_assert(NRUN == 2 || Cfg::CC * XP + DS >= EPI, "the epilogue fits xs + Ds");
};

template <class Cfg, int ST, int WX>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINW) void dwsep_tall_kernel(
    const float* __restrict__ x, const float* __restrict__ w_dw, const float* __restrict__ w_pw,
    const float* __restrict__ b_pw, float* __restrict__ y, int C, int T, int Kr, int O, int pad, int Tout, int n_tt,
    int n_ot, int vec_out, int dil) {
    constexpr int OB = Cfg::OB, TB = Cfg::TB, CC = Cfg::CC, CCP = Cfg::CCP, CPW = Cfg::CPW;
    using G = TallGeom<Cfg, ST, WX>;
    constexpr int TT = Cfg::TT, NW = Cfg::NW, XP = G::XP, OP = G::OP, DSF = G::DSF, NRUN = G::NRUN;
    static_assert(WX == 0 || (ST == 1 && Cfg::KC <= 0), "wide windows: stride 1, runtime K");
    static_assert(Cfg::KC >= -2, "KC: 9, 0, -1 or -2");
    static_assert(Cfg::WT == 1 && TT == 64 && Cfg::WO == NW && (OB == 4 || OB == 2 || OB == 1) && TB == 4,
                  "waves of 16 OB x 64 along o");
    static_assert(CC % NW == 0 && CC % 16 == 0, "whole rows per wave, whole groups per chunk");
    const int K = Cfg::KC > 0 ? Cfg::KC : Kr;
    const int XW = (TT - 1) * ST + (K - 1) * dil + 1;  // input steps the tile reads (<= 64 * NRUN)

    // xs first: the depthwise reads then fit the short LDS offset fields
    extern __shared__ float lds[];
    float* xs = lds;            // [CC][XP]
    float* Ds = lds + CC * XP;  // [TT][CCP]; epilogue: [NW][16][OP]
    float* bs = Ds + DSF;       // [NW][64]: each wave's 64 bias values
    float* ws = bs + NW * 64;   // [CC][K], rounded up to whole 64-float runs: the chunk's taps
    auto* xs3 = (__attribute__((address_space(3))) float*)xs;
    auto* bs3 = (__attribute__((address_space(3))) float*)bs;
    auto* ws3 = (__attribute__((address_space(3))) float*)ws;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4;
    const int l16 = lane & 15;
    // tile = (b * n_ot + ot) * n_tt + tt in launch order.  (Dealing the
    // tiles to the XCDs in contiguous runs, so that neighbouring time tiles
    // share an L2 for their halo lines, read 160 MB instead of 292 MB of x
    // for x[32,256,4096] but ran 2 % slower.)
    const int tile = blockIdx.x;
    const int tq = tile / n_tt;
    const int bi = tq / n_ot;
    const int t0 = (tile - tq * n_tt) * TT;  // first output step
    const int o0 = (tq - bi * n_ot) * Cfg::OT + wave * 16 * OB;  // this wave's first output channel
    const float* xb = x + (size_t)bi * C * T;

    // 1. staging: per row NRUN LDS-direct loads of 64 consecutive steps from
    //    input step t0*ST - pad; rows >= C get an empty resource and load 0
    int voff[NRUN];
#pragma unroll
    for (int r = 0; r < NRUN; ++r) {
        const int u = 64 * r + lane;
        const int src = t0 * ST - pad + u;
        voff[r] = (u < XW && src >= 0) ? src * 4 : kBufOOB;
    }
    auto stage = [&](int c0) {
#pragma unroll
        for (int i = 0; i < CC / NW; ++i) {
            const int row = c0 + wave + i * NW;
            const buf_rsrc rr = make_rsrc(xb + (size_t)min(row, C - 1) * T, row < C ? T * 4 : 0);
#pragma unroll
            for (int r = 0; r < NRUN; ++r)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, xs3 + (wave + i * NW) * XP + 64 * r, 4, voff[r], 0, 0,
                                                         0);
        }
        // the chunk's taps w_dw[c0 .. c0+CC-1][0..K-1] are contiguous: runs of
        // 64 floats (0 past channel C-1; the ws region is whole runs)
        // (each run's resource starts at the run, so every load takes the
        // lane's own offset: no per-run offset register to keep live)
        const int n = min(CC, C - c0) * K;
        for (int q = wave; q < (K * CC + 63) / 64; q += NW) {
            const buf_rsrc rt = make_rsrc(w_dw + (size_t)c0 * K + 64 * q, max(n - 64 * q, 0) * 4);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, ws3 + 64 * q, 4, lane * 4, 0, 0, 0);
        }
    };

    // Pointwise weights.  rw[ob] covers rows o0 + 16*ob .. O-1 of w_pw (none
    // past O), so lanes whose row is >= O load 0; lane (g, l16) reads row
    // 16*ob + l16 of it at channels cb + 4g .. +3, with the channel offset
    // cb*4 in the scalar offset field.  A lane in range stays inside its
    // row, so the loads are in bounds whether or not the scalar offset
    // enters the hardware range check.  Only whole runs of 4 channels below C
    // load (rows of any C are 4-byte aligned, all a 4-dword buffer load
    // needs); a lane whose run reaches C or past it takes an out-of-range
    // offset and loads 0.  The run that C cuts (C % 4 != 0) is added once
    // after the last chunk (step 3b).
    const int woff = (l16 * C + 4 * g) * 4;
    buf_rsrc rw[OB];
#pragma unroll
    for (int ob = 0; ob < OB; ++ob) {
        const int rows = O - (o0 + 16 * ob);
        rw[ob] = make_rsrc(w_pw + (size_t)(rows > 0 ? o0 + 16 * ob : 0) * C, rows > 0 ? rows * C * 4 : 0);
    }
    auto load_pw = [&](int ob, int cb) {
        const int off = cb + 4 * g + 3 < C ? woff : kBufOOB;
        return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(rw[ob], off, cb * 4, 0));
    };

    // D[t][c] sits at column c ^ 4*(t >> 4) of row t: the 4-channel groups
    // stay whole for these 16-byte reads (all lanes of one read share
    // t >> 4 = tb, so they remain conflict-free), while the depthwise
    // stage's writes, whose lanes cover 8 rows 8 apart (row pitch 68:
    // every other row lands on the same banks), spread over 32 banks
    // instead of 8.  This halved the kernel's LDS bank-conflict cycles.
    auto read_d = [&](floatx4& dst, int tb, int s16) {
        dst = *reinterpret_cast<const floatx4*>(Ds + (tb * 16 + l16) * CCP + ((s16 + 4 * g) ^ (tb << 2)));
    };

    floatx4 acc[OB][TB];
    floatx4 a[OB];
#pragma unroll
    for (int ob = 0; ob < OB; ++ob) a[ob] = load_pw(ob, 0);
    stage(0);
    {
        // this wave's 64 bias values (0 past O or without a bias)
        const int rows = O - o0;
        const buf_rsrc rb = make_rsrc(b_pw + (rows > 0 ? o0 : 0), b_pw && rows > 0 ? rows * 4 : 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, bs3 + wave * 64, 4, lane * 4, 0, 0, 0);
    }

    for (int c0 = 0; c0 < C; c0 += CC) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's LDS-direct loads have landed
        __syncthreads();
        if (c0 == 0) {
            // the accumulators start at the bias
#pragma unroll
            for (int ob = 0; ob < OB; ++ob) {
                const floatx4 bo = *reinterpret_cast<const floatx4*>(bs + wave * 64 + 16 * ob + 4 * g);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) acc[ob][tb] = bo;
            }
        }
        // 2. depthwise -> Ds[t][c] for the wave's CPW channels (channels >= C
        //    read the zero rows staged for them, so their D is 0).  Lane
        //    (dc, dj) makes output steps 8dj .. 8dj+7, whose inputs start at
        //    staged step 8*ST*dj: NX = 8*ST + 8 staged steps cover 8 taps.
        constexpr int NX = 8 * ST + 8;
        if constexpr (Cfg::KC == 9) {
            static_assert(CPW == 8, "8 channels x 8 groups of 8 steps per wave");
            const int dj = lane & 7, dc = lane >> 3;
            const int c = wave * CPW + dc;
            float xv[NX], wv[9];
#pragma unroll
            for (int q = 0; q < NX / 4; ++q) {
                const floatx4 v = *reinterpret_cast<const floatx4*>(xs + c * XP + 8 * ST * dj + 4 * q);
                xv[4 * q] = v[0];
                xv[4 * q + 1] = v[1];
                xv[4 * q + 2] = v[2];
                xv[4 * q + 3] = v[3];
            }
#pragma unroll
            for (int k = 0; k < 9; ++k) wv[k] = ws[c * 9 + k];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float s = 0.f;
#pragma unroll
                for (int k = 0; k < 9; ++k) s += wv[k] * xv[ST * i + k];
                Ds[(8 * dj + i) * CCP + (c ^ ((dj >> 1) << 2))] = s;  // swizzled: see read_d
            }
        } else {
            // runtime K: the same lanes and chains, over blocks of 8 / dil
            // taps (KC = 0: dilation 1; KC = -1: dilation 2, 4 or 8, a
            // compile-time copy each, in instances of their own so that the
            // undilated ones keep their registers; KC = -2: any other
            // dilation, tap by tap); block kb reads NX staged
            // steps from 8*ST*dj + kb*dil (16-byte aligned: kb*dil is a
            // multiple of 8), tap kb + kk at step ST*i + kk*dil of them, and
            // (K - 1) * dil <= 63 (127 with WX = 1) keeps them inside the
            // row's 64 * NRUN staged steps
            static_assert(CPW == 8, "8 channels x 8 groups of 8 steps per wave");
            const int dj = lane & 7, dc = lane >> 3;
            const int c = wave * CPW + dc;
            float sacc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) sacc[i] = 0.f;
            auto taps = [&](auto dil_tag) {
                constexpr int D = decltype(dil_tag)::value, TPB = 8 / D;
                for (int kb = 0; kb < K; kb += TPB) {
                    float xv[NX];
#pragma unroll
                    for (int q = 0; q < NX / 4; ++q) {
                        const floatx4 v =
                            *reinterpret_cast<const floatx4*>(xs + c * XP + 8 * ST * dj + kb * D + 4 * q);
                        xv[4 * q] = v[0];
                        xv[4 * q + 1] = v[1];
                        xv[4 * q + 2] = v[2];
                        xv[4 * q + 3] = v[3];
                    }
#pragma unroll
                    for (int kk = 0; kk < TPB; ++kk) {
                        if (kb + kk < K) {
                            const float wk = ws[c * K + kb + kk];
#pragma unroll
                            for (int i = 0; i < 8; ++i) sacc[i] += wk * xv[ST * i + kk * D];
                        }
                    }
                }
            };
            if constexpr (Cfg::KC == -2) {
                // any other dilation: tap k reads the 8 steps ST apart from
                // 8*ST*dj + k*dil one word at a time (paired reads; the start
                // is not 16-byte aligned), the same chains
                for (int k = 0; k < K; ++k) {
                    const float wk = ws[c * K + k];
                    const float* xr = xs + c * XP + 8 * ST * dj + k * dil;
#pragma unroll
                    for (int i = 0; i < 8; ++i) sacc[i] += wk * xr[ST * i];
                }
            } else if constexpr (Cfg::KC < 0) {
                if (dil == 2)
                    taps(std::integral_constant<int, 2>{});
                else if (dil == 4)
                    taps(std::integral_constant<int, 4>{});
                else
                    taps(std::integral_constant<int, 8>{});
            } else {
                taps(std::integral_constant<int, 1>{});
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) Ds[(8 * dj + i) * CCP + (c ^ ((dj >> 1) << 2))] = sacc[i];
        }
        __syncthreads();
        if (c0 + CC < C) stage(c0 + CC);
        // 3. pointwise GEMM over the chunk's 16-channel groups.  Block ob's
        //    weight registers take the next group's weights as soon as its
        //    16 products are issued (past the last group these load 0); the
        //    last block runs in two halves of the time blocks, and each
        //    half's D registers take the next group's D once used.  The
        //    scheduling fences keep that order: without them the compiler
        //    moves the next group's first products up against their loads.
        floatx4 bq[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) read_d(bq[tb], tb, 0);
#pragma unroll
        for (int s16 = 0; s16 < CC; s16 += 16) {
            const int cb = c0 + s16 + 16;  // first channel of the next group
#pragma unroll
            for (int ob = 0; ob < OB - 1; ++ob) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) acc[ob][tb] = mfma_16x16x4(a[ob][j], bq[tb][j], acc[ob][tb]);
                a[ob] = load_pw(ob, cb);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int h = 0; h < TB; h += 2) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int tb = h; tb < h + 2; ++tb)
                        acc[OB - 1][tb] = mfma_16x16x4(a[OB - 1][j], bq[tb][j], acc[OB - 1][tb]);
                if (s16 + 16 < CC) {
                    read_d(bq[h], h, s16 + 16);
                    read_d(bq[h + 1], h + 1, s16 + 16);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            a[OB - 1] = load_pw(OB - 1, cb);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // 3b. C % 4 != 0: channels cl .. C-1 (cl = C rounded down to a multiple
    //     of 4) belong to the lane group g = (cl % 16) / 4 of the group at
    //     channel cl & ~15, in the last chunk, whose D values are still in Ds
    //     (0 past channel C-1).  That lane group loads their weights one
    //     channel at a time (the other lanes and channels >= C load 0), and
    //     three more matrix steps add them.
    if (C & 3) {
        const int cl = C & ~3, cg = cl & ~15;
        const int s16 = cg - (C - 1) / CC * CC;
        const bool mine = 4 * g == (cl & 15);
        floatx4 bq[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) read_d(bq[tb], tb, s16);
#pragma unroll
        for (int ob = 0; ob < OB; ++ob)
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int off = mine && cl + j < C ? woff + 4 * j : kBufOOB;
                a[ob][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw[ob], off, cg * 4, 0));
            }
#pragma unroll
        for (int ob = 0; ob < OB; ++ob)
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) acc[ob][tb] = mfma_16x16x4(a[ob][j], bq[tb][j], acc[ob][tb]);
    }

    // 4. epilogue: lane (g, l16) holds y[o0 + 16*ob + 4g + r, t0 + 16*tb + l16]
    float* yb = y + (size_t)bi * O * Tout;
    __syncthreads();  // every wave is done reading Ds (outside the branch: o0 differs per wave)
    if (vec_out && o0 + 16 * OB <= O && t0 + TT <= Tout) {
        float* ow = (NRUN == 2 ? Ds : lds) + wave * 16 * OP;  // see TallGeom
#pragma unroll
        for (int ob = 0; ob < OB; ++ob) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int r = 0; r < 4; ++r) ow[(4 * g + r) * OP + 16 * tb + l16] = acc[ob][tb][r];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const floatx4 v = *reinterpret_cast<const floatx4*>(ow + (4 * i + g) * OP + 4 * l16);
                __builtin_nontemporal_store(
                    v, reinterpret_cast<floatx4*>(yb + (size_t)(o0 + 16 * ob + 4 * i + g) * Tout + t0 + 4 * l16));
            }
            __builtin_amdgcn_wave_barrier();
        }
    } else {
#pragma unroll
        for (int ob = 0; ob < OB; ++ob)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = o0 + ob * 16 + 4 * g + r;
                if (o >= O) continue;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const int t = t0 + tb * 16 + l16;
                    if (t < Tout) __builtin_nontemporal_store(acc[ob][tb][r], yb + (size_t)o * Tout + t);
                }
            }
    }
}

// The tall tile's heights for one depthwise stage KC: 512 rows (8 waves of
// 64 x 64) for O > 256; 256 rows (8 waves of 32 x 64) and 128 rows (16 x 64)
// for 64 < O <= 256, so no wave computes rows past O; for O <= 64, 64 rows as
// 4 waves of 16 x 64 (32-channel chunks) and 32 rows as 2 waves (16-channel
// chunks), so each wave still makes the depthwise values of 8 channels.  M is
// the 512-row tile's register budget in waves per SIMD: 2 at strides 3 to
// 5, whose staged rows leave LDS for one workgroup per CU anyway (at 128
// VGPRs those instances spilled 11-13 registers).
template <int KC, int M>
struct TallSet {
    using H512 = DwsepCfg<4, 4, 8, 1, 64, KC, M>;
    using H256 = DwsepCfg<2, 4, 8, 1, 64, KC, 4>;
    using H128 = DwsepCfg<1, 4, 8, 1, 64, KC, 4>;
    using H64 = DwsepCfg<1, 4, 4, 1, 32, KC, 4>;
    using H32 = DwsepCfg<1, 4, 2, 1, 16, KC, 4>;
};

template <class Cfg, int ST, int WX>
static constexpr size_t tall_lds_bytes(int K) {
    using G = TallGeom<Cfg, ST, WX>;
    return ((size_t)Cfg::CC * G::XP + G::DSF + (size_t)Cfg::NW * 64 + (size_t)(K * Cfg::CC + 63) / 64 * 64) *
           sizeof(float);
}


// ---------------------------------------------------------------- dense-fused variant

// The l2_p7 trace's dense-fused form: one convolution with the combined
// weight W[o,c,k] = w_pw[o,c] * w_dw[c,k] (equal to the separable result up
// to rounding, with C*K*O instead of C*(K+O) multiply-adds per step).  Kept
// as a second, independently arranged path and a comparison point.
//   Per 16-channel group and tap k the MFMA k-slots hold channels 4g..4g+3
//   (as in the separable kernel); A = w_pw[o, c] * w_dw[c, k] is formed in
//   registers (one multiply per weight fragment and tap), B is the staged
//   input x[c, t*stride + k*dilation - pad] read straight from LDS.
//   Epilogue: each wave's 32 x 64 block goes out 16 rows at a time through
//   LDS, as whole 256-byte row segments (16-byte stores); ragged tiles, an
//   unaligned y or Tout % 4 != 0 store element by element.
template <class Cfg>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINW) void dwsep_dense_kernel(
    const float* __restrict__ x, const float* __restrict__ w_dw, const float* __restrict__ w_pw,
    const float* __restrict__ b_pw, float* __restrict__ y, int C, int T, int K, int O, int pad, int Tout,
    int stride, int dil, int vec_out) {
    constexpr int OB = Cfg::OB, TB = Cfg::TB, WO = Cfg::WO, CC = Cfg::CC, TT = Cfg::TT, NW = Cfg::NW, NT = Cfg::NT;
    static_assert(Cfg::KC == 0, "the dense kernel takes K at run time");

    extern __shared__ float lds[];
    const int XW = (TT - 1) * stride + (K - 1) * dil + 1;
    float* xs = lds;             // [CC][XW]
    float* wsm = lds + CC * XW;  // [CC][K] depthwise taps of the chunk

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wo = wave % WO;
    const int wt = wave / WO;
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int t0 = blockIdx.x * TT;
    const int o0 = blockIdx.y * Cfg::OT + wo * 16 * OB;
    const int b = blockIdx.z;
    const float* xb = x + (size_t)b * C * T;

    int woff[OB];
#pragma unroll
    for (int ob = 0; ob < OB; ++ob) woff[ob] = (min(o0 + ob * 16 + l16, O - 1) * C + 4 * g) * 4;

    floatx4 acc[OB][TB];
#pragma unroll
    for (int i = 0; i < OB; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int nch = (XW + 63) / 64;
    for (int c0 = 0; c0 < C; c0 += CC) {
        __syncthreads();
        for (int ch = 0; ch < nch; ++ch) {
            const int u = ch * 64 + lane;
            const int src = t0 * stride - pad + u;
            const int voff = (u < XW && src >= 0) ? src * 4 : kBufOOB;
            for (int row = wave; row < CC; row += NW) {
                const bool ok = c0 + row < C;
                const buf_rsrc rrow = make_rsrc(xb + (ok ? (size_t)(c0 + row) * T : 0), ok ? T * 4 : 0);
                const float v = buf_load_f32(rrow, voff);
                if (u < XW) xs[row * XW + u] = v;
            }
        }
        const int nw_valid = min(CC, C - c0) * K;
        for (int i = tid; i < CC * K; i += NT) {
            const float v = w_dw[(size_t)c0 * K + min(i, nw_valid - 1)];
            wsm[i] = i < nw_valid ? v : 0.f;
        }
        __syncthreads();
        for (int s16 = 0; s16 < CC; s16 += 16) {
            const int grp = (c0 + s16) / 16;
            if (c0 + s16 >= C) break;
            // pointwise weights of channels 16*grp + 4g .. +3 (past the end of
            // w_pw: 0; past C: the next row's, multiplied by x = 0)
            const buf_rsrc rw = make_rsrc(w_pw + 16 * grp, (O * C - 16 * grp) * 4);
            floatx4 apw[OB];
#pragma unroll
            for (int ob = 0; ob < OB; ++ob)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    apw[ob][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, woff[ob] + 4 * j,
                                                                                              0, 0));
            for (int k = 0; k < K; ++k) {
                float bv[TB][4];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const int tl = (wt * TB + tb) * 16 + l16;
#pragma unroll
                    for (int j = 0; j < 4; ++j) bv[tb][j] = xs[(s16 + 4 * g + j) * XW + tl * stride + k * dil];
                }
                float wk[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) wk[j] = wsm[(s16 + 4 * g + j) * K + k];
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int ob = 0; ob < OB; ++ob) {
                        const float a = apw[ob][j] * wk[j];
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb) acc[ob][tb] = mfma_16x16x4(a, bv[tb][j], acc[ob][tb]);
                    }
            }
        }
    }

    const buf_rsrc rb = make_rsrc(b_pw, b_pw ? O * 4 : 0);
    float* yb = y + (size_t)b * O * Tout;
    float bo[OB][4];
#pragma unroll
    for (int ob = 0; ob < OB; ++ob)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = o0 + ob * 16 + 4 * g + r;
            bo[ob][r] = buf_load_f32(rb, o < O ? o * 4 : kBufOOB);
        }
    // A wave's row segment is TB * 16 steps; with WT = 1 that is the tile.
    static_assert(Cfg::WT == 1 && TB * 16 == 64, "the staged store writes 64-step rows");
    constexpr int OP = 68;  // LDS row pitch: the four lane groups' rows start 16 banks apart
    __syncthreads();  // every wave is done reading xs and wsm (outside the branch: o0 differs per wave)
    if (vec_out && o0 + 16 * OB <= O && t0 + TT <= Tout) {
        float* ow = lds + wave * 16 * OP;
#pragma unroll
        for (int ob = 0; ob < OB; ++ob) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int r = 0; r < 4; ++r) ow[(4 * g + r) * OP + 16 * tb + l16] = acc[ob][tb][r] + bo[ob][r];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const floatx4 v = *reinterpret_cast<const floatx4*>(ow + (4 * i + g) * OP + 4 * l16);
                __builtin_nontemporal_store(
                    v, reinterpret_cast<floatx4*>(yb + (size_t)(o0 + 16 * ob + 4 * i + g) * Tout + t0 + 4 * l16));
            }
            __builtin_amdgcn_wave_barrier();
        }
    } else {
#pragma unroll
        for (int ob = 0; ob < OB; ++ob)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = o0 + ob * 16 + 4 * g + r;
                if (o >= O) continue;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const int t = t0 + (wt * TB + tb) * 16 + l16;
                    if (t < Tout) __builtin_nontemporal_store(acc[ob][tb][r] + bo[ob][r], yb + (size_t)o * Tout + t);
                }
            }
    }
}

using DwDense = DwsepCfg<2, 4, 8, 1, 64, 0, 4>;

// The staged input and taps, or (after the last chunk) the waves' 16-row
// output staging, whichever is larger.
static size_t dense_lds_bytes(const DwsepShape& s) {
    const long xw = (long)(DwDense::TT - 1) * s.stride + (long)(s.K - 1) * s.dil + 1;
    const size_t in = ((size_t)DwDense::CC * xw + (size_t)DwDense::CC * s.K) * sizeof(float);
    const size_t out = (size_t)DwDense::NW * 16 * 68 * sizeof(float);
    return in > out ? in : out;
}

bool dwsep_dense_supported(const DwsepShape& s) { return dense_lds_bytes(s) <= 160 * 1024; }

hipError_t dwsep_dense_launch(const DwsepShape& s, const float* x, const float* w_dw, const float* w_pw,
                              const float* b_pw, float* y, hipStream_t stream) {
    const size_t lds = dense_lds_bytes(s);
    hipError_t e = hipFuncSetAttribute((const void*)dwsep_dense_kernel<DwDense>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    dim3 grid((s.Tout + DwDense::TT - 1) / DwDense::TT, (s.O + DwDense::OT - 1) / DwDense::OT, s.B);
    const int vec_out = (s.Tout % 4 == 0) && ((uintptr_t)y % 16 == 0);
    hipLaunchKernelGGL(dwsep_dense_kernel<DwDense>, grid, dim3(DwDense::NT), lds, stream, x, w_dw, w_pw, b_pw, y, s.C,
                       s.T, s.K, s.O, s.pad, s.Tout, s.stride, s.dil, vec_out);
    return hipGetLastError();
}

template <class Cfg>
static size_t dw_lds_bytes(const DwsepShape& s) {
    const long xw = Cfg::KC > 0 ? Cfg::TT + Cfg::KC - 1 : (long)(Cfg::TT - 1) * s.stride + (long)(s.K - 1) * s.dil + 1;
    return ((size_t)Cfg::TT * Cfg::CCP + (size_t)Cfg::CC * xw) * sizeof(float);
}

static constexpr size_t kDwLdsLimit = 160 * 1024;

template <class Cfg>
static hipError_t launch_dw(const DwsepShape& s, const float* x, const float* w_dw, const float* w_pw,
                            const float* b_pw, float* y, hipStream_t stream) {
    const size_t lds = dw_lds_bytes<Cfg>(s);
    dim3 grid((s.Tout + Cfg::TT - 1) / Cfg::TT, (s.O + Cfg::OT - 1) / Cfg::OT, s.B);
    const bool vec = (s.C % 4 == 0) && ((uintptr_t)w_pw % 16 == 0);
    hipError_t e;
    if (vec) {
        e = hipFuncSetAttribute((const void*)dwsep_mfma_kernel<Cfg, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((dwsep_mfma_kernel<Cfg, true>), grid, dim3(Cfg::NT), lds, stream, x, w_dw, w_pw, b_pw,
                           y, s.C, s.T, s.K, s.O, s.pad, s.Tout, s.stride, s.dil);
    } else {
        e = hipFuncSetAttribute((const void*)dwsep_mfma_kernel<Cfg, false>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((dwsep_mfma_kernel<Cfg, false>), grid, dim3(Cfg::NT), lds, stream, x, w_dw, w_pw, b_pw,
                           y, s.C, s.T, s.K, s.O, s.pad, s.Tout, s.stride, s.dil);
    }
    return hipGetLastError();
}

// The tall kernel's 1-D grid holds every (time tile, output tile, item).
static bool tall_tiles_fit(const DwsepShape& s) {
    const int ot = TallSet<9, 4>::H32::OT;  // the smallest tile height
    const long n = (long)((s.Tout + 63) / 64) * ((s.O + ot - 1) / ot) * s.B;
    return n <= 0x7fffffffL;
}

template <class Cfg, int ST = 1, int WX = 0>
static hipError_t launch_tall(const DwsepShape& s, const float* x, const float* w_dw, const float* w_pw,
                              const float* b_pw, float* y, hipStream_t stream) {
    const size_t lds = tall_lds_bytes<Cfg, ST, WX>(s.K);
    hipError_t e = hipFuncSetAttribute((const void*)dwsep_tall_kernel<Cfg, ST, WX>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const int n_tt = (s.Tout + Cfg::TT - 1) / Cfg::TT, n_ot = (s.O + Cfg::OT - 1) / Cfg::OT;
    const int n_tiles = n_tt * n_ot * s.B;  // < 2^31: checked by tall_tiles_fit
    const int vec_out = (s.Tout % 4 == 0) && ((uintptr_t)y % 16 == 0);
    hipLaunchKernelGGL((dwsep_tall_kernel<Cfg, ST, WX>), dim3(n_tiles), dim3(Cfg::NT), lds, stream, x, w_dw, w_pw, b_pw,
                       y, s.C, s.T, s.K, s.O, s.pad, s.Tout, n_tt, n_ot, vec_out, s.dil);
    return hipGetLastError();
}

// The tall tile's choice for a shape: its depthwise stage (9: K = 9
// compiled, 0: runtime K, -1: dilation 2, 4 or 8, -2: any other dilation),
// its stride (1 to 5) and its window class (wx = 1: one more staged run, for
// windows of 65 to 128 steps at stride 1).  ok = false: no tall instance.
struct TallPick {
    bool ok;
    int kc, st, wx;
};

static TallPick pick_tall(const DwsepShape& s) {
#ifndef FCONV_DW_NO_TALL
    const int64_t win = (int64_t)(s.K - 1) * s.dil;
    if (s.stride <= 5 && (win <= 63 || (win <= 127 && s.stride == 1)) && tall_tiles_fit(s)) {
        const bool pow2 = s.dil == 2 || s.dil == 4 || s.dil == 8;
        const int kc = s.dil == 1 ? (s.K == 9 ? 9 : 0) : pow2 ? -1 : -2;
        return {true, kc, s.stride, win > 63 ? 1 : 0};
    }
#endif
    return {false, 0, 0, 0};
}

template <int KC, int ST, int WX = 0>
static hipError_t launch_tall_o(const DwsepShape& s, const float* x, const float* w_dw, const float* w_pw,
                                const float* b_pw, float* y, hipStream_t stream) {
    using S = TallSet<KC, (ST >= 3 ? 2 : 4)>;
    if (s.O > 256) return launch_tall<typename S::H512, ST, WX>(s, x, w_dw, w_pw, b_pw, y, stream);
    if (s.O > 128) return launch_tall<typename S::H256, ST, WX>(s, x, w_dw, w_pw, b_pw, y, stream);
    if (s.O > 64) return launch_tall<typename S::H128, ST, WX>(s, x, w_dw, w_pw, b_pw, y, stream);
    if (s.O > 32) return launch_tall<typename S::H64, ST, WX>(s, x, w_dw, w_pw, b_pw, y, stream);
    return launch_tall<typename S::H32, ST, WX>(s, x, w_dw, w_pw, b_pw, y, stream);
}

template <int ST>
static hipError_t launch_tall_st(int kc, const DwsepShape& s, const float* x, const float* w_dw,
                                 const float* w_pw, const float* b_pw, float* y, hipStream_t stream) {
    switch (kc) {
        case 9: return launch_tall_o<9, ST>(s, x, w_dw, w_pw, b_pw, y, stream);
        case 0: return launch_tall_o<0, ST>(s, x, w_dw, w_pw, b_pw, y, stream);
        case -1: return launch_tall_o<-1, ST>(s, x, w_dw, w_pw, b_pw, y, stream);
        default: return launch_tall_o<-2, ST>(s, x, w_dw, w_pw, b_pw, y, stream);
    }
}

static hipError_t launch_tall_pick(const TallPick& t, const DwsepShape& s, const float* x, const float* w_dw,
                                   const float* w_pw, const float* b_pw, float* y, hipStream_t stream) {
    if (t.wx) {
        switch (t.kc) {
            case 0: return launch_tall_o<0, 1, 1>(s, x, w_dw, w_pw, b_pw, y, stream);
            case -1: return launch_tall_o<-1, 1, 1>(s, x, w_dw, w_pw, b_pw, y, stream);
            default: return launch_tall_o<-2, 1, 1>(s, x, w_dw, w_pw, b_pw, y, stream);
        }
    }
    switch (t.st) {
        case 1: return launch_tall_st<1>(t.kc, s, x, w_dw, w_pw, b_pw, y, stream);
        case 2: return launch_tall_st<2>(t.kc, s, x, w_dw, w_pw, b_pw, y, stream);
        case 3: return launch_tall_st<3>(t.kc, s, x, w_dw, w_pw, b_pw, y, stream);
        case 4: return launch_tall_st<4>(t.kc, s, x, w_dw, w_pw, b_pw, y, stream);
        default: return launch_tall_st<5>(t.kc, s, x, w_dw, w_pw, b_pw, y, stream);
    }
}

// The older kernels (shapes the tall tile does not take): 0 = none fits,
// 1 = wide K=9, 2 = wide runtime-K, 3 = narrow runtime-K, 4 = small runtime-K.
static int pick_dw(const DwsepShape& s) {
    const bool unit = s.stride == 1 && s.dil == 1;
    if (s.O > 64) {
        if (unit && s.K == 9) return 1;
        if (dw_lds_bytes<DwWideK>(s) <= kDwLdsLimit) return 2;
        if (dw_lds_bytes<DwNarrowK>(s) <= kDwLdsLimit) return 3;
        return 0;
    }
    if (dw_lds_bytes<DwSmallK>(s) <= kDwLdsLimit) return 4;
    if (dw_lds_bytes<DwNarrowK>(s) <= kDwLdsLimit) return 3;
    return 0;
}

bool dwsep_supported(const DwsepShape& s) { return pick_tall(s).ok || pick_dw(s) != 0; }

hipError_t dwsep_launch(const DwsepShape& s, const float* x, const float* w_dw, const float* w_pw,
                        const float* b_pw, float* y, hipStream_t stream) {
    const TallPick t = pick_tall(s);
    if (t.ok) return launch_tall_pick(t, s, x, w_dw, w_pw, b_pw, y, stream);
    switch (pick_dw(s)) {
        case 1: return launch_dw<DwWide9>(s, x, w_dw, w_pw, b_pw, y, stream);
        case 2: return launch_dw<DwWideK>(s, x, w_dw, w_pw, b_pw, y, stream);
        case 3: return launch_dw<DwNarrowK>(s, x, w_dw, w_pw, b_pw, y, stream);
        case 4: return launch_dw<DwSmallK>(s, x, w_dw, w_pw, b_pw, y, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fconv
