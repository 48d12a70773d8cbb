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
//   1. x[c0:c0+CC, t0-pad : t0+TT+K-1-pad] and w_dw[c0:c0+CC, :] -> LDS
//      (coalesced, zero padded)
//   2. D[t][c] for the chunk -> LDS (row pitch CC+4 floats).  A thread makes
//      4 channels x TPT consecutive steps from a register window of the input.
//   3. v_mfma_f32_16x16x4_f32 over the chunk.  Within each group of 16
//      channels, lane group g holds channels 4g..4g+3 for 4 consecutive
//      MFMA steps, so one 16-byte global load gives a lane its 4 weights
//      (w_pw rows are contiguous in c) and one 16-byte LDS read its 4 D
//      values.  The weight loads run one 16-channel group ahead of the
//      matrix instructions that use them.
//   4. + bias, store.
// Out-of-range output channels read a clamped (valid) weight row and are
// never stored; channels >= C have D = 0, so their clamped weights add 0.
#include "fconv_device.hpp"
#include "fconv_internal.hpp"

namespace fconv {

// OB, TB: 16x16 output blocks per wave along o and t; WO, WT: waves along o
// and t; CC: channel chunk; TPT: time steps per thread in the depthwise
// stage; KC: compile-time depthwise taps (0 = runtime K); MINW: waves per
// SIMD the register budget must allow.
template <int OB_, int TB_, int WO_, int WT_, int CC_, int TPT_, int KC_, int MINW_>
struct DwsepCfg {
    static constexpr int OB = OB_, TB = TB_, WO = WO_, WT = WT_, CC = CC_, TPT = TPT_, KC = KC_, MINW = MINW_;
    static constexpr int NW = WO * WT;
    static constexpr int NT = 64 * NW;
    static constexpr int OT = 16 * OB * WO;
    static constexpr int TT = 16 * TB * WT;
    static constexpr int CCP = CC + 4;  // D row pitch in floats
    static_assert(CC % 16 == 0, "channel chunk must be whole 16-channel groups");
    static_assert(TT % TPT == 0, "time tile must split into per-thread runs");
};

template <class Cfg>
__device__ __forceinline__ void load_pw(floatx4 (&a)[Cfg::OB], const float* __restrict__ w_pw, int o_first, int O,
                                        int c, int C, bool vec) {
    // Weights of output rows o_first + ob*16 (clamped to O-1) and channels
    // c..c+3 (clamped to C-1).  Clamped entries multiply D = 0 or feed an
    // output that is not stored.
#pragma unroll
    for (int ob = 0; ob < Cfg::OB; ++ob) {
        const int o = min(o_first + ob * 16, O - 1);
        const float* row = w_pw + (size_t)o * C;
        if (vec) {
            a[ob] = *reinterpret_cast<const floatx4*>(row + min(c, C - 4));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) a[ob][j] = row[min(c + j, C - 1)];
        }
    }
}

template <class Cfg, bool VEC>
__global__ __launch_bounds__(Cfg::NT, Cfg::MINW) void dwsep_mfma_kernel(
    const float* __restrict__ x, const float* __restrict__ w_dw, const float* __restrict__ w_pw,
    const float* __restrict__ b_pw, float* __restrict__ y, int C, int T, int Kr, int O, int pad, int Tout) {
    constexpr int OB = Cfg::OB, TB = Cfg::TB, WO = Cfg::WO, CC = Cfg::CC, CCP = Cfg::CCP, TPT = Cfg::TPT;
    constexpr int TT = Cfg::TT, NT = Cfg::NT, NW = Cfg::NW;
    const int K = Cfg::KC > 0 ? Cfg::KC : Kr;

    extern __shared__ float lds[];
    float* Ds = lds;                    // [TT][CCP]
    float* wsm = lds + TT * CCP;        // [CC][K]
    float* xs = wsm + CC * K;           // [CC][XW]
    const int XW = TT + K - 1;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wo = wave % WO;
    const int wt = wave / WO;
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int t0 = blockIdx.x * TT;
    const int o0 = blockIdx.y * Cfg::OT + wo * 16 * OB;
    const int b = blockIdx.z;
    const float* xb = x + (size_t)b * C * T;
    const int NG = (C + 15) / 16;  // 16-channel groups

    floatx4 acc[OB][TB];
#pragma unroll
    for (int i = 0; i < OB; ++i)
#pragma unroll
        for (int j = 0; j < TB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    floatx4 a_next[OB];
    load_pw<Cfg>(a_next, w_pw, o0 + l16, O, 4 * g, C, VEC);

    for (int c0 = 0; c0 < C; c0 += CC) {
        __syncthreads();  // the previous chunk's LDS data is no longer read
        // 1. input chunk with halo, and the chunk's depthwise weights.  Loads
        //    are branch-free (clamped address, value selected to 0) and issued
        //    STAGE_U at a time so they overlap.
        {
            constexpr int STAGE_U = 8;
            const int nx = CC * XW;
            for (int base = 0; base < nx; base += NT * STAGE_U) {
                float v[STAGE_U];
#pragma unroll
                for (int u = 0; u < STAGE_U; ++u) {
                    const int i = base + u * NT + tid;
                    const int c = i / XW;
                    const int src = t0 - pad + (i - c * XW);
                    const bool ok = (i < nx) && (c0 + c < C) && (src >= 0) && (src < T);
                    const float val = xb[(size_t)(ok ? c0 + c : 0) * T + (ok ? src : 0)];
                    v[u] = ok ? val : 0.f;
                }
#pragma unroll
                for (int u = 0; u < STAGE_U; ++u) {
                    const int i = base + u * NT + tid;
                    if (i < nx) xs[i] = v[u];
                }
            }
            const int nw_valid = min(CC, C - c0) * K;
            for (int i = tid; i < CC * K; i += NT) {
                const float val = w_dw[(size_t)c0 * K + min(i, nw_valid - 1)];
                wsm[i] = i < nw_valid ? val : 0.f;
            }
        }
        __syncthreads();
        // 2. depthwise stage: 4 channels x TPT steps per thread
        for (int i = tid; i < (CC / 4) * (TT / TPT); i += NT) {
            const int tq = i % (TT / TPT);
            const int c4 = (i / (TT / TPT)) * 4;
            const int t = tq * TPT;
            float d[TPT][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float* xr = xs + (c4 + j) * XW + t;
                const float* wr = wsm + (c4 + j) * K;
                if constexpr (Cfg::KC > 0) {
                    float win[TPT + Cfg::KC - 1];
#pragma unroll
                    for (int u = 0; u < TPT + Cfg::KC - 1; ++u) win[u] = xr[u];
                    float wk[Cfg::KC];
#pragma unroll
                    for (int k = 0; k < Cfg::KC; ++k) wk[k] = wr[k];
#pragma unroll
                    for (int tt = 0; tt < TPT; ++tt) {
                        float s = 0.f;
#pragma unroll
                        for (int k = 0; k < Cfg::KC; ++k) s += wk[k] * win[tt + k];
                        d[tt][j] = s;
                    }
                } else {
#pragma unroll
                    for (int tt = 0; tt < TPT; ++tt) {
                        float s = 0.f;
                        for (int k = 0; k < K; ++k) s += wr[k] * xr[tt + k];
                        d[tt][j] = s;
                    }
                }
            }
#pragma unroll
            for (int tt = 0; tt < TPT; ++tt)
                *reinterpret_cast<floatx4*>(Ds + (t + tt) * CCP + c4) = floatx4{d[tt][0], d[tt][1], d[tt][2], d[tt][3]};
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
                if (grp + 1 < NG) load_pw<Cfg>(a_next, w_pw, o0 + l16, O, (grp + 1) * 16 + 4 * g, C, VEC);
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
    float* yb = y + (size_t)b * O * Tout;
#pragma unroll
    for (int ob = 0; ob < OB; ++ob)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = o0 + ob * 16 + 4 * g + r;
            if (o >= O) continue;
            const float bo = b_pw ? b_pw[o] : 0.f;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int t = t0 + (wt * TB + tb) * 16 + l16;
                if (t < Tout) yb[(size_t)o * Tout + t] = acc[ob][tb][r] + bo;
            }
        }
}

// Instances.  Wide (O > 64): 256 x 64 tile, 4 waves of 64 x 64, register
// budget for 3 waves per SIMD so three workgroups share a CU and one's load
// and depthwise phases overlap the others' matrix work.  Small: 32 x 32.
// FCONV_CFG_DW9 lets a build override the K = 9 instance's tiling.
#ifndef FCONV_CFG_DW9
#define FCONV_CFG_DW9 2, 4, 8, 1, 64, 2, 9, 4
#endif
using DwWide9 = DwsepCfg<FCONV_CFG_DW9>;
using DwWideK = DwsepCfg<4, 4, 4, 1, 64, 4, 0, 3>;
using DwSmallK = DwsepCfg<1, 1, 2, 2, 16, 2, 0, 2>;

template <class Cfg>
static size_t dw_lds_bytes(int K) {
    return ((size_t)Cfg::TT * Cfg::CCP + (size_t)Cfg::CC * K + (size_t)Cfg::CC * (Cfg::TT + K - 1)) *
           sizeof(float);
}

template <class Cfg>
static hipError_t launch_dw(const DwsepShape& s, const float* x, const float* w_dw, const float* w_pw,
                            const float* b_pw, float* y, hipStream_t stream) {
    const size_t lds = dw_lds_bytes<Cfg>(s.K);
    dim3 grid((s.Tout + Cfg::TT - 1) / Cfg::TT, (s.O + Cfg::OT - 1) / Cfg::OT, s.B);
    const bool vec = (s.C % 4 == 0) && ((uintptr_t)w_pw % 16 == 0);
    hipError_t e;
    if (vec) {
        e = hipFuncSetAttribute((const void*)dwsep_mfma_kernel<Cfg, true>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((dwsep_mfma_kernel<Cfg, true>), grid, dim3(Cfg::NT), lds, stream, x, w_dw, w_pw, b_pw,
                           y, s.C, s.T, s.K, s.O, s.pad, s.Tout);
    } else {
        e = hipFuncSetAttribute((const void*)dwsep_mfma_kernel<Cfg, false>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((dwsep_mfma_kernel<Cfg, false>), grid, dim3(Cfg::NT), lds, stream, x, w_dw, w_pw, b_pw,
                           y, s.C, s.T, s.K, s.O, s.pad, s.Tout);
    }
    return hipGetLastError();
}

bool dwsep_supported(int K, int O) {
    const size_t limit = 160 * 1024;
    if (O > 64) return dw_lds_bytes<DwWideK>(K) <= limit;
    return dw_lds_bytes<DwSmallK>(K) <= limit;
}

hipError_t dwsep_launch(const DwsepShape& s, const float* x, const float* w_dw, const float* w_pw,
                        const float* b_pw, float* y, hipStream_t stream) {
    if (s.O > 64)
        return s.K == 9 ? launch_dw<DwWide9>(s, x, w_dw, w_pw, b_pw, y, stream)
                        : launch_dw<DwWideK>(s, x, w_dw, w_pw, b_pw, y, stream);
    return launch_dw<DwSmallK>(s, x, w_dw, w_pw, b_pw, y, stream);
}

}  // namespace fconv
