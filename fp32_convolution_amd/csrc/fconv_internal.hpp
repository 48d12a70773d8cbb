// fconv_internal.hpp -- host-side interfaces between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fconv {

// Shapes after validation; every per-batch-item element count fits in int32.
struct Conv2dShape {
    int B, Cin, H, W, Cout, K, S, PH, PW;
};

struct DwsepShape {
    int B, C, T, K, O, pad, Tout;
};

// Returns true (and fills lds_bytes) if the MFMA direct-conv kernel has an
// instance for (K, S) and its LDS tile for Cin channels fits one workgroup.
bool conv2d_mfma_supported(int Cin, int K, int S, size_t* lds_bytes);

// Enqueue kernels; return hipSuccess or the launch error.  `map` selects the
// pooled-map output (pooled[B,Cout,PH,PW]) instead of the fused sum (out[B]).
hipError_t conv2d_mfma_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                              float* dst, bool map, hipStream_t stream);
// Box-sum variant: true if it has an instance for (K, S) and its LDS fits.
bool conv2d_boxsum_supported(int Cin, int K, int S);
hipError_t conv2d_boxsum_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                                float* dst, bool map, hipStream_t stream);
hipError_t conv2d_simple_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                                float* dst, bool map, hipStream_t stream);
hipError_t fill_zero(float* p, int64_t n, hipStream_t stream);

// True if the fused depthwise-separable kernel's LDS tile fits for this K.
bool dwsep_supported(int K, int O);
hipError_t dwsep_launch(const DwsepShape& s, const float* x, const float* w_dw, const float* w_pw,
                        const float* b_pw, float* y, hipStream_t stream);

}  // namespace fconv
