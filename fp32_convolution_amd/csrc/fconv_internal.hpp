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
    int B, C, T, K, O, pad, Tout, stride, dil;
};

// Workgroups per batch item of a Conv2d launch.  A fused sum writes one fp32
// partial per workgroup and reduce_partials adds an item's partials in a
// fixed order: each thread adds at most 4 of them (1024 / 256) in sequence,
// then a 256-thread tree adds the threads' sums, so no chain of additions is
// longer than 12.  Every partial is positive (a sum of sigmoids), so each
// addition rounds by at most 2^-24 of the final out[b], and the reduction by
// at most 12 * 2^-24 = 7.2e-7 |out[b]|, whatever the map size.  A map with
// more units of work (tiles x output-channel ranges) than kMaxPartsPerItem
// has each workgroup walk several units, part, part + parts, ..., summing its
// lanes' sigmoids in fp64 between units.
#ifndef FCONV_MAX_PARTS_PER_ITEM
#define FCONV_MAX_PARTS_PER_ITEM 1024
#endif
constexpr int kMaxPartsPerItem = FCONV_MAX_PARTS_PER_ITEM;
inline int walk_parts(int64_t units) { return units < kMaxPartsPerItem ? (int)units : kMaxPartsPerItem; }

// What a Conv2d kernel writes: the pre-sigmoid pooled map, or one partial
// sum per workgroup into ws[b * parts_per_item + part], which
// reduce_partials then adds in a fixed order into out[b].
// parts_per_item = walk_parts(units per item).
enum OutMode { OUT_MAP = 1, OUT_PARTIAL = 2 };

// The generalised pool: max instead of mean, a ReLU between the conv and the
// pool, PyTorch's ceil output size (partial windows at the bottom/right).
struct PoolOpts {
    bool pool_max, relu, ceil_mode;
};

// Returns true if the MFMA direct-conv path has an instance for (K, S) and
// its LDS tile for Cin channels fits one workgroup.
bool conv2d_mfma_supported(int Cin, int K, int S);

// Enqueue kernels; return hipSuccess or the launch error.  `mode` is an
// OutMode; dst is out[B], pooled[B,Cout,PH,PW] or ws[B * parts_per_item].
hipError_t conv2d_mfma_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                              float* dst, int mode, hipStream_t stream);
// Box-sum variant: true if it has an instance for (K, S) and its LDS fits.
bool conv2d_boxsum_supported(int Cin, int K, int S);
hipError_t conv2d_boxsum_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                                float* dst, int mode, hipStream_t stream);
hipError_t conv2d_simple_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                                float* dst, int mode, hipStream_t stream);
// Workgroups (= partial sums) per batch item of each algorithm's launch.
int64_t conv2d_mfma_parts(const Conv2dShape& s);
int64_t conv2d_boxsum_parts(const Conv2dShape& s);
int64_t conv2d_simple_parts(const Conv2dShape& s);
// Generalised-pool kernels (conv2d_pool_ex.hip).  `s.PH`, `s.PW` are the
// pooled sizes under o.ceil_mode.  The matrix-core kernel has instances for
// K = 3 with s = 2, 3, 4 and K = 5 with s = 3, any Cin (channel-chunked past
// its whole-tile LDS budget); the general kernel takes any shape.
bool conv2d_elem_supported(int Cin, int K, int S);
int64_t conv2d_elem_parts(const Conv2dShape& s, const PoolOpts& o);
int64_t conv2d_general_parts(const Conv2dShape& s);
hipError_t conv2d_elem_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias, float* dst,
                              int mode, const PoolOpts& o, hipStream_t stream);
hipError_t conv2d_general_launch(const Conv2dShape& s, const float* x, const float* w, const float* bias,
                                 float* dst, int mode, const PoolOpts& o, hipStream_t stream);
// out[b] = sum of ws[b*parts .. b*parts+parts-1], in a fixed order.
hipError_t reduce_partials(const float* ws, int64_t parts, int B, float* out, hipStream_t stream);
hipError_t fill_zero(float* p, int64_t n, hipStream_t stream);

// True if a fused depthwise-separable instance's LDS tile fits this shape.
bool dwsep_supported(const DwsepShape& s);
hipError_t dwsep_launch(const DwsepShape& s, const float* x, const float* w_dw, const float* w_pw,
                        const float* b_pw, float* y, hipStream_t stream);
// The dense-fused (combined 9-tap weight) variant.
bool dwsep_dense_supported(const DwsepShape& s);
hipError_t dwsep_dense_launch(const DwsepShape& s, const float* x, const float* w_dw, const float* w_pw,
                              const float* b_pw, float* y, hipStream_t stream);

}  // namespace fconv
