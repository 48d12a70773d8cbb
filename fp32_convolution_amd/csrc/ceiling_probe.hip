// ceiling_probe.hip -- measured ceilings of the GPU, for the benchmark only
// (libfconv_probe.so; not part of the fused-convolution ABI).
//
// The fp32 peaks a datasheet quotes (157.3 TFLOP/s on the matrix cores,
// 78.6 TFLOP/s for non-packed vector FMA on MI355X) assume every SIMD issues
// one instruction of the kind every cycle at the boost clock.  These kernels
// measure what the part sustains for exactly that: each wave runs eight
// independent dependency chains of one instruction, operands in registers,
// no memory traffic, so the rate they reach is the practical ceiling a
// kernel bound by that unit can be compared with.
//   fconv_probe_mfma_f32: v_mfma_f32_16x16x4_f32, 2*16*16*4 = 2048 FLOP per
//     wave-instruction;
//   fconv_probe_fma_f32: v_fma_f32, 2*64 = 128 FLOP per wave-instruction.
// Both launch `blocks` workgroups of 256 threads (4 waves: one per SIMD of a
// CU), each running `iters` iterations of 8 instructions, and write one float
// per thread to out[blocks*256] so that no chain is dead code.  Inline
// assembly pins the instruction (the compiler may neither fuse, pack nor
// reorder the chains into something else).  Return 0 or -3 (launch error).
//
// Whether vector and matrix work overlap on one SIMD:
//   fconv_probe_mfma_valu_f32: one 512-thread workgroup per CU (8 waves, two
//     per SIMD, held to one workgroup per CU by 96 KB of LDS); with mode bit 0
//     waves 0-3 run `iters_m` iterations of the MFMA chains above, with bit 1
//     waves 4-7 run `iters_v` iterations of the FMA chains.  Timing modes 1,
//     2 and 3 tells whether a SIMD issues the second wave's v_fma_f32 while
//     the first wave's matrix instructions execute (mode 3 as long as the
//     longer of 1 and 2) or in turn with them (as long as their sum).
// HBM streaming rates, for kernels that only read (the box-sum Conv2d) or
// mostly write (the depthwise-separable Conv1d's output):
//   fconv_probe_read_f32: `blocks` workgroups of 256 threads read n4 16-byte
//     words of `in` (grid-stride, coalesced) and write one sum per thread to
//     out[blocks*256];
//   fconv_probe_write_f32: the same grid writes n4 16-byte words to `dst`.
#include <hip/hip_runtime.h>

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_f32_rate_kernel(float* __restrict__ out, int iters) {
    const float a = (float)threadIdx.x * 1e-3f, b = 1.0f + (float)threadIdx.x * 1e-6f;
    floatx4 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+v"(c[j]) : "v"(a), "v"(b));
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += c[j][j & 3];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void fma_f32_rate_kernel(float* __restrict__ out, int iters) {
    const float a = 1.0f - (float)threadIdx.x * 1e-7f, b = (float)threadIdx.x * 1e-6f;
    float c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = (float)j;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(c[j]) : "v"(a), "v"(b));
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += c[j];
    out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(512) void mfma_valu_kernel(float* __restrict__ out, int mode, int iters_m, int iters_v) {
    extern __shared__ float hold[];  // only reserves LDS: one workgroup per CU
    float s = 0.f;
    if (threadIdx.x < 256) {
        if (mode & 1) {
            const float a = (float)threadIdx.x * 1e-3f, b = 1.0f + (float)threadIdx.x * 1e-6f;
            floatx4 c[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) c[j] = floatx4{0.f, 0.f, 0.f, 0.f};
            for (int i = 0; i < iters_m; ++i) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    asm volatile("v_mfma_f32_16x16x4_f32 %0, %1, %2, %0" : "+v"(c[j]) : "v"(a), "v"(b));
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) s += c[j][j & 3];
        }
    } else if (mode & 2) {
        const float a = 1.0f - (float)threadIdx.x * 1e-7f, b = (float)threadIdx.x * 1e-6f;
        float c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = (float)j;
        for (int i = 0; i < iters_v; ++i) {
#pragma unroll
            for (int j = 0; j < 8; ++j) asm volatile("v_fma_f32 %0, %1, %2, %0" : "+v"(c[j]) : "v"(a), "v"(b));
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) s += c[j];
    }
    out[blockIdx.x * 512 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void read_f32_rate_kernel(const float4* __restrict__ in, long n4,
                                                             float* __restrict__ out) {
    const long stride = (long)gridDim.x * 256;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const float4 v = in[i];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    out[blockIdx.x * 256 + threadIdx.x] = (acc.x + acc.y) + (acc.z + acc.w);
}

__global__ __launch_bounds__(256) void write_f32_rate_kernel(float4* __restrict__ dst, long n4, float v) {
    const long stride = (long)gridDim.x * 256;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) dst[i] = make_float4(v, v, v, v);
}

}  // namespace

extern "C" {

int fconv_probe_read_f32(int blocks, long n4, const float* in, float* out, void* stream) {
    if (blocks < 1 || n4 < 1 || !in || !out) return -1;
    hipLaunchKernelGGL(read_f32_rate_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const float4*)in, n4,
                       out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

int fconv_probe_write_f32(int blocks, long n4, float* dst, void* stream) {
    if (blocks < 1 || n4 < 1 || !dst) return -1;
    hipLaunchKernelGGL(write_f32_rate_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (float4*)dst, n4,
                       1.0f);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

int fconv_probe_mfma_f32(int blocks, int iters, float* out, void* stream) {
    if (blocks < 1 || iters < 1 || !out) return -1;
    hipLaunchKernelGGL(mfma_f32_rate_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// out holds blocks*512 floats; blocks is the CU count (one workgroup each)
int fconv_probe_mfma_valu_f32(int blocks, int mode, int iters_m, int iters_v, float* out, void* stream) {
    if (blocks < 1 || mode < 1 || mode > 3 || iters_m < 1 || iters_v < 1 || !out) return -1;
    constexpr int kHold = 96 * 1024;
    if (hipFuncSetAttribute((const void*)mfma_valu_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kHold) !=
        hipSuccess)
        return -3;
    hipLaunchKernelGGL(mfma_valu_kernel, dim3(blocks), dim3(512), kHold, (hipStream_t)stream, out, mode, iters_m,
                       iters_v);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

int fconv_probe_fma_f32(int blocks, int iters, float* out, void* stream) {
    if (blocks < 1 || iters < 1 || !out) return -1;
    hipLaunchKernelGGL(fma_f32_rate_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
