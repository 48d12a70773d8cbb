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

}  // namespace

extern "C" {

int fconv_probe_mfma_f32(int blocks, int iters, float* out, void* stream) {
    if (blocks < 1 || iters < 1 || !out) return -1;
    hipLaunchKernelGGL(mfma_f32_rate_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

int fconv_probe_fma_f32(int blocks, int iters, float* out, void* stream) {
    if (blocks < 1 || iters < 1 || !out) return -1;
    hipLaunchKernelGGL(fma_f32_rate_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
