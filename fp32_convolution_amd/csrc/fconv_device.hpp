// fconv_device.hpp -- device helpers shared by the libfconv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fconv {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// One fp32 matrix-core step: D(16x16) = A(16x4) * B(4x16) + C, all fp32
// (v_mfma_f32_16x16x4_f32).  Operand layout per lane l of the wave:
//   A: row l%16, k-index l/16        B: k-index l/16, column l%16
//   C/D element r (0..3): row 4*(l/16) + r, column l%16
__device__ __forceinline__ floatx4 mfma_16x16x4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Raw buffer loads.  A buffer resource covers [base, base + bytes); a load
// whose byte offset is at or beyond `bytes` returns 0 without touching
// memory, so zero padding and masking need no branch.  Offsets are unsigned
// 32-bit; kBufOOB is past the end of every resource the library builds
// (each covers < 2^31 bytes).  0x00020000 is the gfx9-family descriptor word
// for 32-bit data.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
constexpr int kBufOOB = (int)0x80000000u;

__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ float buf_load_f32(buf_rsrc r, int byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
}

// A lane's running sum of sigmoids across the units of work a workgroup
// walks: fp64 when it walks several (its rounding then stays far below the
// fp32 rounding of the final sums), fp32 for a single unit.
template <bool WALK>
using walk_sum_t = typename std::conditional<WALK, double, float>::type;

// Sum over the 64 lanes, valid in every lane; the order is fixed.  Within
// each row of 16 lanes with DPP (pairs, quads, half-row mirror, row mirror:
// every lane then holds its row's sum), then the four row sums read out of
// lanes 0, 16, 32, 48.  Needs all 64 lanes active.
__device__ __forceinline__ float wave_sum(float v) {
    auto dpp = [](float x, auto ctrl) {
        return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                     decltype(ctrl)::value, 0xF, 0xF, false));
    };
    v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm 1,0,3,2
    v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm 2,3,0,1
    v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
    v += dpp(v, std::integral_constant<int, 0x140>{});  // row_mirror
    auto lane = [](float x, int l) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
    };
    return (lane(v, 0) + lane(v, 16)) + (lane(v, 32) + lane(v, 48));
}

// Sums v over the workgroup; the result is valid in thread 0 only.
template <int NWAVES>
__device__ __forceinline__ float block_sum(float v, float* red /* NWAVES floats of LDS */) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = 0.f;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int i = 0; i < NWAVES; ++i) s += red[i];
    }
    return s;
}

// DPP quad permutations: lane l reads lane l^1 (quad_perm 1,0,3,2) or lane
// l^2 (quad_perm 2,3,0,1) of its aligned group of 4 lanes.  Every lane has a
// valid source, so the move needs no old value and can fuse into the
// instruction that uses it.
__device__ __forceinline__ float quad_xor1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
}

// DPP row shifts: lane l reads lane l-1 (row_shr:1) or l-2 (row_shr:2) of its
// row of 16 lanes; the first one or two lanes of each row read 0.
__device__ __forceinline__ float row_shr1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x111, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_shr2(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x112, 0xF, 0xF, true));
}

// DPP wave shift: lane l reads lane l+1 of the wave (wave_shl:1); lane 63
// reads 0 through the bound control, so the move needs no zeroed old value.
__device__ __forceinline__ float wave_shl1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x130, 0xF, 0xF, true));
}

// Logistic sigmoid 1/(1+e^-a) with the hardware exp2 (v_exp_f32) and
// reciprocal: relative error a few ulp for |a| < 80, exactly 1/2 at a = 0,
// saturating to 0 or 1 (never NaN) for large |a|.
__device__ __forceinline__ float logistic(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// logistic(a * scale), the scale (an average pool's 1/s^2) joined to the
// exponent's constant -log2(e): one multiply instead of two.  For a
// power-of-two scale the product rounds exactly as (a * scale) * -log2(e)
// does; otherwise it may differ in the last bit of the exponent's argument.
__device__ __forceinline__ float logistic_scaled(float a, float scale) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * (scale * -1.44269504f)));
}

// An LDS address the compiler cannot relate to others.  Reads off one base
// pair into ds_read2 instructions with 8-bit dword offsets; for rows past
// that reach the compiler otherwise derives a new base register for every
// pair.  A second base made opaque here keeps those rows on one register.
typedef __attribute__((address_space(3))) float* lds_fptr;
__device__ __forceinline__ lds_fptr lds_opaque(lds_fptr p) {
    asm("" : "+v"(p));
    return p;
}

// Block order for 8 XCDs.  The hardware deals consecutive block ids to the
// XCDs round-robin; this maps a block id to a logical tile id so that each
// XCD gets one contiguous run of tiles (neighbouring tiles then share that
// XCD's L2).  A bijection on [0, n).
__device__ __forceinline__ int xcd_spread(int bid, int n) {
    // Inverse of the round-robin deal of block ids to 8 XCDs: XCD k's blocks
    // (bid % 8 == k) get the k-th contiguous share of the logical ids.
    const int per = n / 8, rem = n % 8;
    const int xcd = bid % 8, idx = bid / 8;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

}  // namespace fconv
