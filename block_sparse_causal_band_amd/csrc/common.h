// common.h -- small device helpers shared by the HIP kernels of libswa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// in hardware, so tails need no branches.  Word 3 is the gfx9-family raw
// (untyped, 32-bit data format) descriptor setting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// 16-byte load at byte offset voff (checked against the resource size).
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}

// 16-byte streaming load (non-temporal: the data is read once).
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}

constexpr float kNegInf = -__builtin_huge_valf();
constexpr double kLog2e = 1.4426950408889634074;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Lane l <-> lane l^32 exchange of one 32-bit value, combined with op.
// v_permlane32_swap swaps the upper half of the first operand with the lower
// half of the second; feeding x twice gives {x[l], x[l^32]} in some order on
// every lane, which is all a symmetric reduction needs.
__device__ __forceinline__ float half_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace swa
