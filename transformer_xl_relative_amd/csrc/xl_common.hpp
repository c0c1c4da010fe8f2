// xl_common.hpp -- shared device types and helpers of libxlrel (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xl {

typedef uint16_t bf16_t;  // storage type of bfloat16 values
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- scalar conversions ---------------------------------------------------

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// float -> bfloat16, round to nearest even (finite inputs)
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// two floats -> packed bfloat16 pair (lo in bits 0-15), round to nearest even
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
    return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// double -> bfloat16 with a single rounding: round-to-odd to float first
// (keeps the sticky information), then nearest-even to bfloat16.
__device__ __forceinline__ bf16_t d2bf(double x) {
    float t = __double2float_rz(x);
    uint32_t u = __float_as_uint(t);
    if ((double)t != x) u |= 1u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// ---- element traits -------------------------------------------------------

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr bool kBf16 = false;
    __device__ static float to_f(float v) { return v; }
};
template <> struct Elem<bf16_t> {
    static constexpr bool kBf16 = true;
    __device__ static float to_f(bf16_t v) { return bf2f(v); }
};

// ---- MFMA wrappers ----------------------------------------------------------
// 32x32 output tile, lane l holds column (l % 32) and rows
// 8*(r/4) + 4*(l/32) + (r%4) in accumulator register r (0..15).
// bf16: K = 16 per instruction; lane holds 8 consecutive k at 8*(l/32).
// f32:  K = 2 per instruction; lane holds k = l/32.

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace xl
