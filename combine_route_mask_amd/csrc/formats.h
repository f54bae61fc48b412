// Number-format helpers of the gfx950 kernels: bf16 rounding, OCP e4m3fn
// and e8m0 block scales.  Integer bit manipulation only, so every result
// is exact and independent of the floating-point mode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_ep {

__device__ __forceinline__ float bf16_to_f32(uint32_t b16)
{
    return __uint_as_float(b16 << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return ((u >> 16) & 0x8000u) | 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two packed bf16 (low half = first element) -> two floats.
__device__ __forceinline__ void unpack_bf16x2(uint32_t w, float &lo, float &hi)
{
    lo = __uint_as_float(w << 16);
    hi = __uint_as_float(w & 0xFFFF0000u);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Exponent e of the block scale 2^e for a block whose largest magnitude
// has bf16 bit pattern amax_bits (sign cleared, finite): the smallest e
// with amax <= 448 * 2^e, clamped to [-127, 127].  448 = 1.75 * 2^8, so
// for amax = 1.m * 2^E the answer is E - 8, or E - 7 when 1.m > 1.75.
__device__ __forceinline__ int fp8_block_exponent(uint32_t amax_bits)
{
    if (amax_bits == 0)
        return -127;
    const int eb = (int)(amax_bits >> 7);   // biased exponent
    const uint32_t mant = amax_bits & 0x7Fu; // 7 mantissa bits
    if (eb == 0)                            // subnormal bf16: far below 448 * 2^-127
        return -127;
    int e = eb - 127 - 8 + (mant > 0x60u ? 1 : 0); // 0x60/128 = 0.75
    return e < -127 ? -127 : e;
}

// e4m3fn code of an fp32 value with |v| <= 448 (round to nearest even).
// Values below half the smallest subnormal (2^-10) round to zero.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v)
{
    uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    u &= 0x7FFFFFFFu;
    if (u < 0x3C800000u) {                   // |v| < 2^-6: subnormal grid 2^-9
        // |v| * 2^9 is exact; rint rounds half to even
        const float m = __builtin_rintf(__uint_as_float(u) * 512.0f);
        return sign | (uint32_t)m;           // m == 8 encodes 2^-6 exactly
    }
    // keep exponent and 3 mantissa bits, rounding the 20 dropped bits to even
    const uint32_t r = (u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));         // rebias 127 -> 7
}

// e4m3fn code -> fp32 (exact).  0x7F / 0xFF are NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c)
{
    const uint32_t sign = (c & 0x80u) << 24;
    const uint32_t em = c & 0x7Fu;
    if (em == 0x7Fu)
        return __uint_as_float(0x7FC00000u | sign);
    if (em < 8u)                             // subnormal: m * 2^-9
        return __uint_as_float(sign | __float_as_uint((float)em * (1.0f / 512.0f)));
    return __uint_as_float(sign | ((em + (120u << 3)) << 20));
}

} // namespace moe_ep
