// Number-format helpers of the gfx950 kernels: bf16 rounding and the e8m0
// block-scale exponent of the FP8 (OCP e4m3fn) combine payload.  Integer
// bit manipulation only, so every result is exact and independent of the
// floating-point mode.  The e4m3 codes themselves come from the hardware
// conversions (v_cvt_pk_fp8_f32 / v_cvt_pk_f32_fp8, round to nearest even).
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

} // namespace moe_ep
