// Storage encodings shared by the kernels: bfloat16 and E4M3 (OCP e4m3fn,
// the NVFP4 block-scale byte).  Device-side only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hr {

// float32 -> bfloat16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf2f(uint32_t h) { return __uint_as_float(h << 16); }

// E4M3 byte of d >= 0: nearest, ties to the even mantissa, saturating at
// 448.  From 2^-6 up, rounding the float32 pattern at mantissa bit 20 leaves
// (biased exponent << 3 | three mantissa bits), and the byte is that less
// (127 - 7) << 3; below 2^-6 the byte counts units of 2^-9.
__device__ __forceinline__ uint32_t e4m3_byte(float d) {
    d = fminf(d, 448.0f);
    const uint32_t u = __float_as_uint(d);
    if (u >= 0x3C800000u) return ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - 960u;
    return static_cast<uint32_t>(rintf(d * 512.0f));
}

// value of an E4M3 byte below 0x7F (non-negative, finite)
__device__ __forceinline__ float e4m3_value(uint32_t b) {
    return (b >> 3) ? __uint_as_float((b + 960u) << 20) : static_cast<float>(b) * 0.001953125f;
}

}  // namespace hr
