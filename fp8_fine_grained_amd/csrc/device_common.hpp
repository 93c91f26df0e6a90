// Device-side helpers shared by the quantizer and GEMM kernels (gfx950).
//
// Number formats: E4M3 (4 exponent, 3 mantissa bits) as in the DeepGEMM launch
// article, section "O que e FP8?"; the OCP "FN" flavour (bias 7, max 448, no
// infinities) with round-to-nearest-even and saturation.  BF16 output rounds
// the FP32 accumulator to nearest-even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8fg {

// Native clang vector types: arrays of these stay in registers, unlike arrays
// of HIP's struct-based uint4/float4.
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T ld(const void* p) { return *reinterpret_cast<const T*>(p); }
template <typename T>
__device__ __forceinline__ void st(void* p, T v) { *reinterpret_cast<T*>(p) = v; }

constexpr int kBlock = 128;          // quantization group length and GEMM K-block

// fp32 -> E4M3 code, round to nearest even, saturating at +-448.
// Works on the fp32 bit pattern: the sign is copied, magnitudes >= 448 clamp
// to 0x7E; magnitudes below 2^-6 (E4M3's smallest normal) sit on the
// subnormal grid of step 2^-9, so |y| * 2^9 (exact: a power-of-two scaling)
// rounded to an integer is the code; everything else keeps the top three
// mantissa bits, rounded by adding (half - 1) plus the lowest kept bit, with
// the carry running into the exponent, then rebiased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_from_f32(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t code;
    if (a >= 0x43e00000u) {                       // >= 448
        code = 0x7eu;
    } else if (a < 0x3c800000u) {                 // < 2^-6
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    } else {
        const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
        code = (r >> 20) - (120u << 3);
    }
    return sign | code;
}

// Four codes packed little-endian into one 32-bit word.
__device__ __forceinline__ uint32_t pack4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
    return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Max over the 32 lanes of each half-wave (lanes 0-31 and 32-63 reduce separately).
__device__ __forceinline__ float halfwave_max(float v) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ float abs_max4(v4f v) {
    return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}

// Codes of x / s for a group with scale s (s == 0 only for an all-zero group,
// whose elements are signed zeros and encode as such).
__device__ __forceinline__ uint32_t encode4(v4f v, float s) {
    if (s == 0.0f) {
        return pack4(e4m3_from_f32(v[0]), e4m3_from_f32(v[1]), e4m3_from_f32(v[2]), e4m3_from_f32(v[3]));
    }
    return pack4(e4m3_from_f32(v[0] / s), e4m3_from_f32(v[1] / s),
                 e4m3_from_f32(v[2] / s), e4m3_from_f32(v[3] / s));
}

}  // namespace fp8fg
