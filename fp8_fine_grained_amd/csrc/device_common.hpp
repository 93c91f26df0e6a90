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
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T ld(const void* p) { return *reinterpret_cast<const T*>(p); }
// A load of data read exactly once (the quantizers' inputs), with the
// non-temporal hint: those lines then do not displace ones that are read
// again, such as the codes the GEMM reads next.
template <typename T>
__device__ __forceinline__ T ld_once(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

// Quantizer inputs: fp32, or bf16 carried as its 16-bit pattern (uint16_t).
// A bf16 value widens to fp32 exactly: its bits become the high half.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float f32_of(float v) { return v; }
__device__ __forceinline__ float f32_of(uint16_t b) { return __builtin_bit_cast(float, uint32_t(b) << 16); }
// 4 consecutive elements (16-byte or 8-byte aligned)
__device__ __forceinline__ v4f load4(const float* p) { return ld_once<v4f>(p); }
__device__ __forceinline__ v4f load4(const uint16_t* p) {
    const u32x2_t w = ld_once<u32x2_t>(p);
    return v4f{__builtin_bit_cast(float, w[0] << 16), __builtin_bit_cast(float, w[0] & 0xFFFF0000u),
               __builtin_bit_cast(float, w[1] << 16), __builtin_bit_cast(float, w[1] & 0xFFFF0000u)};
}
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

// Four E4M3 codes (RNE, saturating) of four floats, packed little-endian, by
// the hardware conversion.  v_cvt_pk_fp8_f32 was compared with e4m3_from_f32
// above on every 32-bit pattern whose value is finite with |y| <= 464 and
// agreed on all of them (signed zeros, subnormals, ties, saturation); the
// quantizers only ever convert |y| <= 448 * (1 + 2^-23).
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
    const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true));
}

// Codes of RN32(x / s) for four elements of one group, bit for bit, with
// r = RN32(1 / s) computed once per group (r is +inf only when s is
// subnormal enough for 1/s to overflow; s == 0 only for an all-zero group).
//
// y' = RN32(x * r) differs from x / s by less than 2^-23 |y'|, and RN32(x / s)
// lies within half an ulp of x / s, so both lie inside
// [y' - 2^-21 |y'|, y' + 2^-21 |y'|] (the bracket ends' own rounding costs less
// than an ulp of the 4 ulps of margin).  Rounding to E4M3 is monotone, so when
// both ends of the bracket give the same code every value inside -- RN32(x/s)
// included -- has that code.  Otherwise (the bracket straddles a rounding
// boundary: about 2^-16 of elements) the IEEE quotient is computed.
__device__ __forceinline__ uint32_t encode4(v4f x, float s, float r) {
    if (s == 0.0f) return cvt4(x[0], x[1], x[2], x[3]);       // signed zeros
    if (r < __builtin_inff()) {
        const v4f y = x * r;
        constexpr float e = 0x1p-21f;
        const uint32_t lo = cvt4(__builtin_fmaf(-__builtin_fabsf(y[0]), e, y[0]), __builtin_fmaf(-__builtin_fabsf(y[1]), e, y[1]),
                                 __builtin_fmaf(-__builtin_fabsf(y[2]), e, y[2]), __builtin_fmaf(-__builtin_fabsf(y[3]), e, y[3]));
        const uint32_t hi = cvt4(__builtin_fmaf(__builtin_fabsf(y[0]), e, y[0]), __builtin_fmaf(__builtin_fabsf(y[1]), e, y[1]),
                                 __builtin_fmaf(__builtin_fabsf(y[2]), e, y[2]), __builtin_fmaf(__builtin_fabsf(y[3]), e, y[3]));
        if (lo == hi) return lo;
    }
    return cvt4(x[0] / s, x[1] / s, x[2] / s, x[3] / s);
}

}  // namespace fp8fg
