// Device helpers shared by the gfx950 kernels of libfp8bs.
//
// Formats: BF16 is the upper half of an IEEE float32; E4M3 is OCP OFP8 E4M3
// ("e4m3fn": bias 7, 3 mantissa bits, subnormals m * 2^-9, largest finite 448,
// no infinity), the code format the "Nanbeige4.3-33B FP8" model card names for
// weights and activations (introduction).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;          // activation group / weight block edge
constexpr float kE4M3Max = 448.0f;   // largest finite E4M3 magnitude (code 0x7E)

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float32 -> BF16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// float64 -> BF16 bits, rounded once to nearest even (finite, |d| < 2^128).
// Normal BF16 range: round the 52-bit mantissa to 7 bits on the bit pattern; a
// carry into the exponent is the correct result.  Below 2^-126 the BF16 quantum
// is 2^-133: scale by 2^133 (exact) and round to an integer (v_rndne_f64).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
    uint64_t b = (uint64_t)__double_as_longlong(d);
    uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
    uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
    uint32_t mag;
    if (a >= 0x3810000000000000ull) {                  // |d| >= 2^-126
        uint64_t r = (a + 0x00000FFFFFFFFFFFull + ((a >> 45) & 1ull)) >> 45;
        mag = (uint32_t)(r - ((uint64_t)(1023 - 127) << 7));
    } else {
        mag = (uint32_t)__builtin_rint(__longlong_as_double((long long)a) * 0x1p133);
    }
    return sign | mag;
}

// fl32(x / s) (IEEE division) clamped to +-448: the value a group's code encodes.
__device__ __forceinline__ float quant_value(float x, float s) {
    const float v = x / s;
    return fminf(fmaxf(v, -kE4M3Max), kE4M3Max);
}

// Smallest group scale taken by quant_value_fast.
constexpr float kFastDivMinScale = 0x1p-60f;

// The same value as quant_value for s >= 2^-60, from y = fl32(1 / s) (one IEEE
// division per group) and two correction steps with fused multiply-adds:
//   q = fl32(|x| y);  then twice  r = fma(-q, s, |x|),  q = fma(r, y, q).
// fl32(|x| y) is within 1.5 ulp of |x| / s; a correction step with the exactly
// computed remainder r brings a quotient within 1.5 ulp to within 1 ulp, and from
// within 1 ulp (with y the correctly rounded reciprocal) to the correctly rounded
// quotient (Markstein's theorem on FMA division).  For s >= 2^-60 no step
// underflows while |x| / s >= 2^-11; below that every code is zero anyway.  The
// sign is taken from x at the end, so -0.0 stays -0.0.
__device__ __forceinline__ float quant_value_fast(float x, float s, float y) {
    const float a = fabsf(x);
    float q = a * y;
    float r = fmaf(-q, s, a);
    q = fmaf(r, y, q);
    r = fmaf(-q, s, a);
    q = fmaf(r, y, q);
    return copysignf(fminf(q, kE4M3Max), x);
}

// E4M3 codes of four values with |v| <= 448, packed little-endian: gfx950's
// v_cvt_pk_fp8_f32 converts to OCP E4M3 (bias 7) with round to nearest even,
// subnormal codes included, and takes the sign from the IEEE sign bit (-0.0 and
// negatives that round to zero give 0x80).  Two values per instruction.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// DPP lane moves within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i within each 16 lanes

// Max over the 16 lanes of a DPP row of non-negative values (group amaxes); every
// lane of the row gets the result.  Non-negative floats order as their bit
// patterns, so the max is taken on the integers: exact, order-independent, and
// without the NaN canonicalization a float max would add per step.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float row16_max(float v) {
    uint32_t u = __float_as_uint(v);
    u = max(u, dpp_u32<kDppQuadXor1>(u));
    u = max(u, dpp_u32<kDppQuadXor2>(u));
    u = max(u, dpp_u32<kDppRowHalfMirror>(u));
    u = max(u, dpp_u32<kDppRowMirror>(u));
    return __uint_as_float(u);
}

// Max over a full wave of 64 lanes (non-negative values).
__device__ __forceinline__ float wave_max(float v) {
    uint32_t u = __float_as_uint(row16_max(v));
    u = max(u, (uint32_t)__shfl_xor((int)u, 16));
    u = max(u, (uint32_t)__shfl_xor((int)u, 32));
    return __uint_as_float(u);
}

}  // namespace fp8bs
