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

// E4M3 code of v, |v| <= 448, round to nearest even.  Sign from the IEEE sign bit
// (so -0.0 and negatives that round to zero give 0x80).
//   |v| >= 2^-6 : normal code; round the float32 mantissa to 3 bits on the bit
//                 pattern (carry into the exponent is correct), then rebias 127 -> 7.
//   |v| <  2^-6 : subnormal code = |v| / 2^-9 rounded to an integer; 8 becomes the
//                 smallest normal 0x08, which is again the right code.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
    uint32_t b = __float_as_uint(v);
    uint32_t sign = (b >> 24) & 0x80u;
    uint32_t a = b & 0x7FFFFFFFu;
    uint32_t normal = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
    uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    return (a >= 0x3C800000u ? normal : sub) | sign;
}

// Quantize one value by its group scale s > 0: fl32(x / s) (IEEE division), clamp
// to +-448, encode.
__device__ __forceinline__ uint32_t quant_one(float x, float s) {
    float v = x / s;
    v = fminf(fmaxf(v, -kE4M3Max), kE4M3Max);
    return e4m3_rne(v);
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

// Max over the 16 lanes of a DPP row; every lane of the row gets the result.
// Max is exact and order-independent, so the result is bit-exact.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
    return v;
}

// Max over a full wave of 64 lanes.
__device__ __forceinline__ float wave_max(float v) {
    v = row16_max(v);
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

}  // namespace fp8bs
