// Quantization kernels for gfx950:
//   quant_act_kernel       dynamic per-token, group-128 activation quantization
//   silu_mul_quant_kernel  h = BF16(silu(gate) * up), rounded once, then the same quantization
//   quant_weight_kernel    128x128 block weight quantization (offline step)
//   rmsnorm_quant_kernel   h = BF16(RMSNorm(x) * gamma), rounded once, then the same quantization
//
// Scheme: "Nanbeige4.3-33B FP8" model card, introduction and "Recipe and
// calibration" (E4M3 weights in 128x128 blocks, minmax scales; dynamic per-token
// group-128 activation scales).  Scale = fl32(amax / 448); code = E4M3 of
// fl32(x / scale), nearest even, saturated at 448; an all-zero group has scale +0
// and codes 0x00.
//
// Activation layout: K is a multiple of 128, so the groups of [M, K] row-major
// data are consecutive 256-byte runs and group g's scale sits at s[g] of the
// row-major [M, K/128] scale tensor: the activation quantizer is a flat loop over
// groups.  One group is handled by one 16-lane DPP row: each lane loads 8 BF16
// (16 bytes), the group amax is a 4-step DPP max, and each lane stores 8 codes.
#include "device_common.h"
#include "launch.h"

namespace fp8bs {

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kQuantThreads = 256;           // 16 groups per block pass
// Groups per 16-lane row: 4 for large inputs (more loads in flight per lane), 1
// when the input is too small to fill the GPU otherwise.
constexpr int kQuantUnrollBig = 4;
constexpr int64_t kSmallGroups = 16 * 4 * 1024;
// The SiLU kernel holds more registers per group (its float64 recomputation path), so
// it takes 2 groups per row pass: measured 23.7 against 26.3 us (4 groups) at
// M = 2048, I = 8192, and 94.6 against 96.5 us at M = 8191.
constexpr int kSiluUnrollBig = 2;

__device__ __forceinline__ void unpack8(const uint4& v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

// Codes of 8 values of one group (scale s, already reduced over the group).
__device__ __forceinline__ uint2 quant8(const float (&x)[8], float s) {
    uint2 out = {0u, 0u};
    float v[8];
    if (s >= kFastDivMinScale) {
        const float y = 1.0f / s;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = quant_value_fast(x[i], s, y);
    } else if (s != 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = quant_value(x[i], s);
    } else {
        return out;
    }
    out.x = e4m3_pack4(v[0], v[1], v[2], v[3]);
    out.y = e4m3_pack4(v[4], v[5], v[6], v[7]);
    return out;
}

__device__ __forceinline__ float absmax8(const float (&x)[8]) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
    return m;
}

// Groups [blockIdx.x * 16 * U, +16 * U): pass u handles groups base + 16 u + row.
template <int kQuantUnroll>
__global__ __launch_bounds__(kQuantThreads) void quant_act_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ s, int64_t n_groups) {
    const int row = threadIdx.x >> 4;
    const int sub = threadIdx.x & 15;
    const int64_t base = (int64_t)blockIdx.x * (16 * kQuantUnroll);
    uint4 raw[kQuantUnroll];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
        const int64_t g = base + 16 * u + row;
        if (g < n_groups)
            raw[u] = reinterpret_cast<const uint4*>(x + g * kGroup)[sub];
    }
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
        const int64_t g = base + 16 * u + row;
        if (g >= n_groups) continue;             // uniform over the 16-lane row
        float v[8];
        unpack8(raw[u], v);
        const float amax = row16_max(absmax8(v));
        const float sc = amax / kE4M3Max;
        reinterpret_cast<uint2*>(q + g * kGroup)[sub] = quant8(v, sc);
        if (sub == 0) s[g] = sc;
    }
}

// h = BF16(g u / (1 + e^-g)) for 8 values, exactly rounded.  Float32 first:
// h32 = fl32(fl32(g u) rcp(fl32(1 + expf(-g)))) has a relative error of at most about
// 7 float32 ulps (expf and the hardware reciprocal within 1 ulp each, three
// roundings), so its BF16 rounding (nearest even) is the exact one unless h32 lies
// within 16 ulps of a BF16 rounding midpoint (low 16 bits in [0x7FF0, 0x8010)), or
// outside [2^-120, 2^127) in magnitude while g u is not zero (float32 underflow or
// overflow on the way); those elements (rare) are redone in float64.  g u = 0 gives
// the signed zero float64 gives.  The tests are collected as wave masks.
__device__ __forceinline__ void silu_mul8(const float (&gv)[8], const float (&uv)[8], float (&h)[8]) {
    float h32[8];
    uint64_t redo_mask = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float gu = gv[i] * uv[i];
        h32[i] = gu * __builtin_amdgcn_rcpf(1.0f + expf(-gv[i]));
        const uint32_t b = __float_as_uint(h32[i]);
        const float a = fabsf(h32[i]);
        redo_mask |= __builtin_amdgcn_ballot_w64(((b + 16u) & 0xFFE0u) == 0x8000u);
        redo_mask |= __builtin_amdgcn_ballot_w64(!(a >= 0x1p-120f && a < 0x1p127f)) &
                     __builtin_amdgcn_ballot_w64(gu != 0.0f);
    }
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const v2f pair = {h32[i], h32[i + 1]};
        const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, v2bf));
        h[i] = __uint_as_float(hb << 16);
        h[i + 1] = __uint_as_float(hb & 0xFFFF0000u);
    }
    if (redo_mask) {                                   // wave-uniform; lanes re-test their elements
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t b = __float_as_uint(h32[i]);
            const float a = fabsf(h32[i]);
            if (((b + 16u) & 0xFFE0u) == 0x8000u || (!(a >= 0x1p-120f && a < 0x1p127f) && gv[i] * uv[i] != 0.0f)) {
                const double gd = (double)gv[i];
                const double silu = gd / (1.0 + exp(-gd));
                h[i] = bf16_to_f32(f64_to_bf16_rne(silu * (double)uv[i]));
            }
        }
    }
}

// gu [M, 2I]: gate = columns [0, I), up = [I, 2I).  The grid is 2-D: blockIdx.y walks
// the rows (stride gridDim.y), blockIdx.x the groups of a row, 16 U per block, so a
// lane finds its row and column without a division.  Group j of row m covers h
// columns 128 j + [0, 128); its codes and scale sit at group index m (I/128) + j.
template <int kQuantUnroll>
__global__ __launch_bounds__(kQuantThreads) void silu_mul_quant_kernel(
    const uint16_t* __restrict__ gu, uint8_t* __restrict__ q, float* __restrict__ s,
    int64_t M, int64_t groups_per_row, int64_t I) {
    const int row = threadIdx.x >> 4;
    const int sub = threadIdx.x & 15;
    const int64_t j0 = (int64_t)blockIdx.x * (16 * kQuantUnroll);
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        const uint16_t* grow = gu + m * 2 * I;
        uint4 graw[kQuantUnroll], uraw[kQuantUnroll];
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u) {
            const int64_t j = j0 + 16 * u + row;
            if (j < groups_per_row) {
                const uint16_t* p = grow + j * kGroup;
                graw[u] = reinterpret_cast<const uint4*>(p)[sub];
                uraw[u] = reinterpret_cast<const uint4*>(p + I)[sub];
            }
        }
#pragma unroll
        for (int u = 0; u < kQuantUnroll; ++u) {
            const int64_t j = j0 + 16 * u + row;
            if (j >= groups_per_row) continue;           // uniform over the 16-lane row
            const int64_t g = m * groups_per_row + j;
            float gv[8], uv[8], h[8];
            unpack8(graw[u], gv);
            unpack8(uraw[u], uv);
            silu_mul8(gv, uv, h);
            const float amax = row16_max(absmax8(h));
            const float sc = amax / kE4M3Max;
            reinterpret_cast<uint2*>(q + g * kGroup)[sub] = quant8(h, sc);
            if (sub == 0) s[g] = sc;
        }
    }
}

// One 256-thread block per 128x128 weight block.  Thread t covers row t / 2 of the
// block, columns 64 (t % 2) + [0, 64).
__global__ __launch_bounds__(256) void quant_weight_kernel(
    const uint16_t* __restrict__ w, uint8_t* __restrict__ qw, float* __restrict__ ws,
    int64_t N, int64_t K) {
    __shared__ float wave_amax[4];
    const int64_t kblocks = K / kGroup;
    const int64_t bi = blockIdx.x / kblocks, bj = blockIdx.x % kblocks;
    const int t = threadIdx.x;
    const int64_t r = bi * kGroup + (t >> 1);
    const int64_t c = bj * kGroup + (t & 1) * 64;
    const uint4* src = reinterpret_cast<const uint4*>(w + r * K + c);
    float v[8][8];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        unpack8(src[i], v[i]);
        m = fmaxf(m, absmax8(v[i]));
    }
    m = wave_max(m);
    if ((t & 63) == 0) wave_amax[t >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(wave_amax[0], wave_amax[1]), fmaxf(wave_amax[2], wave_amax[3]));
    const float sc = amax / kE4M3Max;
    uint2* dst = reinterpret_cast<uint2*>(qw + r * K + c);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = quant8(v[i], sc);
    if (t == 0) ws[blockIdx.x] = sc;
}

// RMSNorm + quantization, one workgroup per row m of x [M, K].  Thread (grow, sub)
// -- 16-lane DPP row grow, lane sub -- owns 16-byte chunk sub of the row's groups
// grow, grow + 16, ...:
//   1. it loads those chunks of x and gamma (kept in registers when the row fits,
//      U chunks per thread) and sums the squares of x in float64 (x^2 is exact for
//      BF16 x); the wave (shuffles) and the workgroup (LDS, fixed order, so the
//      result is deterministic) reduce;  r = 1 / sqrt(sum / K + eps) (rsqrt_f64);
//   2. per group: h = BF16((x r) gamma), the BF16 rounding of the float64 value
//      (decided in float32 where that is provably the same), then the group's
//      amax, scale and codes as in quant_act_kernel.
// U = 0 is the general form for long rows: x and gamma are read again in step 2
// (from cache).
// Threads per row: 256, or 1024 for a few rows (a decode batch), where one
// workgroup per row leaves most CUs idle and the row's latency is the call's time:
// four times the threads cut the serial chain of groups per thread by four.
constexpr int kNormThreads = 256;
constexpr int kNormThreadsFew = 1024;
constexpr int64_t kNormFewRows = 64;

// h = BF16((x r) gamma) for 8 values, exactly rounded.  Float32 first:
// h32 = fl32(fl32(x r32) gamma) is within 4 float32 ulps of the exact product, so its
// BF16 rounding (v_cvt_pk_bf16_f32, nearest even) is the exact one unless h32 lies
// within 8 ulps of a BF16 rounding midpoint (low 16 bits in [0x7FF8, 0x8008)) or
// below 2^-120 in magnitude (near the BF16 subnormal range); those elements (rare)
// are redone in float64.
__device__ __forceinline__ void rmsnorm8(const float (&xf)[8], const float (&gf)[8], double r, float r32,
                                         float (&h)[8]) {
    float h32[8];
    // The tests are collected as wave masks (one compare each, the masks combined
    // by scalar instructions), not as per-lane booleans.
    uint64_t redo_mask = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h32[i] = (xf[i] * r32) * gf[i];
        const uint32_t b = __float_as_uint(h32[i]);
        redo_mask |= __builtin_amdgcn_ballot_w64(((b + 8u) & 0xFFF0u) == 0x8000u);
        redo_mask |= __builtin_amdgcn_ballot_w64(fabsf(h32[i]) < 0x1p-120f) &
                     __builtin_amdgcn_ballot_w64(h32[i] != 0.0f);
    }
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const v2f pair = {h32[i], h32[i + 1]};
        const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, v2bf));
        h[i] = __uint_as_float(hb << 16);
        h[i + 1] = __uint_as_float(hb & 0xFFFF0000u);
    }
    if (redo_mask) {                                   // wave-uniform; lanes re-test their elements
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t b = __float_as_uint(h32[i]);
            if (((b + 8u) & 0xFFF0u) == 0x8000u || (fabsf(h32[i]) < 0x1p-120f && h32[i] != 0.0f))
                h[i] = bf16_to_f32(f64_to_bf16_rne(((double)xf[i] * r) * (double)gf[i]));
        }
    }
}

// 1 / sqrt(a) for a > 0, a normal float64: the hardware estimate and three Newton
// steps y <- y + y (1/2 - (a/2) y^2), each at least squaring the relative error, so
// the result is within a few float64 ulps (the BF16 rounding of h needs about
// 2^-40; the FP64 redo of a near-midpoint element sees the same few-ulp r).
__device__ __forceinline__ double rsqrt_f64(double a) {
    const double half_a = 0.5 * a;
    double y = __builtin_amdgcn_rsq(a);
#pragma unroll
    for (int it = 0; it < 3; ++it) {
        const double e = fma(-half_a * y, y, 0.5);
        y = fma(y, e, y);
    }
    return y;
}

template <int U, int NT>
__global__ __launch_bounds__(NT) void rmsnorm_quant_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, double eps, double inv_k, uint8_t* __restrict__ q,
    float* __restrict__ s, int64_t K) {
    __shared__ double part[NT / 64];
    const int64_t m = blockIdx.x;
    const uint16_t* xr = x + m * K;
    const int grow = threadIdx.x >> 4;
    const int sub = threadIdx.x & 15;
    const int64_t groups = K / kGroup;
    constexpr int UR = U > 0 ? U : 1;
    uint4 xraw[UR], graw[UR];
    double ss = 0.0;
    if (U > 0) {
        // x and gamma chunks requested together, before the reduction
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t j = grow + (NT / 16) * u;
            if (j < groups) {
                xraw[u] = reinterpret_cast<const uint4*>(xr + j * kGroup)[sub];
                graw[u] = reinterpret_cast<const uint4*>(gamma + j * kGroup)[sub];
            }
        }
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t j = grow + (NT / 16) * u;
            if (j >= groups) continue;
            float v[8];
            unpack8(xraw[u], v);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += (double)v[i] * (double)v[i];
        }
    } else {
        for (int64_t j = grow; j < groups; j += (NT / 16)) {
            float v[8];
            unpack8(reinterpret_cast<const uint4*>(xr + j * kGroup)[sub], v);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += (double)v[i] * (double)v[i];
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    double total = 0.0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) total += part[w];
    const double r = rsqrt_f64(total * inv_k + eps);
    const float r32 = (float)r;

    auto emit = [&](int64_t j, const uint4& xv, const uint4& gv) {      // uniform over the 16-lane row
        float xf[8], gf[8], h[8];
        unpack8(xv, xf);
        unpack8(gv, gf);
        rmsnorm8(xf, gf, r, r32, h);
        const float amax = row16_max(absmax8(h));
        const float sc = amax / kE4M3Max;
        reinterpret_cast<uint2*>(q + m * K + j * kGroup)[sub] = quant8(h, sc);
        if (sub == 0) s[m * groups + j] = sc;
    };
    if (U > 0) {
#pragma unroll
        for (int u = 0; u < UR; ++u) {
            const int64_t j = grow + (NT / 16) * u;
            if (j < groups) emit(j, xraw[u], graw[u]);
        }
    } else {
        for (int64_t j = grow; j < groups; j += (NT / 16))
            emit(j, reinterpret_cast<const uint4*>(xr + j * kGroup)[sub],
                 reinterpret_cast<const uint4*>(gamma + j * kGroup)[sub]);
    }
}

template <int NT>
static void launch_norm(int64_t M, int64_t K, const uint16_t* xp, const uint16_t* gp, double e, double inv_k, void* q,
                        float* s, hipStream_t st) {
    const int64_t passes = (K / kGroup + NT / 16 - 1) / (NT / 16);     // groups in flight per pass: NT / 16
    const dim3 grid((unsigned)M), block(NT);
    if (passes <= 1)
        hipLaunchKernelGGL((rmsnorm_quant_kernel<1, NT>), grid, block, 0, st, xp, gp, e, inv_k, (uint8_t*)q, s, K);
    else if (passes <= 2)
        hipLaunchKernelGGL((rmsnorm_quant_kernel<2, NT>), grid, block, 0, st, xp, gp, e, inv_k, (uint8_t*)q, s, K);
    else if (passes <= 4)
        hipLaunchKernelGGL((rmsnorm_quant_kernel<4, NT>), grid, block, 0, st, xp, gp, e, inv_k, (uint8_t*)q, s, K);
    else if (passes <= 8)
        hipLaunchKernelGGL((rmsnorm_quant_kernel<8, NT>), grid, block, 0, st, xp, gp, e, inv_k, (uint8_t*)q, s, K);
    else {
        // 16 chunks per thread fit the registers of 256-thread workgroups only.
        if constexpr (NT <= kNormThreads) {
            if (passes <= 16) {
                hipLaunchKernelGGL((rmsnorm_quant_kernel<16, NT>), grid, block, 0, st, xp, gp, e, inv_k, (uint8_t*)q,
                                   s, K);
                return;
            }
        }
        hipLaunchKernelGGL((rmsnorm_quant_kernel<0, NT>), grid, block, 0, st, xp, gp, e, inv_k, (uint8_t*)q, s, K);
    }
}

hipError_t launch_rmsnorm_quant(const void* x, const void* gamma, float eps, void* q, float* s, int64_t M, int64_t K,
                                hipStream_t st) {
    if (M == 0) return hipSuccess;
    const uint16_t* xp = (const uint16_t*)x;
    const uint16_t* gp = (const uint16_t*)gamma;
    const double e = (double)eps;
    const double inv_k = 1.0 / (double)K;
    if (M <= kNormFewRows)
        launch_norm<kNormThreadsFew>(M, K, xp, gp, e, inv_k, q, s, st);
    else
        launch_norm<kNormThreads>(M, K, xp, gp, e, inv_k, q, s, st);
    return hipGetLastError();
}

hipError_t launch_quant_act(const void* x, void* q, float* s, int64_t M, int64_t K, hipStream_t st) {
    const int64_t n_groups = M * (K / kGroup);
    if (n_groups == 0) return hipSuccess;
    if (n_groups < kSmallGroups) {
        hipLaunchKernelGGL(quant_act_kernel<1>, dim3((unsigned)((n_groups + 15) / 16)), dim3(kQuantThreads), 0, st,
                           (const uint16_t*)x, (uint8_t*)q, s, n_groups);
    } else {
        const int64_t per_block = 16 * kQuantUnrollBig;
        hipLaunchKernelGGL(quant_act_kernel<kQuantUnrollBig>, dim3((unsigned)((n_groups + per_block - 1) / per_block)),
                           dim3(kQuantThreads), 0, st, (const uint16_t*)x, (uint8_t*)q, s, n_groups);
    }
    return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const void* gu, void* q, float* s, int64_t M, int64_t I, hipStream_t st) {
    const int64_t gpr = I / kGroup;
    const int64_t n_groups = M * gpr;
    if (n_groups == 0) return hipSuccess;
    // Rows beyond the grid's second dimension are walked by the blocks (stride gridDim.y).
    const unsigned rows = (unsigned)(M < 65535 ? M : 65535);
    if (n_groups < kSmallGroups) {
        hipLaunchKernelGGL(silu_mul_quant_kernel<1>, dim3((unsigned)((gpr + 15) / 16), rows), dim3(kQuantThreads), 0,
                           st, (const uint16_t*)gu, (uint8_t*)q, s, M, gpr, I);
    } else {
        const int64_t per_block = 16 * kSiluUnrollBig;
        hipLaunchKernelGGL(silu_mul_quant_kernel<kSiluUnrollBig>, dim3((unsigned)((gpr + per_block - 1) / per_block), rows),
                           dim3(kQuantThreads), 0, st, (const uint16_t*)gu, (uint8_t*)q, s, M, gpr, I);
    }
    return hipGetLastError();
}

hipError_t launch_quant_weight(const void* w, void* qw, float* ws, int64_t N, int64_t K, hipStream_t st) {
    const int64_t nblocks = (N / kGroup) * (K / kGroup);
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL(quant_weight_kernel, dim3((unsigned)nblocks), dim3(256), 0, st,
                       (const uint16_t*)w, (uint8_t*)qw, ws, N, K);
    return hipGetLastError();
}

}  // namespace fp8bs
