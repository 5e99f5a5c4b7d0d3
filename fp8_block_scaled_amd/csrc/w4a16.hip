// NVFP4 weight-only linear (W4A16) on gfx950: weight-streaming kernel.
//
// y[m, n] = g * sum_k x[m, k] * e2m1(code[n, k]) * e4m3(bs[n, k / 16])
// ("Nanbeige4.3-33B-NVFP4-A16" model card, paragraph on the base revision and
// calibration: E2M1 weights in groups of 16 with E4M3 group scales and a global
// scale; BF16 activations).
//
// Dequantization is exact and happens in registers: gfx950 converts a byte of two
// E2M1 codes to two float32 values in one instruction (v_cvt_scalef32_pk_f32_fp4;
// its scale operand contributes only its exponent, so it is left at 1.0), one
// multiply applies the group scale (a 2-bit times a 4-bit significand: exact), and
// v_cvt_pk_bf16_f32 packs the exact products into BF16 pairs.  The products then
// meet the BF16 activations in v_mfma_f32_16x16x32_bf16, whose FP32 accumulation
// needs no promotion step (the group scales are already inside the operand); the
// global scale multiplies once at the end.
//
// Decode and batched decode (M up to 64) are bound by the weight stream: 0.5625
// bytes per weight against 2 M flops.  One workgroup takes NS strips of 16 output
// columns; its S waves split the 128-wide K blocks, each wave dequantizes a strip's
// fragment once and multiplies it by R 16-token groups of the activations; partial
// sums are added through LDS in a fixed order (deterministic).  A second grid
// dimension covers M in chunks of 16 R rows (rows past M are loaded from row M - 1
// and not stored).
//
// MFMA operands per lane l (g = l / 16, r = l % 16) and K block kb: the lane loads
// the 16 code bytes [64 kb + 16 g, +16) of weight row 16 st + r, i.e. codes
// k = 128 kb + 32 g + i, i < 32.  MFMA j (j < 4) takes codes i in [8 j, 8 j + 8)
// (dword j; group 2 g + j / 2) as B column r, and activations
// x[m][128 kb + 32 g + 8 j + e], e < 8, of token row m = 16 rho + r as A row r.
// A and B use the same k for the same (lane group, element), which is all the
// contraction needs.  Result lane l holds C[4 g + e][r]: token 16 rho + 4 g + e,
// output column 16 st + r.
#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace fp8bs {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v8f __attribute__((ext_vector_type(8)));

constexpr int kW4MaxWaves = 8;

struct W4Args {
    const uint8_t* w;        // [N, K/2] packed codes
    const uint8_t* bs;       // [N, K/16] E4M3 group scales
    const uint16_t* x;       // [M, K] BF16
    uint16_t* y;             // [M, N] BF16
    float g;
    int M;
    int64_t N, K, KB;
    int64_t strips;          // N / 16
};

// Eight weights of one MFMA operand: the codes of dword c (element 2 i in the low
// nibble of byte i) times the group scale s, as BF16 (exact).
__device__ __forceinline__ v8bf dequant8(uint32_t c, float s) {
    const v2f p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
    const v2f p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
    const v2f p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
    const v2f p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
    const v8f v = {p0[0] * s, p0[1] * s, p1[0] * s, p1[1] * s, p2[0] * s, p2[1] * s, p3[0] * s, p3[1] * s};
    return __builtin_convertvector(v, v8bf);
}

__device__ __forceinline__ v8bf as_bf8(v4i v) {
    v8bf r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}

template <int R, int NS>
__global__ __launch_bounds__(kW4MaxWaves * 64) void w4a16_stream_kernel(W4Args a) {
    extern __shared__ __attribute__((aligned(16))) v4f red[];      // [S][NS][R][64] partial sums
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int64_t strip0 = (int64_t)blockIdx.x * NS;
    const int m0 = blockIdx.y * 16 * R;
    const int64_t kb0 = (wave * a.KB) / S;
    const int64_t kb1 = ((wave + 1) * a.KB) / S;

    const uint16_t* xrow[R];
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        const int m = m0 + 16 * rho + r < a.M ? m0 + 16 * rho + r : a.M - 1;
        xrow[rho] = a.x + (int64_t)m * a.K + 32 * g;
    }
    const uint8_t* wrow[NS];
    const uint8_t* srow[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        // Strips past the last one (a partial final workgroup) re-read the last
        // strip; their results are not stored.
        const int64_t st = strip0 + q < a.strips ? strip0 + q : a.strips - 1;
        const int64_t n = st * 16 + r;
        wrow[q] = a.w + n * (a.K / 2) + 16 * g;
        srow[q] = a.bs + n * (a.K / 16) + 2 * g;
    }

    v4f acc[NS][R];
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
        for (int rho = 0; rho < R; ++rho) acc[q][rho] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    struct Frag {
        v4i wv[NS];
        uint32_t sv[NS];
        v4i xv[R][4];
    };
    auto load = [&](Frag& f, int64_t kb) {
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            f.wv[q] = *reinterpret_cast<const v4i*>(wrow[q] + kb * 64);
            f.sv[q] = *reinterpret_cast<const uint16_t*>(srow[q] + kb * 8);
        }
#pragma unroll
        for (int rho = 0; rho < R; ++rho) {
            const v4i* xp = reinterpret_cast<const v4i*>(xrow[rho] + kb * kGroup);
#pragma unroll
            for (int j = 0; j < 4; ++j) f.xv[rho][j] = xp[j];
        }
    };
    auto compute = [&](const Frag& f) {
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)f.sv[q], 0);
            const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)f.sv[q], 1);
            v8bf b[4];
            b[0] = dequant8((uint32_t)f.wv[q].x, s0);
            b[1] = dequant8((uint32_t)f.wv[q].y, s0);
            b[2] = dequant8((uint32_t)f.wv[q].z, s1);
            b[3] = dequant8((uint32_t)f.wv[q].w, s1);
#pragma unroll
            for (int rho = 0; rho < R; ++rho)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[q][rho] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(f.xv[rho][j]), b[j], acc[q][rho], 0, 0, 0);
        }
    };
    // Four token groups hold 64 activation registers per K block: one block in flight.
    constexpr bool kTwoInFlight = R <= 2;
    if (!kTwoInFlight) {
        Frag f;
        for (int64_t kb = kb0; kb < kb1; ++kb) {
            load(f, kb);
            compute(f);
        }
    } else if (kb0 < kb1) {
        Frag fa, fb;
        load(fa, kb0);
        int64_t kb = kb0;
        for (; kb + 1 < kb1; kb += 2) {
            load(fb, kb + 1);
            compute(fa);
            if (kb + 2 < kb1) load(fa, kb + 2);
            compute(fb);
        }
        if (kb < kb1) compute(fa);
    }

#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
        for (int rho = 0; rho < R; ++rho) red[((wave * NS + q) * R + rho) * 64 + lane] = acc[q][rho];
    __syncthreads();
    // Output o: r = o % 16 fastest (16 neighbouring columns per 16 threads), then
    // the lane group gg, the element e, and (q, rho).
    for (int o = threadIdx.x; o < NS * R * 256; o += blockDim.x) {
        const int rr = o & 15, gg = (o >> 4) & 3, e = (o >> 6) & 3, qr = o >> 8;
        const int q = qr / R, rho = qr % R;
        const int m = m0 + 16 * rho + 4 * gg + e;
        if (m >= a.M || strip0 + q >= a.strips) continue;
        const int l = gg * 16 + rr;
        float sum = 0.0f;
        for (int w = 0; w < S; ++w) sum += red[((w * NS + q) * R + rho) * 64 + l][e];
        const int64_t n = (strip0 + q) * 16 + rr;
        a.y[(int64_t)m * a.N + n] = (uint16_t)f32_to_bf16_rne(a.g * sum);
    }
}

// Decode (M <= 16): K chunks folded into the MFMA, activations held in registers.
//
// v_mfma_f32_16x16x32_bf16 multiplies 16 rows of A by 16 columns of B over 32
// k.  With M <= P (P = 4, 8 or 16) the 16 rows and columns are split into
// G = 16 / P groups of P: group t of A holds the P token rows and group t of B the
// P weight rows of the strip, both at K chunk t of a "super block" of G x 128 k.
// The G diagonal P x P blocks of the result are then independent products over
// their own chunks; the off-diagonal blocks are discarded.  A strip is P output
// columns, so decode shapes give many strips and every CU gets an even share (a
// CU's own bandwidth is limited, so one strip more on one CU would set the time).
//
// k of (MFMA u < 4, group t, lane group g, element e) = 128 t + 32 g + 8 u + e
// within the super block: lane l (g = l / 16, r = l % 16, t = r / P) loads 16
// contiguous code bytes of weight row r % P of the strip, its 2 group scales, and
// (once) 64 contiguous activation bytes of token row r % P (zero when >= M).  A
// and B use the same k for the same (t, lane group, element), which is all the
// contraction needs.  Result lane l holds C[4 g + e][r]: token (4 g + e) % P of
// group (4 g + e) / P against weight row r % P of group r / P; it is a diagonal
// element when the two groups agree.
//
// A workgroup's S waves split the super blocks into equal slices of KBW; each
// wave loads its activation slice once (16 VGPRs per super block), then streams the
// workgroup's strips through it with D strips of loads in flight (one 16-byte code
// load and one 2-byte scale load per lane and super block).  The strip loop has no
// branches: strip indices past the workgroup's last strip are clamped to it (a
// repeated load that hits in L2) and their partial sums land in LDS slots that are
// never read.  The diagonal lanes store their partial sums compactly in LDS; after
// one barrier every output adds its G chunk groups and S waves in a fixed order.
constexpr int kW4DecodeMaxWaves = 16;
constexpr int64_t kW4DecodeSlotBytes = 96 * 1024;   // LDS for partial sums (at most)

template <int P, int KBW>
struct W4DecodeShape {
    static constexpr int G = 16 / P;             // chunk groups per MFMA
    static constexpr int U = 4 * P;              // diagonal lanes per wave
    static constexpr int D = KBW <= 2 ? 4 : 2;   // strips of loads in flight
};

// Threads per workgroup at most (the register budget of a wave's slice).
constexpr int w4_decode_threads(int p, int kbw) {
    return (kbw == 1 && p == 16 ? 8 : (kbw <= 2 ? 16 : (kbw <= 4 ? 8 : 4))) * 64;
}

template <int P, int KBW>
__global__ __launch_bounds__(w4_decode_threads(P, KBW)) void w4a16_decode_kernel(
    W4Args a, int64_t strips_per_wg, int slots) {
    typedef W4DecodeShape<P, KBW> Sh;
    constexpr int G = Sh::G, U = Sh::U, D = Sh::D;
    extern __shared__ __attribute__((aligned(16))) v4f red[];      // [S][slots][U]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int t = r / P, j = r % P;
    const int64_t sbk = (int64_t)G * kGroup;                        // k per super block
    const int64_t k0 = (int64_t)wave * KBW * sbk + 128 * t + 32 * g;   // this lane's first k
    const int64_t st_begin = (int64_t)blockIdx.x * strips_per_wg;
    const int64_t st_end = st_begin + strips_per_wg < a.strips ? st_begin + strips_per_wg : a.strips;
    const int64_t last = st_end - 1;         // >= st_begin: the grid has no empty workgroup

    v4i xv[KBW][4];
#pragma unroll
    for (int i = 0; i < KBW; ++i)
#pragma unroll
        for (int u = 0; u < 4; ++u) xv[i][u] = v4i{0, 0, 0, 0};
    if (j < a.M) {
        const uint16_t* xp = a.x + (int64_t)j * a.K + k0;
#pragma unroll
        for (int i = 0; i < KBW; ++i)
#pragma unroll
            for (int u = 0; u < 4; ++u) xv[i][u] = *reinterpret_cast<const v4i*>(xp + i * sbk + 8 * u);
    }

    struct Frag {
        v4i wv[KBW];
        uint32_t sv[KBW];
    };
    auto load = [&](Frag& f, int64_t st) {
        const int64_t n = (st < last ? st : last) * P + j;
        const uint8_t* wp = a.w + n * (a.K / 2) + k0 / 2;
        const uint8_t* sp = a.bs + n * (a.K / 16) + k0 / 16;
#pragma unroll
        for (int i = 0; i < KBW; ++i) {
            f.wv[i] = *reinterpret_cast<const v4i*>(wp + i * (sbk / 2));
            f.sv[i] = *reinterpret_cast<const uint16_t*>(sp + i * (sbk / 16));
        }
    };
    // A diagonal lane (group of its A rows == group of its column) stores its four
    // values at compact index g * P + j.
    const bool diag = (4 * g) / P == t;
    const int cidx = g * P + j;
    auto compute_store = [&](const Frag& f, int slot) {
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < KBW; ++i) {
            const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)f.sv[i], 0);
            const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)f.sv[i], 1);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(xv[i][0]), dequant8((uint32_t)f.wv[i].x, s0), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(xv[i][1]), dequant8((uint32_t)f.wv[i].y, s0), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(xv[i][2]), dequant8((uint32_t)f.wv[i].z, s1), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(xv[i][3]), dequant8((uint32_t)f.wv[i].w, s1), acc, 0, 0, 0);
        }
        if (diag) red[((int64_t)wave * slots + slot) * U + cidx] = acc;
    };

    // slots is a multiple of D and >= the workgroup's strip count.
    Frag fr[D];
#pragma unroll
    for (int d = 0; d < D - 1; ++d) load(fr[d], st_begin + d);
    for (int i = 0; i < slots; i += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            load(fr[(d + D - 1) % D], st_begin + i + d + D - 1);
            compute_store(fr[d], i + d);
        }
    }
    __syncthreads();
    // Output o: weight row jj fastest (P neighbouring columns), then token, strip.
    // Token ti of chunk group tt sits at A row P tt + ti = 4 gg + e.
    const int nb = (int)(st_end - st_begin);
    for (int o = threadIdx.x; o < nb * P * P; o += blockDim.x) {
        const int jj = o % P, ti = (o / P) % P, b = o / (P * P);
        if (ti >= a.M) continue;
        float sum = 0.0f;
        for (int w = 0; w < S; ++w)
            for (int tt = 0; tt < G; ++tt) {
                const int row = P * tt + ti, gg = row >> 2, e = row & 3;
                sum += red[((int64_t)w * slots + b) * U + gg * P + jj][e];
            }
        a.y[(int64_t)ti * a.N + (st_begin + b) * P + jj] = (uint16_t)f32_to_bf16_rne(a.g * sum);
    }
}

// Decode schedule: P from M; waves S (<= 16) and super blocks per wave KBW
// (1, 2, 4 or 8) with S * KBW = K / (128 G), preferring the most waves the
// register budget of the slice allows.  false if K does not split that way.
static bool decode_shape(int64_t M, int64_t K, int* P, int* S, int* KBW) {
    *P = M <= 4 ? 4 : (M <= 8 ? 8 : 16);
    const int64_t G = 16 / *P;
    if (K % (kGroup * G) != 0) return false;
    const int64_t SB = K / (kGroup * G);
    const int kbws[4] = {1, 2, 4, 8};
    int best_s = 0, best_k = 0;
    for (int q = 0; q < 4; ++q)
        if (SB % kbws[q] == 0 && SB / kbws[q] <= w4_decode_threads(*P, kbws[q]) / 64 && SB / kbws[q] > best_s) {
            best_s = (int)(SB / kbws[q]);
            best_k = kbws[q];
        }
    if (best_s == 0) return false;
    *S = best_s;
    *KBW = best_k;
    return true;
}

W4Plan plan_w4a16(int64_t M, int64_t N, int64_t K, int cus) {
    W4Plan p{};
    p.groups = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.strips = N / 16;
    p.kblocks = K / kGroup;
    p.m_chunks = M > 0 ? (M + 16 * p.groups - 1) / (16 * p.groups) : 0;
    p.strips_per_wg = (p.strips >= 4 * (int64_t)cus) ? 2 : 1;
    if (const char* e = getenv("FP8BS_W4_STRIPS")) {        // tuning hook
        const int v = atoi(e);
        if (v == 1 || v == 2) p.strips_per_wg = v;
    }
    p.strip_wgs = (p.strips + p.strips_per_wg - 1) / p.strips_per_wg;
    p.waves = (int)(p.kblocks < kW4MaxWaves ? p.kblocks : kW4MaxWaves);
    if (const char* e = getenv("FP8BS_W4_WAVES")) {         // tuning hook
        const int v = atoi(e);
        if (v >= 1 && v <= kW4MaxWaves) p.waves = v;
    }
    // Decode: K chunks folded into the MFMA, activations in registers.
    int P = 0, S = 0, KBW = 0;
    const char* de = getenv("FP8BS_W4_DECODE");              // tuning hook: 0 = stream kernel
    if (M <= 16 && decode_shape(M, K, &P, &S, &KBW) && !(de && atoi(de) == 0)) {
        p.decode_p = P;
        p.decode_kbw = KBW;
        p.waves = S;
        const int Dp = KBW <= 2 ? 4 : 2;
        const int64_t strips = N / P;
        int64_t spw = (strips + cus - 1) / cus;
        if (const char* e = getenv("FP8BS_W4_DECODE_SPW")) {  // tuning hook
            const int v = atoi(e);
            if (v >= 1) spw = v;
        }
        // LDS: S waves x slots x 4P lanes x 16 bytes.
        const int64_t per_slot = (int64_t)S * 4 * P * 16;
        int64_t max_slots = (kW4DecodeSlotBytes / per_slot) / Dp * Dp;
        if (max_slots < Dp) max_slots = Dp;
        if (spw > max_slots) spw = max_slots;
        p.decode_strips_per_wg = spw;
        p.decode_slots = (int)((spw + Dp - 1) / Dp * Dp);
        p.decode_wgs = (strips + spw - 1) / spw;              // every workgroup gets a strip
    }
    return p;
}

template <int P, int KBW>
static hipError_t launch_w4_decode(const W4Plan& plan, hipStream_t st, const W4Args& a) {
    const unsigned lds = (unsigned)((int64_t)plan.waves * plan.decode_slots * 4 * P * sizeof(v4f));
    static bool attr_set = false;            // idempotent; a race only repeats the call
    if (lds > 65536 && !attr_set) {
        const hipError_t e = hipFuncSetAttribute((const void*)w4a16_decode_kernel<P, KBW>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((w4a16_decode_kernel<P, KBW>), dim3((unsigned)plan.decode_wgs), dim3(plan.waves * 64), lds, st,
                       a, plan.decode_strips_per_wg, plan.decode_slots);
    return hipGetLastError();
}

template <int P>
static hipError_t launch_w4_decode_p(const W4Plan& plan, hipStream_t st, const W4Args& a) {
    switch (plan.decode_kbw) {
        case 1: return launch_w4_decode<P, 1>(plan, st, a);
        case 2: return launch_w4_decode<P, 2>(plan, st, a);
        case 4: return launch_w4_decode<P, 4>(plan, st, a);
        default: return launch_w4_decode<P, 8>(plan, st, a);
    }
}

template <int R, int NS>
static hipError_t launch_w4_rns(dim3 grid, dim3 block, unsigned lds, hipStream_t st, const W4Args& a) {
    // More than 64 KiB of LDS needs the per-kernel limit raised, up to the CU's 160 KiB.
    static bool attr_set = false;            // idempotent; a race only repeats the call
    if (lds > 65536 && !attr_set) {
        const hipError_t e = hipFuncSetAttribute((const void*)w4a16_stream_kernel<R, NS>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((w4a16_stream_kernel<R, NS>), grid, block, lds, st, a);
    return hipSuccess;
}

template <int R>
static hipError_t launch_w4_r(const W4Plan& plan, dim3 grid, dim3 block, unsigned lds, hipStream_t st,
                              const W4Args& a) {
    if (plan.strips_per_wg == 2) return launch_w4_rns<R, 2>(grid, block, lds, st, a);
    return launch_w4_rns<R, 1>(grid, block, lds, st, a);
}

hipError_t launch_w4a16(const W4Plan& plan, const void* x, const void* w, const void* bs, float gscale, void* y,
                        int64_t M, int64_t N, int64_t K, hipStream_t st) {
    if (plan.strip_wgs == 0 || plan.m_chunks == 0) return hipSuccess;
    W4Args a;
    a.w = (const uint8_t*)w;
    a.bs = (const uint8_t*)bs;
    a.x = (const uint16_t*)x;
    a.y = (uint16_t*)y;
    a.g = gscale;
    a.M = (int)M;
    a.N = N;
    a.K = K;
    a.KB = plan.kblocks;
    a.strips = plan.strips;
    if (plan.decode_p > 0) {
        a.strips = N / plan.decode_p;        // strips of P columns
        switch (plan.decode_p) {
            case 4: return launch_w4_decode_p<4>(plan, st, a);
            case 8: return launch_w4_decode_p<8>(plan, st, a);
            default: return launch_w4_decode_p<16>(plan, st, a);
        }
    }
    const dim3 grid((unsigned)plan.strip_wgs, (unsigned)plan.m_chunks), block(plan.waves * 64);
    const unsigned lds = (unsigned)(plan.waves * plan.strips_per_wg * plan.groups * 64 * sizeof(v4f));
    hipError_t e;
    switch (plan.groups) {
        case 1: e = launch_w4_r<1>(plan, grid, block, lds, st, a); break;
        case 2: e = launch_w4_r<2>(plan, grid, block, lds, st, a); break;
        default: e = launch_w4_r<4>(plan, grid, block, lds, st, a); break;
    }
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace fp8bs
