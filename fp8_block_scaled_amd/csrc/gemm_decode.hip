// Decode-shape block-scaled FP8 GEMM (M <= 16) for gfx950.
//
// y[m, n] = sum_kb (s[m, kb] * ws[n/128, kb]) * sum_{k in kb} q[m, k] * w[n, k]
// ("Nanbeige4.3-33B FP8" model card, introduction: E4M3 weights in 128x128 blocks,
// dynamic per-token group-128 activation scales; FP32 accumulation, BF16 out).
//
// At M <= 16 the weight stream is ~all of the traffic (arithmetic intensity
// 2..32 flop/B), so the kernel is built to keep HBM busy:
//   * One v_mfma_f32_16x16x128_f8f6f4 covers a whole 128-wide K block of a
//     16-column strip: A = 16 weight rows (n), B = the M <= 16 token rows (m,
//     zero-padded).  Its FP32 result is promoted once per K block by the product
//     of the two scales.
//   * Work is split stream-K style: the (strip, K block) units are dealt out in
//     equal contiguous ranges to waves ("workers"), so every wave streams the same
//     number of weight bytes whatever N and K are.  A strip shared by several
//     workers is finished by the last of them to arrive (agent-scope counter in
//     the workspace), which adds the partial sums in worker order: deterministic.
//   * Each lane loads 2 x 16 bytes of its weight row per unit; chunks of 4 units
//     are double-buffered in registers so 8 loads per lane stay in flight.
//
// Operand layout per lane l (g = l / 16, r = l % 16): A row r = weight row n0 + r,
// B column r = token row r; both take K-block bytes [16 g, 16 g + 16) and
// [64 + 16 g, 64 + 16 g + 16).  The MFMA sums over the K positions of its operand
// registers, so any assignment of K bytes to register slots that is the same for A
// and B gives the same dot product.  Output: lane l holds C[4 g + i][r], i = 0..3,
// i.e. y[m = r][n0 + 4 g + i].
#include "device_common.h"
#include "launch.h"

namespace fp8bs {

constexpr int kDecodeThreads = 256;   // 4 workers (waves) per block
constexpr int kDecodeWavesPerCU = 8;
constexpr int kChunk = 4;             // K blocks per register buffer
// Workspace layout: [arrival counters, one int per strip, fixed 64 KiB][partials].
constexpr int64_t kMaxSplitStrips = 16384;
constexpr int64_t kCounterBytes = kMaxSplitStrips * 4;

struct DecodeArgs {
    const uint8_t* w;
    const float* ws;
    const uint8_t* x;
    const float* xs;
    uint16_t* y;
    float* part;
    int* cnt;
    int M;
    int64_t N, K, KB, workers, base, rem, maxc;
};

struct Unit {
    v4i w0, w1, x0, x1;
    float xs, ws;
};

__device__ __forceinline__ int64_t worker_of(int64_t u, int64_t base, int64_t rem) {
    const int64_t big = rem * (base + 1);
    return u < big ? u / (base + 1) : rem + (u - big) / base;
}

__device__ __forceinline__ void load_unit(Unit& d, const uint8_t* wrow, const uint8_t* xrow,
                                          const float* xsrow, const float* wsrow, bool mvalid, int64_t kb) {
    const v4i* wp = reinterpret_cast<const v4i*>(wrow + kb * kGroup);
    d.w0 = __builtin_nontemporal_load(wp);
    d.w1 = __builtin_nontemporal_load(wp + 4);
    if (mvalid) {
        const v4i* xp = reinterpret_cast<const v4i*>(xrow + kb * kGroup);
        d.x0 = xp[0];
        d.x1 = xp[4];
        d.xs = xsrow[kb];
    } else {
        d.x0 = v4i{0, 0, 0, 0};
        d.x1 = v4i{0, 0, 0, 0};
        d.xs = 0.0f;
    }
    d.ws = wsrow[kb];
}

__device__ __forceinline__ void mma_unit(const Unit& d, v4f& acc) {
    const v8i a = {d.w0.x, d.w0.y, d.w0.z, d.w0.w, d.w1.x, d.w1.y, d.w1.z, d.w1.w};
    const v8i b = {d.x0.x, d.x0.y, d.x0.z, d.x0.w, d.x1.x, d.x1.y, d.x1.z, d.x1.w};
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // Format 0 = E4M3 for both operands; zero scale operands select the unscaled MFMA.
    const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
    const float sc = d.xs * d.ws;
    acc[0] = fmaf(sc, p[0], acc[0]);
    acc[1] = fmaf(sc, p[1], acc[1]);
    acc[2] = fmaf(sc, p[2], acc[2]);
    acc[3] = fmaf(sc, p[3], acc[3]);
}

__device__ __forceinline__ void store_y(const DecodeArgs& a, const v4f& acc, int64_t n0, int lane) {
    const int m = lane & 15;
    if (m >= a.M) return;
    const int g = lane >> 4;
    uint2 o;
    o.x = f32_to_bf16_rne(acc[0]) | (f32_to_bf16_rne(acc[1]) << 16);
    o.y = f32_to_bf16_rne(acc[2]) | (f32_to_bf16_rne(acc[3]) << 16);
    *reinterpret_cast<uint2*>(a.y + m * a.N + n0 + 4 * g) = o;
}

__global__ __launch_bounds__(kDecodeThreads) void gemm_decode_kernel(DecodeArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t worker = (int64_t)blockIdx.x * (kDecodeThreads / 64) + (threadIdx.x >> 6);
    if (worker >= a.workers) return;
    const int64_t u_begin = worker * a.base + (worker < a.rem ? worker : a.rem);
    const int64_t u_end = u_begin + a.base + (worker < a.rem ? 1 : 0);
    const int g = lane >> 4, r = lane & 15;
    const bool mvalid = r < a.M;
    const uint8_t* xrow = a.x + (mvalid ? r : 0) * a.K + 16 * g;
    const float* xsrow = a.xs + (mvalid ? r : 0) * a.KB;

    for (int64_t u = u_begin; u < u_end;) {
        const int64_t strip = u / a.KB;
        const int64_t kb0 = u - strip * a.KB;
        const int64_t kb1 = (u_end - strip * a.KB) < a.KB ? (u_end - strip * a.KB) : a.KB;
        const int64_t n0 = strip * 16;
        const uint8_t* wrow = a.w + (n0 + r) * a.K + 16 * g;
        const float* wsrow = a.ws + (n0 / kGroup) * a.KB;

        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        Unit bufA[kChunk], bufB[kChunk];
        int64_t kb = kb0;
        {
            const int64_t c = kb1 - kb < kChunk ? kb1 - kb : kChunk;
#pragma unroll
            for (int i = 0; i < kChunk; ++i)
                if (i < c) load_unit(bufA[i], wrow, xrow, xsrow, wsrow, mvalid, kb + i);
        }
        while (true) {
            // bufA holds [kb, kb + cA); prefetch the next chunk into bufB.
            const int64_t cA = kb1 - kb < kChunk ? kb1 - kb : kChunk;
            const int64_t kbB = kb + cA;
            const int64_t cB = kb1 - kbB < kChunk ? kb1 - kbB : kChunk;
#pragma unroll
            for (int i = 0; i < kChunk; ++i)
                if (i < cB) load_unit(bufB[i], wrow, xrow, xsrow, wsrow, mvalid, kbB + i);
#pragma unroll
            for (int i = 0; i < kChunk; ++i)
                if (i < cA) mma_unit(bufA[i], acc);
            kb = kbB;
            if (kb >= kb1) break;
            // bufB holds [kb, kb + cB); prefetch into bufA.
            const int64_t kbA = kb + cB;
            const int64_t cA2 = kb1 - kbA < kChunk ? kb1 - kbA : kChunk;
#pragma unroll
            for (int i = 0; i < kChunk; ++i)
                if (i < cA2) load_unit(bufA[i], wrow, xrow, xsrow, wsrow, mvalid, kbA + i);
#pragma unroll
            for (int i = 0; i < kChunk; ++i)
                if (i < cB) mma_unit(bufB[i], acc);
            kb = kbA;
            if (kb >= kb1) break;
        }

        if (kb0 == 0 && kb1 == a.KB) {
            store_y(a, acc, n0, lane);
        } else {
            // Shared strip: publish the partial, then the last arriver reduces.
            const int64_t first = worker_of(strip * a.KB, a.base, a.rem);
            const int64_t last = worker_of(strip * a.KB + a.KB - 1, a.base, a.rem);
            const int64_t ncontrib = last - first + 1;
            float* slot = a.part + ((strip * a.maxc + (worker - first)) * 64 + lane) * 4;
            *reinterpret_cast<v4f*>(slot) = acc;
            __threadfence();
            int prev = 0;
            if (lane == 0)
                prev = __hip_atomic_fetch_add(a.cnt + strip, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
            prev = __shfl(prev, 0);
            if (prev == ncontrib - 1) {
                __threadfence();
                v4f sum = {0.0f, 0.0f, 0.0f, 0.0f};
                const float* s0 = a.part + (strip * a.maxc * 64 + lane) * 4;
                for (int64_t c = 0; c < ncontrib; ++c) {
                    const v4f p = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(s0 + c * 256));
                    sum += p;
                }
                store_y(a, sum, n0, lane);
                if (lane == 0) __hip_atomic_store(a.cnt + strip, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        u = strip * a.KB + kb1;
    }
}

static int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

DecodePlan plan_decode(int64_t M, int64_t N, int64_t K, int cus, bool allow_split) {
    (void)M;
    DecodePlan p{};
    p.strips = N / 16;
    p.kblocks = K / kGroup;
    p.units = p.strips * p.kblocks;
    const int64_t target = (int64_t)(cus > 0 ? cus : 256) * kDecodeWavesPerCU;
    if (!allow_split || p.strips >= target || p.strips > kMaxSplitStrips || p.units == 0) {
        p.workers = p.strips;
        p.base = p.kblocks;
        p.rem = 0;
        p.max_contrib = 1;
        p.split = false;
    } else {
        p.workers = p.units < target ? p.units : target;
        p.base = p.units / p.workers;
        p.rem = p.units % p.workers;
        p.split = !(p.rem == 0 && p.base % p.kblocks == 0);
        p.max_contrib = p.split ? (p.kblocks + p.base - 1) / p.base + 1 : 1;
    }
    p.part_bytes = p.split ? (size_t)align256(p.strips * p.max_contrib * 1024) : 0;
    p.cnt_bytes = p.split ? (size_t)kCounterBytes : 0;
    return p;
}

size_t decode_workspace_bytes(const DecodePlan& p) { return p.split ? kCounterBytes + p.part_bytes : 0; }

hipError_t launch_gemm_decode(const DecodePlan& plan, const void* q, const float* s, const void* w,
                              const float* ws, void* y, int64_t M, int64_t N, int64_t K,
                              void* workspace, hipStream_t st) {
    if (plan.workers == 0) return hipSuccess;
    DecodeArgs a;
    a.w = (const uint8_t*)w;
    a.ws = ws;
    a.x = (const uint8_t*)q;
    a.xs = s;
    a.y = (uint16_t*)y;
    // Counters first, at a fixed place: a later call of another shape never finds
    // its counters inside an earlier call's partial sums.
    a.cnt = plan.split ? (int*)workspace : nullptr;
    a.part = plan.split ? (float*)((char*)workspace + kCounterBytes) : nullptr;
    a.M = (int)M;
    a.N = N;
    a.K = K;
    a.KB = plan.kblocks;
    a.workers = plan.workers;
    a.base = plan.base;
    a.rem = plan.rem;
    a.maxc = plan.max_contrib;
    const int64_t per_block = kDecodeThreads / 64;
    const int64_t blocks = (plan.workers + per_block - 1) / per_block;
    hipLaunchKernelGGL(gemm_decode_kernel, dim3((unsigned)blocks), dim3(kDecodeThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace fp8bs
