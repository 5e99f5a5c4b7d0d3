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
//   * Split-K inside a workgroup: one workgroup per 16-column strip, its S waves
//     take S equal contiguous K ranges, and wave 0 adds the S partial sums from
//     LDS in wave order (deterministic).  Partial sums never leave the
//     workgroup: a reduction across workgroups would need agent-scope release /
//     acquire, which on this part is a write-back / invalidate of the XCD's L2.
//   * S is chosen per shape so that all workgroups are resident at once and every
//     wave streams about the same number of weight bytes.
//   * Each lane loads 2 x 16 bytes of its weight row per K block, 4 K blocks at a
//     time (32 VGPRs).  At ~60 VGPRs a CU holds 32 waves, so the workgroups of
//     every decode shape (up to 1024 strips of up to 8 waves) are resident at once
//     and no second, mostly idle round of workgroups is needed.
//   * Each wave stages its own K slice of the M x K activation codes (at most a
//     few tens of KB in all at decode) in LDS with direct global -> LDS loads (no
//     VGPRs) while its weight loads are in flight, then reads its B fragments from
//     LDS.  The waves never wait for each other until the final reduction.  When
//     M x K does not fit LDS the B fragments come straight from global memory (L2).
//   * Both scales of a K block are requested together with its weight fragments;
//     the weight scale is a scalar load (the wave index is made wave-uniform).
//
// Operand layout per lane l (g = l / 16, r = l % 16): A row r = weight row n0 + r,
// B column r = token row r; both take K-block bytes [16 g, 16 g + 16) and
// [64 + 16 g, 64 + 16 g + 16).  The MFMA sums over the K positions of its operand
// registers, so any assignment of K bytes to register slots that is the same for A
// and B gives the same dot product.  Output: lane l holds C[4 g + i][r], i = 0..3,
// i.e. y[m = r][n0 + 4 g + i].
#include <climits>
#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace fp8bs {

constexpr int kDecodeMaxWaves = 16;
constexpr int kChunk = 4;                    // K blocks whose weight loads are in flight together
constexpr int kWaveKBlocks = 8;              // target K blocks per wave
constexpr int kRedBytes = kDecodeMaxWaves * 64 * 16;     // partial sums, aliased onto the staged codes
constexpr int kMaxDynLds = 160 * 1024;

struct DecodeArgs {
    const uint8_t* w;
    const float* ws;
    const uint8_t* x;
    const float* xs;
    uint16_t* y;
    int M;
    int64_t N, K, KB;
};

template <bool kXInLds>
__global__ __launch_bounds__(kDecodeMaxWaves * 64) void gemm_decode_kernel(DecodeArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];    // codes, then partial sums
    v4f* red = reinterpret_cast<v4f*>(xlds);
    const int lane = threadIdx.x & 63;
    // Wave-uniform values are made scalar so that the weight-scale loads are scalar.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const bool mvalid = r < a.M;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t kb0 = (wave * a.KB) / S;
    const int64_t kb1 = ((wave + 1) * a.KB) / S;
    const uint8_t* wrow = a.w + (n0 + r) * a.K + 16 * g;
    const float* wsrow = a.ws + (n0 / kGroup) * a.KB;
    const float* xsrow = a.xs + (mvalid ? r : 0) * a.KB;

    // One chunk: the weight fragments and both scales of up to kChunk K blocks, all
    // requested before any is used.  The loads are branch-free (indices past the
    // wave's range are clamped to its last K block and their results unused), so
    // the compiler issues them back to back without intermediate waits.
    v4i wv[kChunk][2];
    float xsv[kChunk], wsv[kChunk];
    auto load_chunk = [&](int64_t kb) {
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const int64_t k = kb + i < kb1 ? kb + i : kb1 - 1;
            const v4i* p = reinterpret_cast<const v4i*>(wrow + k * kGroup);
            wv[i][0] = p[0];
            wv[i][1] = p[4];
        }
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const int64_t k = kb + i < kb1 ? kb + i : kb1 - 1;
            wsv[i] = wsrow[k];
            xsv[i] = xsrow[k];                       // used only by lanes with mvalid
        }
    };
    // Wave-private staging of this wave's K slice of the activation codes: rows
    // [0, M) x bytes [128 kb0, 128 kb1), stored row-major at LDS offset M * 128 kb0
    // (the slices of the S waves tile the M x K codes).  Direct global -> LDS loads:
    // lane l of an instruction writes LDS bytes [16 l, 16 l + 16) past its base, so
    // one instruction moves 64 consecutive 16-byte pieces of the slice.  Only this
    // wave reads its slice, so no barrier is needed: the wave's own vmcnt wait
    // before the first fragment read covers it.
    const int64_t slice_len = (kb1 - kb0) * kGroup;            // bytes per row
    uint8_t* slice = xlds + (int64_t)a.M * kb0 * kGroup;
    if (kXInLds) {
        const int64_t per_row = slice_len / 16;
        const int64_t pieces = (int64_t)a.M * per_row;
        for (int64_t c0 = 0; c0 < pieces; c0 += 64) {
            const int64_t c = c0 + lane;
            if (c < pieces) {
                const int64_t row = c / per_row, col = c - row * per_row;
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void*)(a.x + row * a.K + kb0 * kGroup + col * 16),
                    (__attribute__((address_space(3))) void*)(slice + c0 * 16), 16, 0, 0);
            }
        }
    }

    int64_t kb = kb0;
    int n = (int)(kb1 - kb < kChunk ? kb1 - kb : kChunk);
    if (n > 0) load_chunk(kb);
    if (kXInLds) {
        // The compiler does not see the LDS side of global_load_lds: wait for it
        // (and the first chunk) explicitly, with a memory clobber so that no LDS
        // read is scheduled above.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    while (n > 0) {
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            if (i < n) {
                const int64_t k = kb + i;
                v4i b0 = {0, 0, 0, 0}, b1 = {0, 0, 0, 0};
                if (mvalid) {
                    const uint8_t* xp = kXInLds ? slice + r * slice_len + (k - kb0) * kGroup + 16 * g
                                                : a.x + r * a.K + k * kGroup + 16 * g;
                    b0 = reinterpret_cast<const v4i*>(xp)[0];
                    b1 = reinterpret_cast<const v4i*>(xp)[4];
                }
                const v8i av = {wv[i][0].x, wv[i][0].y, wv[i][0].z, wv[i][0].w,
                                wv[i][1].x, wv[i][1].y, wv[i][1].z, wv[i][1].w};
                const v8i bv = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                // Format 0 = E4M3 for both operands; zero scale operands select the unscaled MFMA.
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, zero, 0, 0, 0, 0, 0, 0);
                const float sc = (mvalid ? xsv[i] : 0.0f) * wsv[i];
                acc[0] = fmaf(sc, p[0], acc[0]);
                acc[1] = fmaf(sc, p[1], acc[1]);
                acc[2] = fmaf(sc, p[2], acc[2]);
                acc[3] = fmaf(sc, p[3], acc[3]);
            }
        }
        kb += n;
        n = (int)(kb1 - kb < kChunk ? kb1 - kb : kChunk);
        if (n > 0) load_chunk(kb);
    }

    __syncthreads();                        // every wave is done reading the staged codes
    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave == 0) {
        v4f sum = red[lane];
        for (int w = 1; w < S; ++w) sum += red[w * 64 + lane];
        if (mvalid) {
            uint2 o;
            o.x = f32_to_bf16_rne(sum[0]) | (f32_to_bf16_rne(sum[1]) << 16);
            o.y = f32_to_bf16_rne(sum[2]) | (f32_to_bf16_rne(sum[3]) << 16);
            *reinterpret_cast<uint2*>(a.y + r * a.N + n0 + 4 * g) = o;
        }
    }
}

// Waves per workgroup for a decode shape: enough waves that each streams at most
// kWaveKBlocks K blocks, at most 16.
static int choose_waves(int64_t kblocks) {
    int64_t s = (kblocks + kWaveKBlocks - 1) / kWaveKBlocks;
    if (s < 1) s = 1;
    if (s > kDecodeMaxWaves) s = kDecodeMaxWaves;
    return (int)s;
}

DecodePlan plan_decode(int64_t M, int64_t N, int64_t K, int cus) {
    (void)M;
    DecodePlan p{};
    p.strips = N / 16;
    p.kblocks = K / kGroup;
    (void)cus;
    p.waves = choose_waves(p.kblocks);
    if (const char* e = getenv("FP8BS_DECODE_WAVES")) {     // tuning hook
        const int v = atoi(e);
        if (v >= 1 && v <= kDecodeMaxWaves) p.waves = v;
    }
    return p;
}

hipError_t launch_gemm_decode(const DecodePlan& plan, const void* q, const float* s, const void* w,
                              const float* ws, void* y, int64_t M, int64_t N, int64_t K, hipStream_t st) {
    if (plan.strips == 0) return hipSuccess;
    DecodeArgs a;
    a.w = (const uint8_t*)w;
    a.ws = ws;
    a.x = (const uint8_t*)q;
    a.xs = s;
    a.y = (uint16_t*)y;
    a.M = (int)M;
    a.N = N;
    a.K = K;
    a.KB = plan.kblocks;
    const int64_t staged = M * K;
    const int64_t red_bytes = (int64_t)plan.waves * 64 * 16;
    const int64_t lds = staged > red_bytes ? staged : red_bytes;
    if (lds <= kMaxDynLds) {
        if (lds > 64 * 1024) {
            // Allow more than the default 64 KiB of dynamic LDS (idempotent).
            static bool attr_set = false;
            if (!attr_set) {
                hipError_t e = hipFuncSetAttribute((const void*)gemm_decode_kernel<true>,
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, kMaxDynLds);
                if (e != hipSuccess) return e;
                attr_set = true;
            }
        }
        hipLaunchKernelGGL(gemm_decode_kernel<true>, dim3((unsigned)plan.strips), dim3(plan.waves * 64),
                           (unsigned)lds, st, a);
    } else {
        hipLaunchKernelGGL(gemm_decode_kernel<false>, dim3((unsigned)plan.strips), dim3(plan.waves * 64),
                           (unsigned)red_bytes, st, a);
    }
    return hipGetLastError();
}

}  // namespace fp8bs
