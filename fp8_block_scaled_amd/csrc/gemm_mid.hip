// Block-scaled FP8 GEMM for mid-size M (16 < M <= 64) on gfx950.
//
// y[m, n] = sum_kb (s[m, kb] * ws[n/128, kb]) * sum_{k in kb} q[m, k] * w[n, k]
// ("Nanbeige4.3-33B FP8" model card, introduction: E4M3 weights in 128x128 blocks,
// dynamic per-token group-128 activation scales; FP32 accumulation, BF16 out).
//
// Batched decode and short prompts (up to a few tens of tokens) are still bound by
// the weight stream (2 M flop per weight byte, far below the MFMA ridge), but a
// 16-token MFMA group no longer holds them.  The kernel streams the weights like
// the decode kernel -- one workgroup per NS strips of 16 output columns, the K
// blocks split over its S waves, partial sums added through LDS in a fixed order
// (deterministic) -- and multiplies each 16 x 128 weight fragment by the R 16-token
// groups of the activations (R = 2, 4 or 8; rows past M are loaded from row M - 1
// and not stored):
//   v_mfma_f32_16x16x128_f8f6f4, A = 16 weight rows (the strip), B = 16 token rows,
//   one MFMA per (strip, token group) and K block, each promoted by its own
//   scales (acc += s[m, kb] * ws[nb, kb] * P).
// Activation codes come from L2: every workgroup reads all M x K of them, R KiB per
// wave and K block, against 2 KiB of weights per strip.
// Operand layout per lane l (g = l / 16, r = l % 16): A row r = weight row 16 st + r,
// B column r = token row 16 rho + r, both K-block bytes [16 g, 16 g + 16) and
// [64 + 16 g, 64 + 16 g + 16).  Result lane l holds C[4 g + e][r], e = 0..3: output
// column 16 st + 4 g + e, token row 16 rho + r.
#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace fp8bs {

constexpr int kMidMaxWaves = 8;
constexpr int kMidWaves = 8;

struct MidArgs {
    const uint8_t* w;
    const float* ws;
    const uint8_t* x;
    const float* xs;
    uint16_t* y;
    int M;
    int64_t N, K, KB;
    int64_t strips;                          // N / 16
};

template <int R, int NS>
__global__ __launch_bounds__(kMidMaxWaves * 64) void gemm_mid_kernel(MidArgs a) {
    extern __shared__ __attribute__((aligned(16))) v4f red[];      // [S][NS][R][64] partial sums
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int64_t strip0 = (int64_t)blockIdx.x * NS;
    const int64_t kb0 = (wave * a.KB) / S;
    const int64_t kb1 = ((wave + 1) * a.KB) / S;

    const uint8_t* xrow[R];
    const float* xsrow[R];
#pragma unroll
    for (int rho = 0; rho < R; ++rho) {
        const int m = 16 * rho + r < a.M ? 16 * rho + r : a.M - 1;
        xrow[rho] = a.x + (int64_t)m * a.K + 16 * g;
        xsrow[rho] = a.xs + (int64_t)m * a.KB;
    }
    // Weight loads read whole 128-byte lines, as in the decode kernel: lanes r and
    // r ^ 8 are partners; the first load of lane r takes chunk c = g + 4 hh (hh = r / 8)
    // of strip row r ^ 8 hh, the second chunk c of the other partner's row, and a DPP
    // exchange leaves chunks g and g + 4 of row r in every lane.  The loads are
    // nontemporal (the weight stream is read once).
    const int hh = r >> 3;
    const int rowA = r ^ (8 * hh), rowB = rowA ^ 8;
    const int cw = 16 * (g + 4 * hh);
    const uint8_t* wrowA[NS];
    const uint8_t* wrowB[NS];
    const float* wsrow[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        // Strips past the last one (a partial final workgroup) re-read the last
        // strip; their results are not stored.
        const int64_t st = strip0 + q < a.strips ? strip0 + q : a.strips - 1;
        wrowA[q] = a.w + (st * 16 + rowA) * a.K + cw;
        wrowB[q] = a.w + (st * 16 + rowB) * a.K + cw;
        wsrow[q] = a.ws + ((st * 16) / kGroup) * a.KB;
    }

    v4f acc[NS][R];
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
        for (int rho = 0; rho < R; ++rho) acc[q][rho] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // Fragments and scales of one K block; with R <= 4 the next block's are
    // requested before this one's MFMAs (two K blocks in flight per wave).
    struct Frag {
        v4i wv[NS][2], xv[R][2];
        float wsv[NS], xsv[R];
    };
    auto load = [&](Frag& f, int64_t kb) {
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            f.wv[q][0] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrowA[q] + kb * kGroup));
            f.wv[q][1] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrowB[q] + kb * kGroup));
            f.wsv[q] = wsrow[q][kb];
        }
#pragma unroll
        for (int rho = 0; rho < R; ++rho) {
            const v4i* xp = reinterpret_cast<const v4i*>(xrow[rho] + kb * kGroup);
            f.xv[rho][0] = xp[0];
            f.xv[rho][1] = xp[4];
            f.xsv[rho] = xsrow[rho][kb];
        }
    };
    auto compute = [&](const Frag& f) {
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            // The partner exchange (DPP row_ror:8 swaps lanes r and r ^ 8 of each row).
            const v4i la = f.wv[q][0], lb = f.wv[q][1];
            const v4i snd = hh ? la : lb;
            v4i rcv;
            rcv.x = __builtin_amdgcn_update_dpp(0, snd.x, 0x128, 0xF, 0xF, false);
            rcv.y = __builtin_amdgcn_update_dpp(0, snd.y, 0x128, 0xF, 0xF, false);
            rcv.z = __builtin_amdgcn_update_dpp(0, snd.z, 0x128, 0xF, 0xF, false);
            rcv.w = __builtin_amdgcn_update_dpp(0, snd.w, 0x128, 0xF, 0xF, false);
            const v4i lo = hh ? rcv : la, hi = hh ? lb : rcv;          // chunks g and g + 4
            const v8i av = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int rho = 0; rho < R; ++rho) {
                const v8i bv = {f.xv[rho][0].x, f.xv[rho][0].y, f.xv[rho][0].z, f.xv[rho][0].w,
                                f.xv[rho][1].x, f.xv[rho][1].y, f.xv[rho][1].z, f.xv[rho][1].w};
                // Format 0 = E4M3 for both operands; zero scale operands select the unscaled MFMA.
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, zero, 0, 0, 0, 0, 0, 0);
                const float sc = f.xsv[rho] * f.wsv[q];
                acc[q][rho][0] = fmaf(sc, p[0], acc[q][rho][0]);
                acc[q][rho][1] = fmaf(sc, p[1], acc[q][rho][1]);
                acc[q][rho][2] = fmaf(sc, p[2], acc[q][rho][2]);
                acc[q][rho][3] = fmaf(sc, p[3], acc[q][rho][3]);
            }
        }
    };
    // Eight token groups leave no registers for a second block in flight.
    constexpr bool kTwoInFlight = R <= 4;
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
    // Output element o = ((q R + rho) 64 + l) 4 + e: the sum over waves of component e
    // of lane l's partial for strip q and token group rho.
    for (int o = threadIdx.x; o < NS * R * 256; o += blockDim.x) {
        const int e = o & 3, l = (o >> 2) & 63, qr = o >> 8;
        const int q = qr / R, rho = qr % R;
        const int m = 16 * rho + (l & 15);
        if (m >= a.M || strip0 + q >= a.strips) continue;
        float sum = 0.0f;
        for (int w = 0; w < S; ++w) sum += red[((w * NS + q) * R + rho) * 64 + l][e];
        const int64_t n = (strip0 + q) * 16 + 4 * (l >> 4) + e;
        a.y[(int64_t)m * a.N + n] = (uint16_t)f32_to_bf16_rne(sum);
    }
}

MidPlan plan_mid(int64_t M, int64_t N, int64_t K, int cus) {
    MidPlan p{};
    p.groups = M <= 32 ? 2 : (M <= 64 ? 4 : 8);          // 8 only through kMidMaxM changes
    p.strips = N / 16;
    p.kblocks = K / kGroup;
    // Strips per workgroup: every workgroup reads all 16 R activation rows (from L2)
    // plus 16 weight rows per strip, and a CU holds several workgroups at once, so the
    // busiest CU moves ceil(workgroups / CUs) (16 R + 16 NS) K bytes.  NS minimizes
    // that (ties to the larger NS: less L2 traffic in total).  Measured at K = 7168,
    // M = 17 .. 32: N = 7168 takes NS = 2 (16.3 .. 19.9 us, against 21 .. 28 with one
    // strip), N = 9216 and 16384 take NS = 4 (23 .. 29 us, against 30 .. 53).
    // NS = 4 only with R = 2 (registers), NS = 2 with R <= 4.
    {
        const int max_ns = p.groups <= 2 ? 4 : (p.groups <= 4 ? 2 : 1);
        int64_t best = -1;
        for (int ns = 1; ns <= max_ns; ns *= 2) {
            const int64_t wgs = (p.strips + ns - 1) / ns;
            const int64_t per_cu = (wgs + cus - 1) / cus;
            const int64_t bytes = per_cu * (p.groups + ns);
            if (best < 0 || bytes <= best) {
                best = bytes;
                p.strips_per_wg = ns;
            }
        }
    }
    if (const char* e = getenv("FP8BS_MID_STRIPS")) {       // tuning hook (4 only with R = 2, 2 with R <= 4)
        const int v = atoi(e);
        if (v == 1 || (v == 2 && p.groups <= 4) || (v == 4 && p.groups <= 2)) p.strips_per_wg = v;
    }
    p.workgroups = (p.strips + p.strips_per_wg - 1) / p.strips_per_wg;
    p.waves = (int)(p.kblocks < kMidWaves ? p.kblocks : kMidWaves);
    if (const char* e = getenv("FP8BS_MID_WAVES")) {        // tuning hook
        const int v = atoi(e);
        if (v >= 1 && v <= kMidMaxWaves) p.waves = v;
    }
    return p;
}

template <int R, int NS>
static hipError_t launch_rns(dim3 grid, dim3 block, unsigned lds, hipStream_t st, const MidArgs& a) {
    // More than 64 KiB of LDS (more waves or token groups) needs the per-kernel limit
    // raised, up to the CU's 160 KiB.
    static std::atomic<uint64_t> raised{0};
    if (lds > 65536) {
        const hipError_t e = raise_lds_limit((const void*)gemm_mid_kernel<R, NS>, raised, 160 * 1024);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gemm_mid_kernel<R, NS>), grid, block, lds, st, a);
    return hipSuccess;
}

template <int R>
static hipError_t launch_r(const MidPlan& plan, dim3 grid, dim3 block, unsigned lds, hipStream_t st,
                           const MidArgs& a) {
    if (R <= 2 && plan.strips_per_wg == 4) return launch_rns<R, R <= 2 ? 4 : 1>(grid, block, lds, st, a);
    if (R <= 4 && plan.strips_per_wg == 2) return launch_rns<R, R <= 4 ? 2 : 1>(grid, block, lds, st, a);
    return launch_rns<R, 1>(grid, block, lds, st, a);
}

hipError_t launch_gemm_mid(const MidPlan& plan, const void* q, const float* s, const void* w, const float* ws,
                           void* y, int64_t M, int64_t N, int64_t K, hipStream_t st) {
    if (plan.workgroups == 0) return hipSuccess;
    MidArgs a;
    a.w = (const uint8_t*)w;
    a.ws = ws;
    a.x = (const uint8_t*)q;
    a.xs = s;
    a.y = (uint16_t*)y;
    a.M = (int)M;
    a.N = N;
    a.K = K;
    a.KB = plan.kblocks;
    a.strips = plan.strips;
    const dim3 grid((unsigned)plan.workgroups), block(plan.waves * 64);
    const unsigned lds = (unsigned)(plan.waves * plan.strips_per_wg * plan.groups * 64 * sizeof(v4f));
    hipError_t e;
    switch (plan.groups) {
        case 2: e = launch_r<2>(plan, grid, block, lds, st, a); break;
        case 4: e = launch_r<4>(plan, grid, block, lds, st, a); break;
        default: e = launch_r<8>(plan, grid, block, lds, st, a); break;
    }
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace fp8bs
