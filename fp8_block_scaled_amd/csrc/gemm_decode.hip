// Decode-shape block-scaled FP8 GEMM (M <= 16) for gfx950.
//
// y[m, n] = sum_kb (s[m, kb] * ws[n/128, kb]) * sum_{k in kb} q[m, k] * w[n, k]
// ("Nanbeige4.3-33B FP8" model card, introduction: E4M3 weights in 128x128 blocks,
// dynamic per-token group-128 activation scales; FP32 accumulation, BF16 out).
//
// At M <= 16 the weight stream is ~all of the traffic (arithmetic intensity
// 2..32 flop/B), so the kernel is built to keep HBM busy on every CU:
//   * K-blocks folded into the MFMA.  v_mfma_f32_16x16x128_f8f6f4 multiplies 16
//     rows of A by 16 columns of B over one 128-wide K block.  With M <= P (P = 4,
//     8 or 16) the 16 rows and columns are split into G = 16 / P groups of P: group
//     t of A holds the P weight rows of this strip at K block kbase + t, group t of
//     B the P token rows at the same K block.  The diagonal P x P blocks of the
//     16 x 16 result are then G independent K-block products, each promoted by its
//     own scales; the off-diagonal blocks are discarded.  A strip is P output
//     columns, so decode shapes give many strips: the work per CU stays even (a CU
//     that receives one strip more than another would set the kernel's time: a
//     CU's own bandwidth is limited).
//   * Split-K inside a workgroup: one workgroup per strip, its S waves take equal
//     contiguous ranges of "super blocks" (G K blocks each), and the partial sums
//     over waves and groups are added through LDS in a fixed order
//     (deterministic).  Partial sums never leave the workgroup: a reduction across
//     workgroups would need agent-scope release / acquire, which on this part is
//     a write-back / invalidate of the XCD's L2.
//   * Each workgroup owns NS adjacent strips; each wave loads one activation
//     fragment per super block and uses it for the NS strips' MFMAs.  Every
//     workgroup reads the whole M x K activation codes (from L2), so NS trades
//     activation traffic against the number of workgroups.
//   * Each lane requests the fragments and scales of CH super blocks at a time.
//     The weight scale index is made wave-uniform.
//
// Operand layout per lane l (g = l / 16, r = l % 16, row rr = r % P, group
// tb = r / P): A row r = weight row n0 + rr at K block kbase + tb; B column r =
// token row rr at the same K block; both take K-block bytes [16 g, 16 g + 16) and
// [64 + 16 g, 64 + 16 g + 16) (any assignment of K bytes to register slots that
// is the same for A and B gives the same dot product).  The result lane l holds
// C[4 g + e][r], e = 0..3: A row i = 4 g + e is weight row n0 + i % P of group
// i / P, so the lane is on a diagonal block exactly when 4 g / P == tb.
#include <climits>
#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace fp8bs {

constexpr int kDecodeMaxWaves = 16;
// Workgroup shape, from measurement on the decode shapes (M = 1 and 8, K = 7168
// and 8192, N = 7168..16384): 8 waves per workgroup and 2 strips per workgroup
// gave the shortest times; fewer waves leave a CU short of loads in flight, more
// strips per workgroup leave too few workgroups to spread evenly over the CUs.
constexpr int kWavesPerWg = 8;
constexpr int kStripsPerWg = 2;

struct DecodeArgs {
    const uint8_t* w;
    const float* ws;
    const uint8_t* x;
    const float* xs;
    uint16_t* y;
    int M;
    int64_t N, K, KB;
    int64_t strips;                          // N / P
};

template <int P, int NS>
__global__ __launch_bounds__(kDecodeMaxWaves * 64) void gemm_decode_kernel(DecodeArgs a) {
    constexpr int G = 16 / P;
    constexpr int CH = NS <= 2 ? 2 : 1;      // super blocks per load batch
    extern __shared__ __attribute__((aligned(16))) v4f red[];      // [S][NS][64] partial sums
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int rr = r % P, tb = r / P;
    const bool mvalid = rr < a.M;
    const int64_t strip0 = (int64_t)blockIdx.x * NS;
    const int64_t SKB = (a.KB + G - 1) / G;
    const int64_t sb0 = (wave * SKB) / S;
    const int64_t sb1 = ((wave + 1) * SKB) / S;
    const uint8_t* xrow = a.x + (mvalid ? rr : 0) * a.K + 16 * g;
    const float* xsrow = a.xs + (mvalid ? rr : 0) * a.KB;
    const uint8_t* wrow[NS];
    const float* wsrow[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        // Strips past the last one (a partial final workgroup) re-read the last
        // strip; their results are not stored.
        const int64_t st = strip0 + q < a.strips ? strip0 + q : a.strips - 1;
        wrow[q] = a.w + (st * P + rr) * a.K + 16 * g;
        wsrow[q] = a.ws + ((st * P) / kGroup) * a.KB;
    }

    // A batch: fragments and scales of up to CH super blocks, requested before any
    // is used.  Branch-free: K blocks past KB (a last, partial super block) are
    // clamped to valid addresses and zeroed at use.
    v4i wv[CH][NS][2], xv[CH][2];
    float xsv[CH], wsv[CH][NS];
    auto load_batch = [&](int64_t sb) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            int64_t k = (sb + i) * G + tb;
            k = k < a.KB ? k : a.KB - 1;
            const v4i* xp = reinterpret_cast<const v4i*>(xrow + k * kGroup);
            xv[i][0] = xp[0];
            xv[i][1] = xp[4];
            xsv[i] = xsrow[k];
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                const v4i* wp = reinterpret_cast<const v4i*>(wrow[q] + k * kGroup);
                wv[i][q][0] = wp[0];
                wv[i][q][1] = wp[4];
                wsv[i][q] = wsrow[q][k];
            }
        }
    };

    v4f acc[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) acc[q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const v4i z4 = {0, 0, 0, 0};
    for (int64_t sb = sb0; sb < sb1; sb += CH) {
        load_batch(sb);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            if (sb + i < sb1) {                                  // uniform
                const bool use = mvalid && (sb + i) * G + tb < a.KB;
                const v4i b0 = use ? xv[i][0] : z4, b1 = use ? xv[i][1] : z4;
                const v8i bv = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
                const float xsc = use ? xsv[i] : 0.0f;
#pragma unroll
                for (int q = 0; q < NS; ++q) {
                    const v8i av = {wv[i][q][0].x, wv[i][q][0].y, wv[i][q][0].z, wv[i][q][0].w,
                                    wv[i][q][1].x, wv[i][q][1].y, wv[i][q][1].z, wv[i][q][1].w};
                    // Format 0 = E4M3 for both operands; zero scale operands select the unscaled MFMA.
                    const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, zero, 0, 0, 0, 0, 0, 0);
                    const float sc = xsc * wsv[i][q];
                    acc[q][0] = fmaf(sc, p[0], acc[q][0]);
                    acc[q][1] = fmaf(sc, p[1], acc[q][1]);
                    acc[q][2] = fmaf(sc, p[2], acc[q][2]);
                    acc[q][3] = fmaf(sc, p[3], acc[q][3]);
                }
            }
        }
    }

#pragma unroll
    for (int q = 0; q < NS; ++q) red[(wave * NS + q) * 64 + lane] = acc[q];
    __syncthreads();
    // Output (m, c) of strip q: sum over waves, then over the G groups, of the
    // diagonal-block entry C[t P + c][t P + m], held by lane 16 ((t P + c) / 4) +
    // t P + m in its component c % 4.
    if (wave == 0) {
        for (int o = lane; o < NS * a.M * P; o += 64) {
            const int q = o / (a.M * P), rem = o % (a.M * P);
            const int m = rem / P, c = rem % P;
            if (strip0 + q >= a.strips) continue;
            float sum = 0.0f;
            for (int w = 0; w < S; ++w) {
#pragma unroll
                for (int t = 0; t < G; ++t) {
                    const int src = 16 * ((t * P + c) >> 2) + t * P + m;
                    sum += red[(w * NS + q) * 64 + src][c & 3];
                }
            }
            a.y[m * a.N + (strip0 + q) * P + c] = (uint16_t)f32_to_bf16_rne(sum);
        }
    }
}

// Row-group size for M tokens: the smallest of 4, 8, 16 that holds them.
static int choose_rows(int64_t M) { return M <= 4 ? 4 : (M <= 8 ? 8 : 16); }

DecodePlan plan_decode(int64_t M, int64_t N, int64_t K, int cus) {
    DecodePlan p{};
    p.rows = choose_rows(M);
    (void)cus;
    p.strips_per_wg = kStripsPerWg;
    if (const char* e = getenv("FP8BS_DECODE_STRIPS")) {    // tuning hook
        const int v = atoi(e);
        if (v >= 1 && v <= 4) p.strips_per_wg = v;
    }
    p.strips = N / p.rows;
    p.workgroups = (p.strips + p.strips_per_wg - 1) / p.strips_per_wg;
    p.kblocks = K / kGroup;
    const int64_t super_blocks = (p.kblocks + (16 / p.rows) - 1) / (16 / p.rows);
    p.waves = (int)(super_blocks < kWavesPerWg ? super_blocks : kWavesPerWg);
    if (const char* e = getenv("FP8BS_DECODE_WAVES")) {     // tuning hook
        const int v = atoi(e);
        if (v >= 1 && v <= kDecodeMaxWaves) p.waves = v;
    }
    return p;
}

template <int P>
static void launch_p(const DecodePlan& plan, dim3 grid, dim3 block, unsigned lds, hipStream_t st, const DecodeArgs& a) {
    switch (plan.strips_per_wg) {
        case 1: hipLaunchKernelGGL((gemm_decode_kernel<P, 1>), grid, block, lds, st, a); break;
        case 2: hipLaunchKernelGGL((gemm_decode_kernel<P, 2>), grid, block, lds, st, a); break;
        case 3: hipLaunchKernelGGL((gemm_decode_kernel<P, 3>), grid, block, lds, st, a); break;
        default: hipLaunchKernelGGL((gemm_decode_kernel<P, 4>), grid, block, lds, st, a); break;
    }
}

hipError_t launch_gemm_decode(const DecodePlan& plan, const void* q, const float* s, const void* w,
                              const float* ws, void* y, int64_t M, int64_t N, int64_t K, hipStream_t st) {
    if (plan.workgroups == 0) return hipSuccess;
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
    a.strips = plan.strips;
    const dim3 grid((unsigned)plan.workgroups), block(plan.waves * 64);
    const unsigned lds = (unsigned)(plan.waves * plan.strips_per_wg * 64 * sizeof(v4f));
    switch (plan.rows) {
        case 4: launch_p<4>(plan, grid, block, lds, st, a); break;
        case 8: launch_p<8>(plan, grid, block, lds, st, a); break;
        default: launch_p<16>(plan, grid, block, lds, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace fp8bs
