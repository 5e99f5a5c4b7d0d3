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
//   * Split-K inside a workgroup: one workgroup per NS strips, its S waves split the
//     "super blocks" (G K blocks each) evenly -- as contiguous ranges, or interleaved
//     (wave w takes w, w + S, ...: at any moment the workgroup reads one stretch of
//     each weight row), chosen per shape -- and the partial sums over waves and
//     groups are added through LDS in a fixed order (deterministic).  Partial sums never leave the workgroup: a reduction across
//     workgroups would need agent-scope release / acquire, which on this part is
//     a write-back / invalidate of the XCD's L2, or a second kernel (measured
//     slower than the imbalance it removes).
//   * Each workgroup owns NS adjacent strips; each wave loads one activation
//     fragment per super block and uses it for the NS strips' MFMAs.  Every
//     workgroup reads the whole M x K activation codes (from L2), so NS trades
//     activation traffic against the number of workgroups; it is chosen per shape
//     so that every CU receives as nearly the same number of strips as possible.
//   * Each lane requests the fragments and scales of CH super blocks (1 by
//     default) before it uses any.  Weight loads read whole cache lines (a DPP
//     exchange between partner lanes restores the operand layout) and are
//     nontemporal; the weight scales of a super block come in one scalar load per
//     strip.
//
// Operand layout per lane l (g = l / 16, r = l % 16, row rr = r % P, group
// tb = r / P): A row r = weight row n0 + rr at K block kbase + tb; B column r =
// token row rr at the same K block; both take K-block bytes [16 g, 16 g + 16) and
// [64 + 16 g, 64 + 16 g + 16) (any assignment of K bytes to register slots that
// is the same for A and B gives the same dot product).  The result lane l holds
// C[4 g + e][r], e = 0..3: A row i = 4 g + e is weight row n0 + i % P of group
// i / P, so the lane is on a diagonal block exactly when 4 g / P == tb.
#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace fp8bs {

typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

// At most 8 waves per workgroup: the launch bound then allows 128+ VGPRs per wave,
// so 4 strips with two super blocks per batch (136 VGPRs) do not spill.  A bound of
// 16 waves capped them at 128 and spilled; the 8-wave bound measured 2.5% faster at
// M = 8, N = 16384, K = 7168 and equal elsewhere.  A 16-wave bound for the one-batch
// kernels alone (which fit 128 registers) was slower at 8 waves (M = 8, N = 7168,
// K = 8192: 13.68 against 13.19-13.26 us) and at 12 or 16 waves on every decode
// workload.
constexpr int kDecodeMaxWaves = 8;
// Workgroup shape, from measurement on the decode shapes (M = 1 and 8, K = 7168
// and 8192, N = 7168..16384): 8 waves per workgroup; fewer leave a CU short of
// loads in flight.  Strips per workgroup (1..4) are chosen per shape in
// plan_decode.
constexpr int kWavesPerWg = 8;
constexpr int kMaxStripsPerWg = 4;

struct DecodeArgs {
    const uint8_t* w;
    const float* ws;
    const uint8_t* x;
    const float* xs;
    uint16_t* y;
    int M;
    int64_t N, K, KB;
    int64_t strips;                          // N / P
    int interleave;                          // 1: wave w takes super blocks w, w + S, ...; 0: a contiguous range
};

template <int P, int NS, int CH>
__global__ __launch_bounds__(kDecodeMaxWaves * 64) void gemm_decode_kernel(DecodeArgs a) {
    constexpr int G = 16 / P;
    extern __shared__ __attribute__((aligned(16))) v4f red[];      // [S][NS][64] partial sums
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int rr = r % P, tb = r / P;
    const bool mvalid = rr < a.M;
    const int64_t strip0 = (int64_t)blockIdx.x * NS;
    const int64_t SKB = (a.KB + G - 1) / G;
    const int64_t sb0 = a.interleave ? wave : (wave * SKB) / S;
    const int64_t sb1 = a.interleave ? SKB : ((wave + 1) * SKB) / S;
    const int64_t sstep = a.interleave ? S : 1;
    const uint8_t* xrow = a.x + (mvalid ? rr : 0) * a.K + 16 * g;
    const float* xsrow = a.xs + (mvalid ? rr : 0) * a.KB;
    // Weight loads read whole 128-byte lines.  Lanes r and r ^ 8 of a 16-lane row
    // are partners (operand rows pair(r) and pair(r ^ 8), pair p = weight row p % P
    // at K block p / P of the super block): the first load of lane r takes chunk
    // c = g + 4 hh (hh = r / 8) of pair r ^ 8 hh, the second chunk c of the other
    // pair, so each load instruction covers 8 lines in full (chunks 0-3 from one
    // partner, 4-7 from the other) instead of 16 halves.  One DPP exchange between
    // partners then leaves every lane with chunks g and g + 4 of its own pair, the
    // layout described above.  With each line requested once, the weight loads are
    // nontemporal: the stream, read once, does not displace the activations and other
    // data in the caches.  (Half-line loads, each line requested by two instructions,
    // lost with nontemporal loads: the second request missed.)  Measured together in
    // one session against half-line temporal loads: M = 1, N = 9216, K = 7168 13.4 ->
    // 12.2 us; M = 8, N = 16384, K = 7168 23.0 -> 21.8 us; M = 8, N = 7168, K = 8192
    // 15.2 -> 14.6 us; whole lines with temporal loads were 0.1-0.5 us slower than
    // half lines.
    const int hh = r >> 3;
    const int pA = r ^ (8 * hh), pB = pA ^ 8;
    const int rowA = pA % P, tbA = pA / P, rowB = pB % P, tbB = pB / P;
    const int cw = 16 * (g + 4 * hh);
    // Strip bases are wave-uniform (scalar registers); the lane's offset within a strip
    // is 32-bit and the same for every strip (below (P + 1) K, so K <= kDecodeMaxK keeps
    // it in range).  Against 64-bit lane addresses per strip: 67 instead of 72 registers
    // with 3 strips, 79 instead of 88 with 4; same-box A/B, two rounds: M = 8, N = 7168,
    // K = 8192 13.28-13.34 against 13.50-13.58 us, M = 8, N = 16384 20.38-20.66 against
    // 20.46-21.76, M = 1, N = 9216 12.11-12.42 against 12.16-12.56.
    const uint8_t* wst[NS];
    const uint32_t offA = (uint32_t)(rowA * a.K + cw), offB = (uint32_t)(rowB * a.K + cw);
    const float* wsrow[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        // Strips past the last one (a partial final workgroup) re-read the last
        // strip; their results are not stored.
        const int64_t st = strip0 + q < a.strips ? strip0 + q : a.strips - 1;
        wst[q] = a.w + st * P * a.K;
        wsrow[q] = a.ws + ((st * P) / kGroup) * a.KB;
    }

    // A batch: fragments and scales of CH super blocks, all requested before any is
    // used.  Branch-free, so that no load is sunk past another super block's MFMAs:
    // a super block past the wave's range re-reads super block sb1 - 1, a K block
    // past KB (a last, partial super block) is clamped to the last K block, and both
    // are zeroed at use.
    v4i wv[CH][NS][2], xv[CH][2];
    // Weight scales: the G K blocks of a super block have consecutive scales in a
    // strip's scale row, at a wave-uniform address, so each strip's G scales come in
    // one scalar load (from K block KB - G for a last, partial super block; the plan
    // keeps KB >= G) and each lane picks its own, wsi.  The vector memory pipeline
    // then carries only the fragments and the activation scales.
    float xsv[CH], wsg[CH][NS][G];
    int wsi[CH];
    auto load_batch = [&](int64_t sb) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int64_t sbi = sb + i * sstep < sb1 ? sb + i * sstep : sb1 - 1;
            int64_t k = sbi * G + tb, kA = sbi * G + tbA, kB = sbi * G + tbB;
            k = k < a.KB ? k : a.KB - 1;
            kA = kA < a.KB ? kA : a.KB - 1;
            kB = kB < a.KB ? kB : a.KB - 1;
            const int64_t wbase = sbi * G + G <= a.KB ? sbi * G : a.KB - G;
            wsi[i] = (int)(k - wbase);
            const v4i* xp = reinterpret_cast<const v4i*>(xrow + k * kGroup);
            xv[i][0] = xp[0];
            xv[i][1] = xp[4];
            xsv[i] = xsrow[k];
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                wv[i][q][0] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4i*>(wst[q] + (offA + (uint32_t)kA * (uint32_t)kGroup)));
                wv[i][q][1] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4i*>(wst[q] + (offB + (uint32_t)kB * (uint32_t)kGroup)));
                if constexpr (G == 4) {
                    const f32x4_a4 v = *reinterpret_cast<const f32x4_a4*>(wsrow[q] + wbase);
                    wsg[i][q][0] = v[0];
                    wsg[i][q][1] = v[1];
                    wsg[i][q][2] = v[2];
                    wsg[i][q][3] = v[3];
                } else if constexpr (G == 2) {
                    const f32x2_a4 v = *reinterpret_cast<const f32x2_a4*>(wsrow[q] + wbase);
                    wsg[i][q][0] = v[0];
                    wsg[i][q][1] = v[1];
                } else {
                    wsg[i][q][0] = wsrow[q][wbase];
                }
            }
        }
    };

    v4f acc[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) acc[q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const v4i z4 = {0, 0, 0, 0};
    for (int64_t sb = sb0; sb < sb1; sb += CH * sstep) {
        load_batch(sb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const bool use = mvalid && sb + i * sstep < sb1 && (sb + i * sstep) * G + tb < a.KB;
            const v4i b0 = use ? xv[i][0] : z4, b1 = use ? xv[i][1] : z4;
            const v8i bv = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            const float xsc = use ? xsv[i] : 0.0f;
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                // The partner exchange: send the chunk that belongs to the partner, keep
                // the own one (DPP row_ror:8 swaps lanes r and r ^ 8 of each row).
                const v4i la = wv[i][q][0], lb = wv[i][q][1];
                const v4i snd = hh ? la : lb;
                v4i rcv;
                rcv.x = __builtin_amdgcn_update_dpp(0, snd.x, 0x128, 0xF, 0xF, false);
                rcv.y = __builtin_amdgcn_update_dpp(0, snd.y, 0x128, 0xF, 0xF, false);
                rcv.z = __builtin_amdgcn_update_dpp(0, snd.z, 0x128, 0xF, 0xF, false);
                rcv.w = __builtin_amdgcn_update_dpp(0, snd.w, 0x128, 0xF, 0xF, false);
                const v4i lo = hh ? rcv : la, hi = hh ? lb : rcv;      // chunks g and g + 4
                const v8i av = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                // Format 0 = E4M3 for both operands; zero scale operands select the unscaled MFMA.
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, zero, 0, 0, 0, 0, 0, 0);
                float wsl = wsg[i][q][0];
#pragma unroll
                for (int t = 1; t < G; ++t) wsl = wsi[i] == t ? wsg[i][q][t] : wsl;
                const float sc = xsc * wsl;
                acc[q][0] = fmaf(sc, p[0], acc[q][0]);
                acc[q][1] = fmaf(sc, p[1], acc[q][1]);
                acc[q][2] = fmaf(sc, p[2], acc[q][2]);
                acc[q][3] = fmaf(sc, p[3], acc[q][3]);
            }
        }
    }

#pragma unroll
    for (int q = 0; q < NS; ++q) red[(wave * NS + q) * 64 + lane] = acc[q];
    __syncthreads();
    // Output (m, c) of strip q: sum over waves, then over the G groups, of the
    // diagonal-block entry C[t P + c][t P + m], held by lane 16 ((t P + c) / 4) +
    // t P + m in its component c % 4.  Every thread of the workgroup takes outputs:
    // each output is still summed by one thread in a fixed order.
    {
        for (int o = threadIdx.x; o < NS * a.M * P; o += blockDim.x) {
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

int64_t decode_max_k() {
    if (const char* e = getenv("FP8BS_DECODE_MAX_K")) {     // test hook: route longer rows to the mid-size kernel
        const long long v = atoll(e);
        if (v > 0 && v < kDecodeMaxK) return v;
    }
    return kDecodeMaxK;
}

// Row-group size for M tokens: the smallest of 4, 8, 16 that holds them.
static int choose_rows(int64_t M) { return M <= 4 ? 4 : (M <= 8 ? 8 : 16); }

DecodePlan plan_decode(int64_t M, int64_t N, int64_t K, int cus) {
    DecodePlan p{};
    p.rows = choose_rows(M);
    while (16 / p.rows > K / kGroup) p.rows *= 2;          // KB >= G: a super block fits in K
    p.strips = N / p.rows;
    // Measured at M = 1, N = 9216, K = 7168 (2304 strips of 4): NS = 3 (9 strips on
    // every CU) 13.4 us, NS = 2 (up to 10) 13.8 us, NS = 4 (up to 12) 15.9 us; at
    // M = 8, N = 16384 NS = 1, 2, 3, 4 took 36.3, 25.5, 26.7, 23.6 us.
    p.strips_per_wg = decode_strips_per_wg(p.strips, cus, p.rows * K, M * K, kMaxStripsPerWg);
    if (const char* e = getenv("FP8BS_DECODE_STRIPS")) {    // tuning hook
        const int v = atoi(e);
        if (v >= 1 && v <= kMaxStripsPerWg) p.strips_per_wg = v;
    }
    p.workgroups = (p.strips + p.strips_per_wg - 1) / p.strips_per_wg;
    p.kblocks = K / kGroup;
    const int64_t super_blocks = (p.kblocks + (16 / p.rows) - 1) / (16 / p.rows);
    p.waves = (int)(super_blocks < kWavesPerWg ? super_blocks : kWavesPerWg);
    if (const char* e = getenv("FP8BS_DECODE_WAVES")) {     // tuning hook
        const int v = atoi(e);
        if (v >= 1 && v <= kDecodeMaxWaves) p.waves = v;
    }
    // One super block per load batch: with whole-line nontemporal weight loads the
    // batch of two was slower on every decode shape measured (M = 8, N = 7168,
    // K = 8192, NS = 4: 14.4 against 13.9 us; M = 1, N = 9216, K = 7168, NS = 3: 13.0
    // against 12.2 us).  Batches of two stay reachable through the tuning hook.
    p.batch = 1;
    if (const char* e = getenv("FP8BS_DECODE_BATCH")) {     // tuning hook
        const int v = atoi(e);
        if (v >= 1 && v <= 2) p.batch = v;
    }
    // Interleaved super blocks, except where a weight row is a multiple of 8 KiB.
    // Same-session rounds on three boxes (graph-timed, 8 waves): q/k/v (K = 7168)
    // 12.07-12.17 / 12.09-12.13 / 12.28-12.29 against 12.21-12.22 / 12.25-12.30 /
    // 12.43-12.51 us contiguous; gate/up (K = 7168) 20.42-20.49 / 20.57 / 20.88-20.94
    // against 20.9-21.2 / 20.94-21.27 / 21.28-21.48; down (K = 8192) 15.2 / 15.0-15.1 /
    // 14.7-14.8 against 13.3 / 13.2-13.3 / 13.4 (slower at every wave count tried,
    // 3-8; visiting each workgroup's super blocks in a rotated order was slower still).
    p.interleave = (K % 8192) != 0;
    if (const char* e = getenv("FP8BS_DECODE_INTERLEAVE")) p.interleave = atoi(e) != 0;   // tuning hook
    return p;
}

template <int P>
static void launch_p(const DecodePlan& plan, dim3 grid, dim3 block, unsigned lds, hipStream_t st, const DecodeArgs& a) {
    switch (plan.strips_per_wg * 10 + plan.batch) {
        case 11: hipLaunchKernelGGL((gemm_decode_kernel<P, 1, 1>), grid, block, lds, st, a); break;
        case 12: hipLaunchKernelGGL((gemm_decode_kernel<P, 1, 2>), grid, block, lds, st, a); break;
        case 21: hipLaunchKernelGGL((gemm_decode_kernel<P, 2, 1>), grid, block, lds, st, a); break;
        case 22: hipLaunchKernelGGL((gemm_decode_kernel<P, 2, 2>), grid, block, lds, st, a); break;
        case 31: hipLaunchKernelGGL((gemm_decode_kernel<P, 3, 1>), grid, block, lds, st, a); break;
        case 32: hipLaunchKernelGGL((gemm_decode_kernel<P, 3, 2>), grid, block, lds, st, a); break;
        case 41: hipLaunchKernelGGL((gemm_decode_kernel<P, 4, 1>), grid, block, lds, st, a); break;
        default: hipLaunchKernelGGL((gemm_decode_kernel<P, 4, 2>), grid, block, lds, st, a); break;
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
    a.interleave = plan.interleave;
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
