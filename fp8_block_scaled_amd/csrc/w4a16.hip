// NVFP4 weight-only linear (W4A16) on gfx950.
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
// Three schedules, by M:
//   M <= 16       w4a16_decode_kernel: K chunks folded into the MFMA, strips of
//                 4 / 8 / 16 output columns, split-K inside the workgroup.
//   16 < M <= 64  w4a16_stream_kernel (below): weights streamed once per workgroup,
//                 each dequantized fragment multiplied by up to 4 token groups.
//   M > 64        w4a16_tile_kernel: LDS-tiled, codes kept in LDS as FP4.
// Every reduction runs in a fixed order: results are bitwise deterministic.
//
// Streaming kernel.  Decode and batched decode (M up to 64) are bound by the weight
// stream: 0.5625 bytes per weight against 2 M flops.  One workgroup takes NS strips
// of 16 output columns; its S waves split the 128-wide K blocks, each wave
// dequantizes a strip's fragment once and multiplies it by R 16-token groups of the
// activations; partial sums are added through LDS in a fixed order.  A second grid
// dimension covers M in chunks of 16 R rows (rows past M are loaded from row M - 1
// and not stored).
//
// Its MFMA operands per lane l (g = l / 16, r = l % 16) and K block kb: the lane
// loads the 16 code bytes [64 kb + 16 g, +16) of weight row 16 st + r, i.e. codes
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
constexpr int64_t kW4StreamMaxM = 64;      // above: LDS-tiled kernel
// Above this many rows split-K tiles (given a workspace) beat the streaming kernel
// (measured at K = 7168, N = 7168 / 9216 / 16384: 31.9 / 35.7 / 48.8 against
// 34.9 / 64.1 / 67.7 us at M = 40; up to 32 rows the streaming kernel wins: 23.6 /
// 31.7 / 33.5 against 31.4 / 34.0 / 47.5 us at M = 32).
constexpr int64_t kW4SplitMinM = 32;
constexpr int64_t kW4MaxSplit = 8;         // split-K ways at most

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

// Decode (M <= 16): K chunks folded into the MFMA.
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
// contiguous code bytes of weight row r % P of the strip and their 2 group scales,
// and 64 contiguous activation bytes of token row r % P (zeroed at use when the row
// is >= M or the chunk is past K).  A and B use the same k for the same (t, lane
// group, element), which is all the contraction needs.  Result lane l holds
// C[4 g + e][r]: token (4 g + e) % P of group (4 g + e) / P against weight row
// r % P of group r / P; it is a diagonal element when the two groups agree.  The
// MFMA accumulates straight into the strip's FP32 sums: the group scales are
// already inside the dequantized operand, so no promotion step is needed.
//
// One workgroup owns NS adjacent strips; its S waves take equal contiguous ranges
// of super blocks and each requests the fragments of CH super blocks before it uses
// any.  Branch-free, so that no load is sunk past another super block's MFMAs: a
// super block past the wave's range re-reads the wave's last one, chunks past K are
// clamped to the last one, and both are zeroed at use.
// The waves are light on registers, so a CU holds several workgroups and many
// loads in flight.  Partial sums over waves and groups are added through LDS in a
// fixed order (deterministic).
template <int P, int NS, int CH>
__global__ __launch_bounds__(kW4MaxWaves * 64) void w4a16_decode_kernel(W4Args a) {
    constexpr int G = 16 / P;
    extern __shared__ __attribute__((aligned(16))) v4f red[];      // [S][NS][64]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = blockDim.x >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int t = r / P, j = r % P;
    const bool mvalid = j < a.M;
    const int64_t strip0 = (int64_t)blockIdx.x * NS;
    const int64_t SB = (a.KB + G - 1) / G;
    const int64_t sb0 = (wave * SB) / S;
    const int64_t sb1 = ((wave + 1) * SB) / S;
    const uint16_t* xrow = a.x + (int64_t)(mvalid ? j : 0) * a.K + 32 * g;
    // Strip bases are wave-uniform (scalar registers); the lane's offsets within a strip
    // are 32-bit and the same for every strip (below (P + 1) K / 2, so K <= kDecodeMaxK
    // keeps them in range).
    const uint8_t* wst[NS];
    const uint8_t* sst[NS];
    const uint32_t woff = (uint32_t)(j * (a.K / 2) + 16 * g), soff = (uint32_t)(j * (a.K / 16) + 2 * g);
#pragma unroll
    for (int q = 0; q < NS; ++q) {
        // Strips past the last one (a partial final workgroup) re-read the last
        // strip; their results are not stored.
        const int64_t st = strip0 + q < a.strips ? strip0 + q : a.strips - 1;
        wst[q] = a.w + st * P * (a.K / 2);
        sst[q] = a.bs + st * P * (a.K / 16);
    }

    v4i wv[CH][NS], xv[CH][4];
    uint32_t sv[CH][NS];
    auto load_batch = [&](int64_t sb) {
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int64_t sbi = sb + i < sb1 ? sb + i : sb1 - 1;
            int64_t kc = sbi * G + t;                            // K block of this lane's chunk
            kc = kc < a.KB ? kc : a.KB - 1;
            const v4i* xp = reinterpret_cast<const v4i*>(xrow + kc * kGroup);
#pragma unroll
            for (int u = 0; u < 4; ++u) xv[i][u] = xp[u];
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                // Nontemporal: the code stream is read once; at P = 4 and 8 one load
                // instruction covers whole 128-byte lines (G adjacent K blocks of a row).
                wv[i][q] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4i*>(wst[q] + (woff + (uint32_t)kc * 64u)));
                sv[i][q] = *reinterpret_cast<const uint16_t*>(sst[q] + (soff + (uint32_t)kc * 8u));
            }
        }
    };

    v4f acc[NS];
#pragma unroll
    for (int q = 0; q < NS; ++q) acc[q] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    const v4i z4 = {0, 0, 0, 0};
    for (int64_t sb = sb0; sb < sb1; sb += CH) {
        load_batch(sb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const bool use = mvalid && sb + i < sb1 && (sb + i) * G + t < a.KB;
            v8bf xa[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) xa[u] = as_bf8(use ? xv[i][u] : z4);
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sv[i][q], 0);
                const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)sv[i][q], 1);
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[0], dequant8((uint32_t)wv[i][q].x, s0), acc[q], 0, 0, 0);
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[1], dequant8((uint32_t)wv[i][q].y, s0), acc[q], 0, 0, 0);
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[2], dequant8((uint32_t)wv[i][q].z, s1), acc[q], 0, 0, 0);
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[3], dequant8((uint32_t)wv[i][q].w, s1), acc[q], 0, 0, 0);
            }
        }
    }

#pragma unroll
    for (int q = 0; q < NS; ++q) red[(wave * NS + q) * 64 + lane] = acc[q];
    __syncthreads();
    // Output (token m, column c) of strip q: sum over waves, then over the G groups,
    // of the diagonal-block entry C[tt P + m][tt P + c], held by lane
    // 16 ((tt P + m) / 4) + tt P + c in its component (tt P + m) % 4.
    for (int o = threadIdx.x; o < NS * a.M * P; o += blockDim.x) {
        const int q = o / (a.M * P), rem = o % (a.M * P);
        const int m = rem / P, c = rem % P;
        if (strip0 + q >= a.strips) continue;
        float sum = 0.0f;
        for (int w = 0; w < S; ++w) {
#pragma unroll
            for (int tt = 0; tt < G; ++tt) {
                const int row = tt * P + m;
                sum += red[(w * NS + q) * 64 + 16 * (row >> 2) + tt * P + c][row & 3];
            }
        }
        a.y[(int64_t)m * a.N + (strip0 + q) * P + c] = (uint16_t)f32_to_bf16_rne(a.g * sum);
    }
}

// Prefill and batched decode (M > 64): LDS-tiled bf16 MFMA.
//
// A workgroup of 8 waves computes a BM x BN tile of y; its waves form a
// (BM / WM) x (BN / WN) grid of WM x WN wave tiles.  K advances in steps of 64:
// the next step's activations (BM x 64 BF16), codes (BN x 32 bytes) and group
// scales (BN x 4 bytes) are loaded into registers while the current step is
// computed from LDS, then written to the other half of a double buffer; one
// barrier per step.  Smaller tiles compute less per step, so their loads are
// requested DEPTH steps ahead (DEPTH register sets) to cover the memory latency.
//
// k of (MFMA kk < 2, lane group g, element e) = 16 g + 8 kk + e within the step,
// so a lane's codes for both MFMAs of a column are 8 contiguous bytes of one group
// of 16 (one LDS read, one scale byte), dequantized in registers (exact, as above)
// and used against all WM / 16 activation fragments of the wave.  Activations sit in
// LDS as 16-byte chunks (8 k of one row), chunk c of row i at slot c * BM + (i ^ c):
// an A fragment (16 rows, one chunk) is 256 contiguous bytes, and the 8 threads that
// stage one row's 128 bytes write 8 different bank groups.  Rows past M are loaded
// from row M - 1 and not stored; weight rows past N from row N - 1.
constexpr int kW4TileK = 64;

template <int BM, int BN, int WM, int WN, int DEPTH>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void w4a16_tile_kernel(W4Args a, int64_t tiles_n, int ksplit,
                                                                               float* part) {
    constexpr int NT = (BM / WM) * (BN / WN) * 64;            // threads
    static_assert(NT == 256 || NT == 512, "4 or 8 waves per workgroup");
    static_assert((BN * 2) % NT == 0 || BN * 2 < NT, "code pieces per thread");
    constexpr int TM = WM / 16, TN = WN / 16;                 // MFMA tiles per wave
    constexpr int A_PIECES = BM * 8 / NT;                      // 16-byte activation pieces per thread
    constexpr int B_PIECES = BN * 2 > NT ? BN * 2 / NT : 1;    // 16-byte code pieces per thread
    constexpr int A_BYTES = BM * 128, B_BYTES = BN * 32, S_BYTES = BN * 4;
    constexpr int BUF = A_BYTES + B_BYTES + S_BYTES;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // [2][BUF]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / (BN / WN), wn = wave % (BN / WN);
    const int g = lane >> 4, r = lane & 15;
    // Split-K: workgroup (tile, ks) covers K steps [KT ks / ksplit, KT (ks + 1) / ksplit)
    // and, when part is given, stores FP32 partial sums there instead of y.
    const int64_t tile = blockIdx.x / ksplit;
    const int ks = (int)(blockIdx.x % ksplit);
    const int64_t tm = tile / tiles_n, tn = tile % tiles_n;
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int64_t KT = a.K / kW4TileK;
    const int64_t s_begin = KT * ks / ksplit;
    const int64_t KS = KT * (ks + 1) / ksplit - s_begin;          // steps of this workgroup (>= 1)

    // Staging assignments.
    const uint16_t* xsrc[A_PIECES];
    int adst[A_PIECES];
#pragma unroll
    for (int i = 0; i < A_PIECES; ++i) {
        const int p = tid + NT * i;
        const int row = p >> 3, c = p & 7;
        const int64_t m = m0 + row < a.M ? m0 + row : a.M - 1;
        xsrc[i] = a.x + m * a.K + 8 * c;
        adst[i] = (c * BM + (row ^ c)) * 16;
    }
    const bool has_b = tid < BN * 2;          // with B_PIECES > 1 every thread has pieces
    const bool has_s = tid < BN;
    const uint8_t* wsrc[B_PIECES];
    const uint8_t* ssrc;
#pragma unroll
    for (int i = 0; i < B_PIECES; ++i) {
        const int p = tid + NT * i;
        const int brow = p >> 1, half = p & 1;
        const int64_t n = n0 + brow < a.N ? n0 + brow : a.N - 1;
        wsrc[i] = a.w + n * (a.K / 2) + 16 * half;
    }
    {
        const int64_t ns = n0 + tid < a.N ? n0 + tid : a.N - 1;
        ssrc = a.bs + (has_s ? ns : n0) * (a.K / 16);
    }
    // DEPTH register sets: step s + DEPTH is requested while step s is computed.
    v4i ra[DEPTH][A_PIECES], rb[DEPTH][B_PIECES];
    uint32_t rs[DEPTH];
    auto gload = [&](int d, int64_t s) {
        s = s < KS ? s : KS - 1;             // past the end: a repeated (cached) load, never stored
        const int64_t k0 = (s_begin + s) * kW4TileK;
#pragma unroll
        for (int i = 0; i < A_PIECES; ++i) ra[d][i] = *reinterpret_cast<const v4i*>(xsrc[i] + k0);
#pragma unroll
        for (int i = 0; i < B_PIECES; ++i)
            rb[d][i] = has_b ? *reinterpret_cast<const v4i*>(wsrc[i] + k0 / 2) : v4i{0, 0, 0, 0};
        rs[d] = has_s ? *reinterpret_cast<const uint32_t*>(ssrc + k0 / 16) : 0u;
    };
    auto lstore = [&](int d, int buf) {
        uint8_t* base = smem + buf * BUF;
#pragma unroll
        for (int i = 0; i < A_PIECES; ++i) *reinterpret_cast<v4i*>(base + adst[i]) = ra[d][i];
#pragma unroll
        for (int i = 0; i < B_PIECES; ++i)
            if (has_b) *reinterpret_cast<v4i*>(base + A_BYTES + (tid + NT * i) * 16) = rb[d][i];
        if (has_s) *reinterpret_cast<uint32_t*>(base + A_BYTES + B_BYTES + tid * 4) = rs[d];
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn) acc[i][jn] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // LDS byte offsets of this lane's fragments within a buffer: A tile i of MFMA kk at
    // aoff[kk] + 256 i (rows 16 i + r of the wave, chunk c = 2 g + kk, stored at slot
    // c * BM + (row ^ c) with (16 i + r) ^ c = 16 i + (r ^ c)); codes of column tile jn
    // at boff + 512 jn, its scales at soff + 64 jn.  All per-step addresses are a base
    // plus immediates.
    int aoff[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const int c = 2 * g + kk;
        aoff[kk] = (c * BM + wm * WM + (r ^ c)) * 16;
    }
    const int boff = A_BYTES + (wn * WN + r) * 32 + 8 * g;
    const int soff = A_BYTES + B_BYTES + (wn * WN + r) * 4;
    auto compute = [&](const uint8_t* base) {
        // Codes and group scale of the wave's TN column tiles: 8 bytes per lane and
        // tile cover both MFMAs of the step; each half is dequantized just before use.
        uint2 cw[TN];
        float sc[TN];
#pragma unroll
        for (int jn = 0; jn < TN; ++jn) {
            cw[jn] = *reinterpret_cast<const uint2*>(base + boff + 512 * jn);
            const uint32_t sw = *reinterpret_cast<const uint32_t*>(base + soff + 64 * jn);
            sc[jn] = __builtin_amdgcn_cvt_f32_fp8((int)(sw >> (8 * g)), 0);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            v8bf bq[TN];
#pragma unroll
            for (int jn = 0; jn < TN; ++jn) bq[jn] = dequant8(kk ? cw[jn].y : cw[jn].x, sc[jn]);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const v4i av = *reinterpret_cast<const v4i*>(base + aoff[kk] + 256 * i);
#pragma unroll
                for (int jn = 0; jn < TN; ++jn)
                    acc[i][jn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(av), bq[jn], acc[i][jn], 0, 0, 0);
            }
        }
        if constexpr (TM * TN >= 32) {
            // Scheduling pattern for the large tile: the first sub-step's dequantization,
            // then one MFMA per two VALU instructions (the second sub-step's
            // dequantization runs while the first sub-step's MFMAs execute), then the
            // remaining MFMAs.  Measured: about 5% on a 2048-token chunk.
            __builtin_amdgcn_sched_group_barrier(0x002, 40, 0);              // VALU
#pragma unroll
            for (int q = 0; q < TM * TN + TM * TN / 2; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);            // VALU
            }
            __builtin_amdgcn_sched_group_barrier(0x008, TM * TN / 2, 0);
        }
    };

    // The step loop is unrolled over an even number of steps (a multiple of DEPTH),
    // so that the LDS buffer of every step is a compile-time constant.
    constexpr int UNROLL = DEPTH % 2 == 0 ? DEPTH : 2 * DEPTH;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) gload(d, d);
    lstore(0, 0);
    __syncthreads();
    for (int64_t s0 = 0; s0 < KS; s0 += UNROLL) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t s = s0 + u;
            const int d = u % DEPTH, buf = u & 1;
            if (s < KS) {                                        // uniform
                gload(d, s + DEPTH);                             // set d held step s, already in LDS
                compute(smem + buf * BUF);
                if (s + 1 < KS) lstore((d + 1) % DEPTH, buf ^ 1);
                __syncthreads();
            }
        }
    }

#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jn = 0; jn < TN; ++jn)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + wm * WM + 16 * i + 4 * g + e;
                const int64_t n = n0 + wn * WN + 16 * jn + r;
                if (m < a.M && n < a.N) {
                    if (part) part[((int64_t)ks * a.M + m) * a.N + n] = acc[i][jn][e];
                    else a.y[m * a.N + n] = (uint16_t)f32_to_bf16_rne(a.g * acc[i][jn][e]);
                }
            }
}

template <int BM, int BN, int WM, int WN, int DEPTH>
static hipError_t launch_w4_tile(int64_t M, int64_t N, hipStream_t st, const W4Args& a, int ksplit = 1,
                                 float* part = nullptr) {
    constexpr unsigned lds = 2 * (BM * 128 + BN * 32 + BN * 4);
    static std::atomic<uint64_t> raised{0};
    if (lds > 65536) {
        const hipError_t e =
            raise_lds_limit((const void*)w4a16_tile_kernel<BM, BN, WM, WN, DEPTH>, raised, 160 * 1024);
        if (e != hipSuccess) return e;
    }
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    hipLaunchKernelGGL((w4a16_tile_kernel<BM, BN, WM, WN, DEPTH>), dim3((unsigned)(tiles_m * tiles_n * ksplit)),
                       dim3((BM / WM) * (BN / WN) * 64), lds, st, a, tiles_n, ksplit, part);
    if (part) {
        const int64_t mn = M * N;
        return launch_splitk_reduce(part, ksplit, mn, a.g, a.y, st);
    }
    return hipGetLastError();
}

size_t w4a16_workspace_size(int64_t M, int64_t N, int64_t K) {
    // Sized for the largest split any device up to 256 CUs would choose.
    if (M <= kW4SplitMinM || M <= 0 || N <= 0 || K <= 0) return 0;
    const int64_t t2 = ((M + 127) / 128) * ((N + 255) / 256);
    int64_t split = t2 < 256 ? 256 / t2 : 1;
    if (split > kW4MaxSplit) split = kW4MaxSplit;
    if (split > (K / kW4TileK) / 2) split = (K / kW4TileK) / 2;
    return split >= 2 ? (size_t)split * (size_t)M * (size_t)N * sizeof(float) : 0;
}

W4Plan plan_w4a16(int64_t M, int64_t N, int64_t K, int cus, size_t workspace_bytes) {
    W4Plan p{};
    p.groups = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.strips = N / 16;
    p.kblocks = K / kGroup;
    p.m_chunks = M > 0 ? (M + 16 * p.groups - 1) / (16 * p.groups) : 0;
    // Strips per workgroup of the streaming kernel: every workgroup reads its 16 R
    // BF16 activation rows (from L2) and, per strip, 16 rows of codes and scales
    // (K / 2 + K / 16 bytes each), and a CU runs several workgroups at once, so the
    // busiest CU moves ceil(workgroups / CUs) (32 R + 9 NS) K bytes; NS minimizes that
    // (ties to the larger NS).  NS = 4 only with R <= 2 (registers).
    {
        const int max_ns = p.groups <= 2 ? 4 : 2;
        int64_t best = -1;
        for (int ns = 1; ns <= max_ns; ns *= 2) {
            const int64_t wgs = (p.strips + ns - 1) / ns;
            const int64_t bytes = ((wgs + cus - 1) / cus) * (32 * (int64_t)p.groups + 9 * ns);
            if (best < 0 || bytes <= best) {
                best = bytes;
                p.strips_per_wg = ns;
            }
        }
    }
    if (const char* e = getenv("FP8BS_W4_STRIPS")) {        // tuning hook
        const int v = atoi(e);
        if (v == 1 || v == 2 || (v == 4 && p.groups <= 2)) p.strips_per_wg = v;
    }
    p.strip_wgs = (p.strips + p.strips_per_wg - 1) / p.strips_per_wg;
    p.waves = (int)(p.kblocks < kW4MaxWaves ? p.kblocks : kW4MaxWaves);
    if (const char* e = getenv("FP8BS_W4_WAVES")) {         // tuning hook
        const int v = atoi(e);
        if (v >= 1 && v <= kW4MaxWaves) p.waves = v;
    }
    // M > 64: LDS-tiled kernel, the largest tile that still gives (nearly) every CU
    // a workgroup; 32 < M <= 64 too when a split-K schedule fits the workspace.
    const int64_t t2s = ((M + 127) / 128) * ((N + 255) / 256);
    const bool small_split = M > kW4SplitMinM && M <= kW4StreamMaxM && t2s < cus - cus / 8 &&
                             (K / kW4TileK) / 2 >= 2 &&
                             workspace_bytes / ((size_t)M * N * sizeof(float)) >= 2;
    if (M > kW4StreamMaxM || small_split) {
        const int64_t enough = cus - cus / 8;
        auto tiles = [&](int64_t bm, int64_t bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
        // A CU runs one tile at a time, so a call takes ceil(tiles / CUs) rounds; one
        // round with every CU busy takes 75 (64 x 128), 94 (128 x 128), 150 (128 x 256)
        // and 221 us (256 x 256) at N = K = 7168.  The shape with the least rounds x
        // round time wins (measured: M = 768 on N = 7168 takes 128 x 256, 149 against
        // 184 us; M = 1536 takes 256 x 256, 208 against 290 us).
        {
            const int shapes[4][3] = {{64, 128, 75}, {128, 128, 94}, {128, 256, 150}, {256, 256, 221}};
            int64_t best = -1;
            for (const auto& sh : shapes) {
                const int64_t cost = ((tiles(sh[0], sh[1]) + cus - 1) / cus) * sh[2];
                if (best < 0 || cost < best) {
                    best = cost;
                    p.tile = sh[0] * 1000 + sh[1];
                }
            }
        }
        if (const char* e = getenv("FP8BS_W4_TILE")) {       // tuning hook
            const int v = atoi(e);
            if (v == 256256 || v == 128256 || v == 128128 || v == 64128) p.tile = v;
        }
        // Too few 128 x 256 tiles for the CUs (a batch of up to a few hundred tokens):
        // split K over workgroups when the caller gives room for the FP32 partial sums.
        const int64_t t2 = ((M + 127) / 128) * ((N + 255) / 256);
        const int64_t kt = K / kW4TileK;
        int64_t split = t2 < enough ? cus / t2 : 1;
        if (split > kW4MaxSplit) split = kW4MaxSplit;
        if (split > kt / 2) split = kt / 2;                   // at least 2 K steps each
        const int64_t room = (int64_t)(workspace_bytes / ((size_t)M * N * sizeof(float)));
        if (split > room) split = room;
        if (const char* e = getenv("FP8BS_W4_KSPLIT")) {     // tuning hook (within the room)
            const int v = atoi(e);
            if (v >= 1 && v <= kW4MaxSplit && v <= room && v <= kt) split = v;
        }
        if (split >= 2) {
            p.tile = 128256;
            p.ksplit = (int)split;
            return p;
        }
        if (M > kW4StreamMaxM) return p;
        p.tile = 0;                                           // no split after all: streaming
    }
    // Decode: K chunks folded into the MFMA; NS strips of P columns per workgroup.
    const char* de = getenv("FP8BS_W4_DECODE");              // tuning hook: 0 = stream kernel
    if (M <= 16 && K <= decode_max_k() && !(de && atoi(de) == 0)) {
        const int P = M <= 4 ? 4 : (M <= 8 ? 8 : 16);
        p.decode_p = P;
        const int64_t strips = N / P;
        // A strip is P rows of codes and scales (K / 2 + K / 16 bytes each); every
        // workgroup also reads the M x K BF16 activations.
        p.decode_ns = decode_strips_per_wg(strips, cus, P * (K / 2 + K / 16), 2 * M * K, 4);
        if (const char* e = getenv("FP8BS_W4_DECODE_NS")) {   // tuning hook
            const int v = atoi(e);
            if (v >= 1 && v <= 4) p.decode_ns = v;
        }
        const int64_t SB = (p.kblocks + 16 / P - 1) / (16 / P);
        p.waves = (int)(SB < kW4MaxWaves ? SB : kW4MaxWaves);
        if (const char* e = getenv("FP8BS_W4_DECODE_WAVES")) {   // tuning hook
            const int v = atoi(e);
            if (v >= 1 && v <= kW4MaxWaves && v <= SB) p.waves = v;
        }
        p.decode_wgs = (strips + p.decode_ns - 1) / p.decode_ns;
        // Two super blocks per load batch when a wave has more than one and a CU
        // holds fewer than two workgroups on average, as in the FP8 decode kernel
        // (M = 1, N = 7168, K = 8192, 448 workgroups: 10.3 us against 11.4 us with one
        // super block; q/k/v, 768 workgroups: 11.9 against 12.3 us).
        p.decode_ch = SB > p.waves && p.decode_wgs < 2 * (int64_t)cus ? 2 : 1;
        if (const char* e = getenv("FP8BS_W4_DECODE_CH")) {   // tuning hook
            const int v = atoi(e);
            if (v == 1 || v == 2) p.decode_ch = v;
        }
    }
    return p;
}

template <int P, int NS, int CH>
static hipError_t launch_w4_decode(const W4Plan& plan, hipStream_t st, const W4Args& a) {
    const unsigned lds = (unsigned)(plan.waves * NS * 64 * sizeof(v4f));
    hipLaunchKernelGGL((w4a16_decode_kernel<P, NS, CH>), dim3((unsigned)plan.decode_wgs), dim3(plan.waves * 64), lds, st,
                       a);
    return hipGetLastError();
}

template <int P, int NS>
static hipError_t launch_w4_decode_ns(const W4Plan& plan, hipStream_t st, const W4Args& a) {
    return plan.decode_ch == 2 ? launch_w4_decode<P, NS, 2>(plan, st, a) : launch_w4_decode<P, NS, 1>(plan, st, a);
}

template <int P>
static hipError_t launch_w4_decode_p(const W4Plan& plan, hipStream_t st, const W4Args& a) {
    switch (plan.decode_ns) {
        case 1: return launch_w4_decode_ns<P, 1>(plan, st, a);
        case 2: return launch_w4_decode_ns<P, 2>(plan, st, a);
        case 3: return launch_w4_decode_ns<P, 3>(plan, st, a);
        default: return launch_w4_decode_ns<P, 4>(plan, st, a);
    }
}

template <int R, int NS>
static hipError_t launch_w4_rns(dim3 grid, dim3 block, unsigned lds, hipStream_t st, const W4Args& a) {
    // More than 64 KiB of LDS needs the per-kernel limit raised, up to the CU's 160 KiB.
    static std::atomic<uint64_t> raised{0};
    if (lds > 65536) {
        const hipError_t e = raise_lds_limit((const void*)w4a16_stream_kernel<R, NS>, raised, 160 * 1024);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((w4a16_stream_kernel<R, NS>), grid, block, lds, st, a);
    return hipSuccess;
}

template <int R>
static hipError_t launch_w4_r(const W4Plan& plan, dim3 grid, dim3 block, unsigned lds, hipStream_t st,
                              const W4Args& a) {
    if (R <= 2 && plan.strips_per_wg == 4) return launch_w4_rns<R, R <= 2 ? 4 : 1>(grid, block, lds, st, a);
    if (plan.strips_per_wg == 2) return launch_w4_rns<R, 2>(grid, block, lds, st, a);
    return launch_w4_rns<R, 1>(grid, block, lds, st, a);
}

hipError_t launch_w4a16(const W4Plan& plan, const void* x, const void* w, const void* bs, float gscale, void* y,
                        int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t st) {
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
    switch (plan.tile) {
        case 256256: return launch_w4_tile<256, 256, 128, 64, 1>(M, N, st, a);
        case 128256:
            return plan.ksplit >= 2 ? launch_w4_tile<128, 256, 64, 64, 2>(M, N, st, a, plan.ksplit, (float*)workspace)
                                    : launch_w4_tile<128, 256, 64, 64, 2>(M, N, st, a);
        case 128128: return launch_w4_tile<128, 128, 64, 32, 3>(M, N, st, a);
        case 64128: return launch_w4_tile<64, 128, 32, 32, 4>(M, N, st, a);
        default: break;
    }
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
