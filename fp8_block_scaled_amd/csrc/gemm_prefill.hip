// Prefill-shape block-scaled FP8 GEMM (M > 16) for gfx950.
//
// y[m, n] = sum_kb (s[m, kb] * ws[n/128, kb]) * sum_{k in kb} q[m, k] * w[n, k]
// ("Nanbeige4.3-33B FP8" model card, introduction: E4M3 weights in 128x128 blocks,
// dynamic per-token group-128 activation scales; FP32 accumulation, BF16 out).
//
// Tiling: a workgroup of WM x WN waves (4 x 2 in the shapes launched) computes a
// BM (m) x BN (n) output tile, each wave owning (BM/WM) x (BN/WN).  The K loop steps one
// 128-wide scale block at a time through two LDS stages:
//   1. at the top of step kb the wave waits for its own copies into stage kb%2
//      and the workgroup meets at a barrier; the copies of K block kb + 1 into the
//      other stage are then issued, two per subtile row over the first rows --
//      direct global -> LDS loads (global_load_lds_dwordx4: no VGPRs, no LDS write
//      instructions), overlapping the compute of step kb.  Each thread also
//      touches one 128-byte line of K block kb + 2 (a 4-byte direct-to-LDS load
//      into a dump area) so that the copies of the next step find their lines in
//      L2: a double-buffered 256 x 256 tile fills 128 KB of LDS, leaving no room
//      for a third stage, and the first touch of a line from HBM takes longer
//      than one step of compute;
//   2. each wave runs v_mfma_f32_16x16x128_f8f6f4 over its 16 x 16 subtiles (A = 16
//      weight rows, B = 16 token rows; one MFMA covers the whole K block) and folds
//      each FP32 result into its accumulators with acc += (s[m] * ws[nb]) * P: the
//      promotion of partial sums per 128-wide K block.
// LDS rows are 128 bytes; 16-byte chunk c of tile row r is stored at chunk
// position c ^ ((r >> 1) & 7), so the 16 rows a fragment read touches fall in 16
// distinct 4-bank groups.  A direct-to-LDS load writes lane l's 16 bytes at
// position l of the wave's 1 KiB destination, so the swizzle is applied by
// choosing which source chunk each lane fetches (8 lanes per 128-byte row: still
// whole cache lines).
// BN/2 <= 128 and tiles start at multiples of BN, so a wave's n-range lies in one
// 128-row weight block: one weight scale per lane per K block, plus one token scale
// per m-subtile.  Rows past M (the ragged last m-tile) load the last valid row and
// are not stored.
// Workgroup ids are remapped so that the tiles each XCD receives are contiguous in
// a grouped (8 tile-rows) raster order: tiles that share q rows or w rows then
// share an XCD's L2.
#include <cstdlib>

#include "device_common.h"
#include "launch.h"

namespace fp8bs {

constexpr int kGroupRows = 8;
constexpr int kXcds = 8;
constexpr int kPrefillMaxSplit = 8;

struct PrefillArgs {
    const uint8_t* w;
    const float* ws;
    const uint8_t* x;
    const float* xs;
    uint16_t* y;
    int64_t M, N, K, KB;
    int64_t tiles_m, tiles_n;
    int ksplit;          // >= 1: K blocks split over this many workgroups per tile
    float* part;         // split-K: FP32 partial sums [ksplit][M][N] (else nullptr)
};

// Bytes of one LDS stage: w tile, q tile, BM token scales, weight scales (one
// wave's 4-byte copy writes 256 bytes; the first BN/128 are the tile's weight blocks).
constexpr int stage_bytes(int BM, int BN) { return (BM + BN) * 128 + BM * 4 + 256; }
// Dynamic LDS of a launch: two stages and the 256-byte warm-up dump.
constexpr int prefill_lds_bytes(int BM, int BN) { return 2 * stage_bytes(BM, BN) + 256; }

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int row, int g) {
    const v4i lo = *reinterpret_cast<const v4i*>(tile + swz(row, g));
    const v4i hi = *reinterpret_cast<const v4i*>(tile + swz(row, g + 4));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

template <int BM, int BN, int WM, int WN, bool CLAMP>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_prefill_kernel(PrefillArgs a) {
    constexpr int kWaves = WM * WN, kThreads = 64 * kWaves;
    constexpr int WTM = BM / WM, WTN = BN / WN;        // wave tile (m, n)
    constexpr int TJ = WTM / 16, TI = WTN / 16;         // subtiles (m, n)
    constexpr int kStage = stage_bytes(BM, BN);
    // A stage is (BM + BN) / 8 copy units of 8 tile rows (1 KiB, one 64-lane
    // 16-byte direct-to-LDS load); wave w takes kUnitsLo or kUnitsLo + 1 of them.
    constexpr int kUnits = (BM + BN) / 8;
    constexpr int kUnitsLo = kUnits / kWaves, kUnitsExtra = kUnits % kWaves;
    constexpr int kCopies = kUnitsLo + (kUnitsExtra ? 1 : 0);    // per wave, at most
    constexpr int kCopyRows = (kCopies + 1) / 2;                  // subtile rows issuing copies
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tiles are whole MFMA subtiles");
    static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's n-range must lie in one weight block");
    static_assert(BN % 8 == 0 && BM % 8 == 0, "copies: 8-row groups");
    static_assert(kCopyRows <= TI, "two copies per subtile row");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // ---- tile selection: XCD-contiguous, grouped raster
    const int64_t T = a.tiles_m * a.tiles_n;
    // Split-K: workgroup b covers K blocks [KB ks / ksplit, KB (ks + 1) / ksplit) of
    // tile b / ksplit.
    const int64_t b = blockIdx.x / a.ksplit;
    const int ks = (int)(blockIdx.x % a.ksplit);
    const int64_t kb0 = a.KB * ks / a.ksplit, kb1 = a.KB * (ks + 1) / a.ksplit;
    const int64_t xcd = b % kXcds, jx = b / kXcds;
    const int64_t per = T / kXcds, extra = T % kXcds;
    const int64_t t = xcd * per + (xcd < extra ? xcd : extra) + jx;
    const int64_t group_span = kGroupRows * a.tiles_n;
    const int64_t grp = t / group_span;
    const int64_t first_m = grp * kGroupRows;
    const int64_t gm = (a.tiles_m - first_m) < kGroupRows ? (a.tiles_m - first_m) : kGroupRows;
    const int64_t in_grp = t - grp * group_span;
    const int64_t tm = first_m + in_grp % gm;
    const int64_t tn = in_grp / gm;
    // Without CLAMP (M >= BM) the last tile row is moved back to end at row M - 1:
    // every row it loads is valid, and the rows it shares with the tile row before
    // are computed identically by both and stored twice with the same value.
    const int64_t m0 = CLAMP ? tm * BM : (tm * BM + BM <= a.M ? tm * BM : a.M - BM);
    const int64_t n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int g = lane >> 4, r = lane & 15;

    // ---- copy assignment: stage rows [0, BN) are w rows n0.., rows [BN, BN+BM) are
    // q rows m0..; copy unit u moves the 8 tile rows starting at R = 8 u (64
    // chunks, 1 KiB of LDS at u KiB); lane l takes row R + l / 8 and LDS chunk
    // position l % 8, i.e. source chunk (l % 8) ^ ((row >> 1) & 7).  A unit lies in
    // one operand (BN is a multiple of 8), so each copy is a wave-uniform base (row
    // R's address) plus a 32-bit lane offset.  The lane offset depends on u only
    // through its parity (the swizzle): two offsets serve all copies -- except
    // with CLAMP, where rows past M are replaced by row M - 1 and the offset is
    // formed per copy.
    const int ucount = kUnitsLo + (wave < kUnitsExtra ? 1 : 0);
    const int ubase = wave * kUnitsLo + (wave < kUnitsExtra ? wave : kUnitsExtra);
    const int lrow = lane >> 3;
    uint32_t voff[2];
#pragma unroll
    for (int par = 0; par < 2; ++par) {
        const int chunk = (lane & 7) ^ ((4 * par + (lrow >> 1)) & 7);
        voff[par] = (uint32_t)(lrow * a.K + chunk * 16);
    }
    // Wave-uniform row addresses of this wave's copies (scalar registers).
    const uint8_t* cbase[kCopies];
#pragma unroll
    for (int c = 0; c < kCopies; ++c) {
        int u = ubase + c;
        u = u < kUnits ? u : kUnits - 1;        // an unused last slot of a short wave
        const int R = 8 * u;
        int64_t row = R < BN ? n0 + R : m0 + (R - BN);
        if (CLAMP && R >= BN) row = row < a.M ? row : a.M - 1;
        cbase[c] = (R < BN ? a.w : a.x) + row * a.K;
    }
    auto copy_one = [&](int64_t kb, int stage, int c) {
        if (c >= ucount) return;                // wave-uniform
        const int u = ubase + c;
        const int R = 8 * u;
        uint32_t off = voff[u & 1];
        if (CLAMP && R >= BN) {
            // rows past M read row M - 1 (never stored)
            const int64_t row = (int64_t)((cbase[c] - a.x) / a.K);
            int64_t lr = row + lrow;
            lr = lr < a.M ? lr : a.M - 1;
            off = (uint32_t)((lr - row) * a.K) + (voff[u & 1] - (uint32_t)(lrow * a.K));
        }
        // The empty asm keeps the per-iteration scalar address opaque, so the lane
        // offset is added at the load (scalar base + 32-bit offset) instead of being
        // folded into a loop-invariant 64-bit address per copy.
        const uint8_t* src = cbase[c] + kb * kGroup;
        asm volatile("" : "+s"(src));
        uint8_t* dst = lds + stage * kStage + u * 1024;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + off),
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    };
    auto copy_stage = [&](int64_t kb, int stage) {
#pragma unroll
        for (int c = 0; c < kCopies; ++c) copy_one(kb, stage, c);
    };

    // ---- L2 warm-up of K block kb + 2: thread t touches stage row t mod (BM + BN)
    // (one line).  Every thread issues it, so it is always each wave's last load.
    static_assert(BM + BN <= kThreads, "one warm-up line per thread covers the stage");
    const int pf_row = tid % (BM + BN);
    const bool pf_w = pf_row < BN;
    int64_t pf_off;
    {
        int64_t row = pf_w ? n0 + pf_row : m0 + (pf_row - BN);
        if (CLAMP && !pf_w) row = row < a.M ? row : a.M - 1;
        pf_off = row * a.K;
    }
    auto warm = [&](int64_t kb) {
        const uint8_t* base = (pf_w ? a.w : a.x) + kb * kGroup;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(base + pf_off),
                                         (__attribute__((address_space(3))) void*)(lds + 2 * kStage), 4, 0, 0);
    };

    // ---- scales: the BM token scales and the weight-block scales of K block kb are
    // copied into the stage with the tiles (4-byte direct-to-LDS loads), so the
    // warm-up touch is always each wave's last vector load and nothing waits on it.
    static_assert(BM % 64 == 0 && BM / 64 <= kWaves, "one scale copy per wave");
    const bool xs_copy = wave < BM / 64;
    uint32_t xs_off;
    {
        int64_t m = m0 + wave * 64 + lane;
        m = m < a.M ? m : a.M - 1;
        xs_off = (uint32_t)(m * a.KB);
    }
    auto copy_scales = [&](int64_t kb, int stage) {
        if (xs_copy)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a.xs + xs_off + kb),
                                             (__attribute__((address_space(3))) void*)(lds + stage * kStage +
                                                                                      (BM + BN) * 128 + wave * 256),
                                             4, 0, 0);
    };
    // Weight scales of the tile's BN/128 weight blocks: wave (BM/64) mod waves copies
    // them (lane l takes block l mod (BN/128)).
    const bool ws_copy = wave == (BM / 64) % kWaves;
    const uint32_t ws_off = (uint32_t)((n0 / kGroup + lane % (BN / kGroup)) * a.KB);
    auto copy_wscales = [&](int64_t kb, int stage) {
        if (ws_copy)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a.ws + ws_off + kb),
                                             (__attribute__((address_space(3))) void*)(lds + stage * kStage +
                                                                                      (BM + BN) * 128 + BM * 4),
                                             4, 0, 0);
    };
    bool mok[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) mok[j] = !CLAMP || m0 + wm * WTM + 16 * j + r < a.M;

    v4f acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    copy_stage(kb0, 0);
    copy_scales(kb0, 0);
    copy_wscales(kb0, 0);
    warm(kb0 + 1 < kb1 ? kb0 + 1 : kb1 - 1);

    for (int64_t kb = kb0; kb < kb1; ++kb) {
        const int stage = (int)((kb - kb0) & 1);
        // This wave's copies into `stage` (and the scale loads) have landed -- all
        // but the last load issued, the warm-up touch; the barrier makes everyone's
        // copies visible and frees the other stage.
        // A plain s_barrier: __syncthreads() would add a full vmcnt(0) wait (its
        // fence) and so wait for the warm-up touch as well.  Every LDS read of the
        // previous step was consumed before a wave reaches the barrier, and each
        // wave has waited for its own copies above; the empty asm statements keep
        // the compiler from moving LDS accesses across the barrier.
        asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        const bool more = kb + 1 < kb1;
        const uint8_t* wt = lds + stage * kStage;
        const uint8_t* xt = wt + BN * 128;
        v8i bf[TJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) bf[j] = lds_frag(xt, wm * WTM + 16 * j + r, g);
        const float* xs_lds = reinterpret_cast<const float*>(xt + BM * 128);
        const float wsc = reinterpret_cast<const float*>(xt + BM * 128 + BM * 4)[(wn * WTN) / kGroup];
        float sc[TJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) sc[j] = xs_lds[wm * WTM + 16 * j + r] * wsc;
        // Subtile row i: TJ independent MFMAs (own result registers), then their
        // promotions; the next A fragment is read from LDS meanwhile.
        v8i af_next = lds_frag(wt, wn * WTN + r, g);
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            // The copies of K block kb + 1 are spread over the first rows, so the
            // workgroup's vector-memory requests do not queue up at the top of the
            // step in front of its LDS reads; past the last K block they repeat it
            // into the idle stage (no branch in the loop).
            const int64_t kn = more ? kb + 1 : kb;
            if (i < kCopyRows) {
                copy_one(kn, stage ^ 1, 2 * i);
                if (2 * i + 1 < kCopies) copy_one(kn, stage ^ 1, 2 * i + 1);
            }
            if (i == kCopyRows - 1) {
                copy_scales(kn, stage ^ 1);
                copy_wscales(kn, stage ^ 1);
                warm(kb + 2 < kb1 ? kb + 2 : kb1 - 1);         // always one warm-up load last
            }
            const v8i af = af_next;
            if (i + 1 < TI) af_next = lds_frag(wt, wn * WTN + 16 * (i + 1) + r, g);
            v4f p[TJ];
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                // Format 0 = E4M3 for both operands; zero scale operands select the unscaled MFMA.
                p[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], zero, 0, 0, 0, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                acc[i][j][0] = fmaf(sc[j], p[j][0], acc[i][j][0]);
                acc[i][j][1] = fmaf(sc[j], p[j][1], acc[i][j][1]);
                acc[i][j][2] = fmaf(sc[j], p[j][2], acc[i][j][2]);
                acc[i][j][3] = fmaf(sc[j], p[j][3], acc[i][j][3]);
            }
        }
    }

    // No direct-to-LDS load (the last warm-up touch) may still be in flight when
    // the workgroup's LDS is released.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: lane holds y[m][n .. n + 3] for each (i, j)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
        if (!mok[j]) continue;
        const int64_t m = m0 + wm * WTM + 16 * j + r;
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const int64_t n = n0 + wn * WTN + 16 * i + 4 * g;
            if (a.part) {                                      // split-K partial sums
                *reinterpret_cast<v4f*>(a.part + ((int64_t)ks * a.M + m) * a.N + n) = acc[i][j];
                continue;
            }
            uint2 o;
            o.x = f32_to_bf16_rne(acc[i][j][0]) | (f32_to_bf16_rne(acc[i][j][1]) << 16);
            o.y = f32_to_bf16_rne(acc[i][j][2]) | (f32_to_bf16_rne(acc[i][j][3]) << 16);
            *reinterpret_cast<uint2*>(a.y + m * a.N + n) = o;
        }
    }
}

template <int BM, int BN, int WM, int WN, bool CLAMP>
static hipError_t launch_tiles(PrefillArgs a, hipStream_t st) {
    a.tiles_m = (a.M + BM - 1) / BM;
    a.tiles_n = a.N / BN;
    const int64_t T = a.tiles_m * a.tiles_n;
    if (T == 0) return hipSuccess;
    constexpr int lds = prefill_lds_bytes(BM, BN);
    static std::atomic<uint64_t> raised{0};
    {
        const hipError_t e = raise_lds_limit((const void*)gemm_prefill_kernel<BM, BN, WM, WN, CLAMP>, raised, lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gemm_prefill_kernel<BM, BN, WM, WN, CLAMP>), dim3((unsigned)(T * a.ksplit)),
                       dim3(64 * WM * WN), lds, st, a);
    if (a.part) return launch_splitk_reduce(a.part, a.ksplit, a.M * a.N, 1.0f, a.y, st);
    return hipGetLastError();
}

template <int BM, int BN, int WM, int WN>
static hipError_t launch_shape(PrefillArgs a, hipStream_t st) {
    // M < BM: one partial tile row whose rows past M are clamped.
    if (a.M < BM) return launch_tiles<BM, BN, WM, WN, true>(a, st);
    return launch_tiles<BM, BN, WM, WN, false>(a, st);
}

// Split-K ways for a shape whose 128 x 128 tiles leave CUs idle (0: none); the
// workspace size query assumes up to 256 CUs.  Above kSplitMinM rows split-K tiles
// beat the weight-streaming mid-size kernel (measured on the 7168 x 7168
// projection: 25.0 against 26.2 us at M = 48, 25.7 against 30.0 us at M = 64; at
// M <= 32 the mid-size kernel is faster: 19.9 against 24.6 us at M = 32).
int prefill_split(int64_t M, int64_t N, int64_t K, int cus) {
    if (M <= kSplitMinM) return 0;
    const int64_t t = (M + 127) / 128 * (N / 128);
    if (t >= cus - cus / 8) return 0;
    int64_t split = cus / t;
    if (split > kPrefillMaxSplit) split = kPrefillMaxSplit;
    if (split > (K / kGroup) / 4) split = (K / kGroup) / 4;   // at least 4 K blocks each
    return split >= 2 ? (int)split : 0;
}

int prefill_plan_split(int64_t M, int64_t N, int64_t K, int cus, size_t workspace_bytes) {
    int split = prefill_split(M, N, K, cus);
    const int64_t room = (int64_t)(workspace_bytes / ((size_t)M * N * sizeof(float)));
    if (split > room) split = (int)room;
    if (const char* e = getenv("FP8BS_PREFILL_KSPLIT")) {     // tuning hook (within the room)
        const int v = atoi(e);
        if (v >= 1 && v <= kPrefillMaxSplit && v <= room && v <= K / kGroup && M > kSplitMinM) split = v;
    }
    return split >= 2 ? split : 0;
}

size_t prefill_workspace_size(int64_t M, int64_t N, int64_t K) {
    const int split = prefill_split(M, N, K, 256);
    return split ? (size_t)split * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_prefill(const void* q, const float* s, const void* w, const float* ws, void* y,
                               int64_t M, int64_t N, int64_t K, int cus, void* workspace, size_t workspace_bytes,
                               hipStream_t st) {
    PrefillArgs a;
    a.w = (const uint8_t*)w;
    a.ws = ws;
    a.x = (const uint8_t*)q;
    a.xs = s;
    a.y = (uint16_t*)y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.KB = K / kGroup;
    a.ksplit = 1;
    a.part = nullptr;
    // Tile shape, 8 waves each.  A CU runs one tile at a time, so a call takes
    // ceil(tiles / CUs) rounds of one tile's time; the tile times per round measured
    // at N = K = 7168 with every CU busy are 107 (256 x 256, waves of 64 x 128),
    // 76 (128 x 256) and 57 us (128 x 128), i.e. relative costs 187 : 133 : 100.
    // The shape with the least rounds x cost wins (measured: M = 768 takes 128 x 256,
    // 74 against 98 us with 128 x 128 tiles; M = 1536 takes 256 x 256, 98 against
    // 138 us with 128 x 256).  N not a multiple of 256: the largest of 256 x 128 and
    // 128 x 128 that still gives nearly every CU a tile.  Tuning hook
    // FP8BS_PREFILL_TILE = 256256, 256128, 128256 or 128128 forces a shape.
    const bool n256 = N % 256 == 0;
    const int64_t enough = cus - cus / 8;
    auto tiles = [&](int64_t bm, int64_t bn) { return (M + bm - 1) / bm * (N / bn); };
    auto rounds = [&](int64_t t) { return (t + cus - 1) / cus; };
    int tile = 128128;
    if (n256) {
        int64_t best = rounds(tiles(128, 128)) * 100;
        if (rounds(tiles(128, 256)) * 133 < best) {
            best = rounds(tiles(128, 256)) * 133;
            tile = 128256;
        }
        if (rounds(tiles(256, 256)) * 187 < best) tile = 256256;
    } else if (tiles(256, 128) >= enough) {
        tile = 256128;
    }
    if (const char* e = getenv("FP8BS_PREFILL_TILE")) {
        const int t = atoi(e);
        if (t == 256128 || t == 128128 || (n256 && (t == 256256 || t == 128256))) tile = t;
    }
    // Few tiles (a batch of up to a few hundred tokens): with a workspace, split K
    // over the workgroups of each 128 x 128 tile; FP32 partial sums, then a reduce
    // kernel adds them in a fixed order.
    const int split = prefill_plan_split(M, N, K, cus, workspace ? workspace_bytes : 0);
    if (split >= 2) {
        tile = 128128;
        a.ksplit = split;
        a.part = (float*)workspace;
    }
    switch (tile) {
        case 256256: return launch_shape<256, 256, 4, 2>(a, st);
        case 128256: return launch_shape<128, 256, 2, 4>(a, st);
        case 128128: return launch_shape<128, 128, 2, 4>(a, st);
        default: return launch_shape<256, 128, 4, 2>(a, st);
    }
}

}  // namespace fp8bs
