// Prefill-shape block-scaled FP8 GEMM (M > 16) for gfx950.
//
// y[m, n] = sum_kb (s[m, kb] * ws[n/128, kb]) * sum_{k in kb} q[m, k] * w[n, k]
// ("Nanbeige4.3-33B FP8" model card, introduction: E4M3 weights in 128x128 blocks,
// dynamic per-token group-128 activation scales; FP32 accumulation, BF16 out).
//
// Tiling: a workgroup of WM x WN waves (4 x 2 in the shapes launched) computes a
// BM (m) x BN (n) output tile, each wave owning (BM/WM) x (BN/WN).  The K loop steps one
// 128-wide scale block at a time through a ring of NST LDS stages (as many as the
// 160 KiB of LDS holds: 2 for 256 x 256 tiles, 3 for 128 x 256 and 256 x 128, 4 for
// 128 x 128), stage (kb - kb0) mod NST holding K block kb:
//   1. during step kb the copies of K block kb + NST - 1 go into the stage that step
//      kb - 1 read, issued over the first subtile rows -- direct global -> LDS loads
//      (global_load_lds_dwordx4: no VGPRs, no LDS write instructions), overlapping the
//      compute.  A copy that the memory pipeline cannot take yet stalls its wave,
//      MFMAs included, so with BN = 256 tiles waves 0-3 (one per SIMD) issue all of
//      them, 8 per subtile row over the first two rows (128 x 256: 4 per row over
//      three rows), while the other wave on each SIMD keeps the MFMA pipe busy;
//      128 x 128 tiles spread them over every wave, two per row.  At the end of the
//      step each wave waits until its copies of K block kb + 1 have landed -- the
//      NST - 2 younger stages' copies stay in flight -- and the workgroup meets at a
//      barrier.  With two stages a step's copies must land within that step: with
//      only 8 or 16 MFMAs per wave per step (128-row tiles) each step then lasted
//      about one global-load latency;
//   2. each wave runs v_mfma_f32_16x16x128_f8f6f4 over its 16 x 16 subtiles (A = 16
//      weight rows, B = 16 token rows; one MFMA covers the whole K block) and folds
//      each FP32 result into its accumulators with acc += (s[m] * ws[nb]) * P: the
//      promotion of partial sums per 128-wide K block;
//   3. the epilogue rounds the tile to BF16 (or keeps FP32 split-K partial sums),
//      passes it through the then-free stage ring and stores whole lines.
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
// a grouped (2 tile-rows) raster order: tiles that share q rows or w rows then
// share an XCD's L2.
#include <cstdlib>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace fp8bs {

// Tile rows per raster group.  Measured with 256 x 256 tiles (prefill_oproj /
// fusion_fc): 2 rows 425 us / 4.65 ms, 1 row 424 us / 4.84 ms, 4 rows 441 us / 4.64 ms,
// 8 rows 439 us / 4.83 ms, 16 and 32 rows slower still.
constexpr int kGroupRows = 2;
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
// LDS stages of the K loop's ring: as many as fit 160 KiB (stage_bytes: 66.8 KiB for
// 256 x 256, 49-50 KiB for 128 x 256 and 256 x 128, 33.5 KiB for 128 x 128).
constexpr int prefill_stages(int BM, int BN) { return BM == 256 && BN == 256 ? 2 : (BM == 128 && BN == 128 ? 4 : 3); }
// Waves that issue the stage copies, and copies per subtile row.  256 x 256 tiles: 4
// waves (one per SIMD), 8 per row -- measured against all 8 waves with 2 per row:
// prefill_oproj 424 -> 412 us, fusion_fc 4.74 -> 4.52 ms, M = 2048 on the 7168 x 7168
// projection 131.5 -> 125.4 us (4 per row: 418 us / 4.58 ms; 16 in the first row:
// 431 us / 4.71 ms).  128 x 256 tiles: 4 waves, 4 per row (M = 640 / 768 / 1024 on that
// projection: 88.0 / 90.1 / 97.9 -> 82.8 / 84.4 / 92.8 us).  128 x 128 tiles were slower
// that way (M = 64, split-K tiles: 25.7 -> 29.8 us), so they keep every wave, 2 per row.
constexpr int prefill_copy_waves(int BM, int BN, int waves) { return BN == 256 ? 4 : waves; }
constexpr int prefill_copies_per_row(int BM, int BN) { return BN == 256 ? (BM == 256 ? 8 : 4) : 2; }
// Dynamic LDS of a launch: the ring of stages.
constexpr int prefill_lds_bytes(int BM, int BN) { return prefill_stages(BM, BN) * stage_bytes(BM, BN); }
static_assert(prefill_lds_bytes(256, 256) <= 160 * 1024 && prefill_lds_bytes(128, 256) <= 160 * 1024 &&
                  prefill_lds_bytes(256, 128) <= 160 * 1024 && prefill_lds_bytes(128, 128) <= 160 * 1024,
              "the stage ring fits the LDS");

// s_waitcnt vmcnt(N) lgkmcnt(0), expcnt not waited (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt in 6:4, lgkmcnt in 11:8).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

// acc += sc * p: the promotion of one 16 x 16 K-block product into its accumulators.
__device__ __forceinline__ void promote(v4f& acc, float sc, const v4f& p) {
    acc[0] = fmaf(sc, p[0], acc[0]);
    acc[1] = fmaf(sc, p[1], acc[1]);
    acc[2] = fmaf(sc, p[2], acc[2]);
    acc[3] = fmaf(sc, p[3], acc[3]);
}

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
    constexpr int NST = prefill_stages(BM, BN);
    // A stage is (BM + BN) / 8 copy units of 8 tile rows (1 KiB, one 64-lane
    // 16-byte direct-to-LDS load); copying wave w takes kUnitsLo or kUnitsLo + 1 of
    // them.
    constexpr int kUnits = (BM + BN) / 8;
    constexpr int kCopyWaves = prefill_copy_waves(BM, BN, kWaves);
    constexpr int kUnitsLo = kUnits / kCopyWaves, kUnitsExtra = kUnits % kCopyWaves;
    constexpr int kCopies = kUnitsLo + (kUnitsExtra ? 1 : 0);    // per copying wave, at most
    constexpr int kPer = prefill_copies_per_row(BM, BN);          // copies per subtile row
    constexpr int kCopyRows = (kCopies + kPer - 1) / kPer;        // subtile rows issuing copies
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tiles are whole MFMA subtiles");
    static_assert(WTN <= 128 && 128 % WTN == 0, "a wave's n-range must lie in one weight block");
    static_assert(BN % 8 == 0 && BM % 8 == 0, "copies: 8-row groups");
    static_assert(kCopyRows <= TI, "the copies fit the subtile rows");
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
    const int ucount = wave < kCopyWaves ? kUnitsLo + (wave < kUnitsExtra ? 1 : 0) : 0;
    const int ubase = wave < kCopyWaves ? wave * kUnitsLo + (wave < kUnitsExtra ? wave : kUnitsExtra) : 0;
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
            // rows past M read row M - 1 (never stored); the unit's base row is
            // min(r0, M - 1), so lane row min(r0 + lrow, M - 1) is 0..7 rows past it
            const int64_t r0 = m0 + (R - BN);
            const int64_t crow = r0 < a.M ? r0 : a.M - 1;
            const int64_t lr = r0 + lrow < a.M ? r0 + lrow : a.M - 1;
            off = (uint32_t)(lr - crow) * (uint32_t)a.K + (voff[u & 1] - (uint32_t)(lrow * a.K));
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

    // ---- scales: the BM token scales and the weight-block scales of K block kb are
    // copied into the stage with the tiles (4-byte direct-to-LDS loads).
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

    // Prologue: K blocks kb0 .. kb0 + NST - 2 into stages 0 .. NST - 2 (past kb1 - 1
    // the last block is repeated, so every stage and step issues the same loads).
#pragma unroll
    for (int st = 0; st < NST - 1; ++st) {
        const int64_t k = kb0 + st < kb1 ? kb0 + st : kb1 - 1;
        copy_stage(k, st);
        copy_scales(k, st);
        copy_wscales(k, st);
    }
    // Loads this wave issues per stage (wave-uniform).
    const int c_w = ucount + (xs_copy ? 1 : 0) + (ws_copy ? 1 : 0);

    // Fragments of one step, read from LDS stage `st`: the TJ B fragments (token rows),
    // their promotion factors s[m] * ws[nb], and the first A fragment (weight rows).
    v8i bf[TJ], af_next;
    float xsv[TJ], wsc = 0.0f;
    auto load_frags = [&](int st) {
        const uint8_t* wt = lds + st * kStage;
        const uint8_t* xt = wt + BN * 128;
        // Scales first: LDS reads return in order, so their wait does not include the
        // fragments issued after them.
        const float* xs_lds = reinterpret_cast<const float*>(xt + BM * 128);
        wsc = reinterpret_cast<const float*>(xt + BM * 128 + BM * 4)[(wn * WTN) / kGroup];
#pragma unroll
        for (int j = 0; j < TJ; ++j) xsv[j] = xs_lds[wm * WTM + 16 * j + r];
#pragma unroll
        for (int j = 0; j < TJ; ++j) bf[j] = lds_frag(xt, wm * WTM + 16 * j + r, g);
        af_next = lds_frag(wt, wn * WTN + r, g);
    };
    // This wave's copies (and scale loads) into the next stage have landed and it has
    // consumed every LDS read of the current one; the barrier makes everyone's copies
    // visible.  Loads complete in issue order, so the wait leaves in flight exactly the
    // NST - 2 younger stages' loads, c_w per stage: vmcnt((NST - 2) c_w), an immediate,
    // hence one branch per value c_w takes (kCopies or 0 copies, plus 0 or 1 scale
    // load; any other count waits for everything).  A plain s_barrier: __syncthreads()
    // would add a full vmcnt(0) wait (its fence).  The empty asm statements keep the
    // compiler from moving LDS accesses across the wait and the barrier.
    auto stage_ready = [&]() {
        asm volatile("" ::: "memory");
        if constexpr (NST == 2) {
            wait_vm_lgkm0<0>();
        } else {
            if (c_w == kCopies + 1)
                wait_vm_lgkm0<(NST - 2) * (kCopies + 1)>();
            else if (c_w == kCopies)
                wait_vm_lgkm0<(NST - 2) * kCopies>();
            else if (c_w == 1)
                wait_vm_lgkm0<NST - 2>();
            else
                wait_vm_lgkm0<0>();
        }
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    stage_ready();
    load_frags(0);

    int stage = 0;
    for (int64_t kb = kb0; kb < kb1; ++kb) {
        const int fill = stage == 0 ? NST - 1 : stage - 1;     // the stage step kb - 1 read
        const int nxt = stage + 1 == NST ? 0 : stage + 1;
        const uint8_t* wt = lds + stage * kStage;
        // Subtile row i: TJ independent MFMAs (own result registers), each followed by
        // the promotion of row i - 1's result in the same column (one row later than it
        // was issued, so the FMAs do not wait for the MFMA pipe); the next A fragment is
        // read from LDS meanwhile.  After the last row's MFMAs are issued, the workgroup
        // meets at the barrier for the next stage and reads the next step's fragments
        // while those MFMAs run and the last row is promoted: the step boundary does not
        // drain the MFMA pipe.
        v4f pend[TJ];
        float sc[TJ];                                   // promotion factors s[m] * ws[nb]
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            // Formed where first needed (row 1's promotions), past the wait for row 0's
            // fragments, so the scale reads add no wait of their own.
            if (i == (TI > 1 ? 1 : 0)) {
#pragma unroll
                for (int j = 0; j < TJ; ++j) sc[j] = xsv[j] * wsc;
            }
            // The copies of K block kb + NST - 1 are spread over the first rows, so the
            // workgroup's vector-memory requests do not queue up at the top of the
            // step in front of its LDS reads; past the last K block they repeat it
            // (no branch in the loop, and the same loads every step).
            const int64_t kn = kb + NST - 1 < kb1 ? kb + NST - 1 : kb1 - 1;
            if (i < kCopyRows) {
#pragma unroll
                for (int c = 0; c < kPer; ++c)
                    if (kPer * i + c < kCopies) copy_one(kn, fill, kPer * i + c);
            }
            if (i == kCopyRows - 1) {
                copy_scales(kn, fill);
                copy_wscales(kn, fill);
            }
            const v8i af = af_next;
            if (i + 1 < TI) af_next = lds_frag(wt, wn * WTN + 16 * (i + 1) + r, g);
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                // Format 0 = E4M3 for both operands; zero scale operands select the unscaled MFMA.
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], zero, 0, 0, 0, 0, 0, 0);
                // The promotion of the previous row's subtile j, TJ MFMAs after it was issued:
                // its result is ready, so the FMAs run while this row's MFMAs execute.  The
                // scheduling barriers keep the compiler from moving FMAs next to the MFMA
                // whose result they read.
                __builtin_amdgcn_sched_barrier(0);
                if (i > 0) promote(acc[i - 1][j], sc[j], pend[j]);
                __builtin_amdgcn_sched_barrier(0);
                pend[j] = p;
            }
        }
        float sc_last[TJ];
#pragma unroll
        for (int j = 0; j < TJ; ++j) sc_last[j] = sc[j];
        // Past the last K block the next stage holds a repeat of the last block: reading
        // it keeps the loop free of branches (a branch here would keep both fragment
        // sets alive across it).
        stage_ready();
        load_frags(nxt);
#pragma unroll
        for (int j = 0; j < TJ; ++j) promote(acc[TI - 1][j], sc_last[j], pend[j]);
        stage = nxt;
    }

    // No direct-to-LDS load (the repeats of the last K block) may still be in flight
    // when the workgroup's LDS is released.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: lane holds y[m][n .. n + 3] for each (i, j), as FP32 partial sums
    // (split-K) or rounded to BF16.  Stored straight from the accumulator layout, each
    // store instruction writes 32- (BF16) or 64-byte (FP32) pieces of 16 rows, and a
    // 256 x 256 BF16 tile took about 9.5 us to write (4.7 us to issue wave 0's stores,
    // 5 us to drain them) against a 110 us K loop.  Instead each wave puts its
    // WTM x WTN tile into its own LDS region (the stages are free once every wave has
    // finished its last fragment reads: the barrier), reads it back by rows and stores
    // 16 bytes per lane, whole lines.  Region rows are WTN * EB bytes; 16-byte chunk c
    // of region row m sits at chunk c ^ (m mod CPR), so that the rows an accumulator
    // write covers fall in different banks.  FP32 tiles of 256 rows do not fit the
    // ring; split-K never runs them, and they keep the direct stores.
    const bool fp32_out = a.part != nullptr;
    constexpr bool kStagedF32 = BM * BN * 4 <= prefill_lds_bytes(BM, BN);
    static_assert(BM * BN * 2 <= prefill_lds_bytes(BM, BN), "the BF16 tile fits the stage ring");
    if (!kStagedF32 && fp32_out) {
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            if (!mok[j]) continue;
            const int64_t m = m0 + wm * WTM + 16 * j + r;
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const int64_t n = n0 + wn * WTN + 16 * i + 4 * g;
                *reinterpret_cast<v4f*>(a.part + ((int64_t)ks * a.M + m) * a.N + n) = acc[i][j];
            }
        }
        return;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    auto staged = [&](auto eb) {
        constexpr int EB = decltype(eb)::value;                // bytes per element: 2 or 4
        constexpr int RB = WTN * EB;                           // region row bytes
        constexpr int CPR = RB / 16;                           // 16-byte chunks per region row
        constexpr int RPI = 64 / CPR;                          // region rows per read instruction
        static_assert(RB % 16 == 0 && 64 % CPR == 0 && WTM % RPI == 0, "epilogue row mapping");
        uint8_t* region = lds + wave * (WTM * RB);
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int ml = 16 * j + r;
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                // n = 16 i + 4 g .. + 3 within the wave tile
                if constexpr (EB == 4) {
                    *reinterpret_cast<v4f*>(region + ml * RB + (((4 * i + g) ^ (ml % CPR)) << 4)) = acc[i][j];
                } else {
                    const bf16x2 lo = __builtin_convertvector(f32x2{acc[i][j][0], acc[i][j][1]}, bf16x2);
                    const bf16x2 hi = __builtin_convertvector(f32x2{acc[i][j][2], acc[i][j][3]}, bf16x2);
                    uint2 o;
                    __builtin_memcpy(&o.x, &lo, 4);
                    __builtin_memcpy(&o.y, &hi, 4);
                    const int chunk = 2 * i + (g >> 1);
                    *reinterpret_cast<uint2*>(region + ml * RB + ((chunk ^ (ml % CPR)) << 4) + (g & 1) * 8) = o;
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int rl = lane / CPR, cl = lane % CPR;
#pragma unroll
        for (int it = 0; it < WTM / RPI; ++it) {
            const int ml = it * RPI + rl;
            const v4i v = *reinterpret_cast<const v4i*>(region + ml * RB + ((cl ^ (ml % CPR)) << 4));
            const int64_t m = m0 + wm * WTM + ml;
            if (CLAMP && m >= a.M) continue;
            const int64_t n = n0 + wn * WTN + (16 / EB) * cl;
            if constexpr (EB == 4)
                *reinterpret_cast<v4i*>(a.part + ((int64_t)ks * a.M + m) * a.N + n) = v;
            else
                *reinterpret_cast<v4i*>(a.y + m * a.N + n) = v;
        }
    };
    if (kStagedF32 && fp32_out)
        staged(std::integral_constant<int, 4>{});
    else
        staged(std::integral_constant<int, 2>{});
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
// Tile columns of the split-K schedule: 256 from two tile rows of 128 on (M > 128,
// N a multiple of 256), else 128.  Measured on the 7168 x 7168 projection, 128 x 256
// split tiles against 128 x 128 (split or not): M = 160 / 256 / 300 / 384 / 512:
// 42.5 / 43.6 / 67.2 / 67.4 / 67.9 -> 37.4 / 39.6 / 48.9 / 50.0 / 59.9 us (the wider
// tiles halve the activation re-reads, and give a split where the 128 x 128 tiles
// were too many to split); M = 128 the same, M = 48 - 96 slower (30.8 against 25.4 us
// at M = 48).
static int64_t prefill_split_bn(int64_t M, int64_t N) { return N % 256 == 0 && M > 128 ? 256 : 128; }

int prefill_split(int64_t M, int64_t N, int64_t K, int cus) {
    if (M <= kSplitMinM) return 0;
    const int64_t t = (M + 127) / 128 * (N / prefill_split_bn(M, N));
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
    // over the workgroups of each 128 x 128 or 128 x 256 tile (prefill_split_bn);
    // FP32 partial sums, then a reduce kernel adds them in a fixed order.
    const int split = prefill_plan_split(M, N, K, cus, workspace ? workspace_bytes : 0);
    if (split >= 2) {
        tile = prefill_split_bn(M, N) == 256 ? 128256 : 128128;
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
