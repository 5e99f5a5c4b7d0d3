// Prefill-shape block-scaled FP8 GEMM (M > 16) for gfx950.
//
// y[m, n] = sum_kb (s[m, kb] * ws[n/128, kb]) * sum_{k in kb} q[m, k] * w[n, k]
// ("Nanbeige4.3-33B FP8" model card, introduction: E4M3 weights in 128x128 blocks,
// dynamic per-token group-128 activation scales; FP32 accumulation, BF16 out).
//
// Tiling: a 256-thread workgroup computes a 128 (m) x 128 (n) output tile; each of
// its 4 waves owns 64 x 64.  The K loop steps one 128-wide scale block at a time:
//   1. the 128x128-byte tiles of q and w for the next K block are loaded from
//      global memory into registers while the current block is computed;
//   2. each wave issues 4 x 4 v_mfma_f32_16x16x128_f8f6f4 (A = 16 weight rows,
//      B = 16 token rows; one MFMA covers the whole K block), and folds every
//      16x16 FP32 result into its accumulators with acc += (s[m] * ws[nb]) * P:
//      the promotion of partial sums per 128-wide K block;
//   3. the prefetched tiles are written to the other LDS buffer.
// LDS rows are 128 bytes; 16-byte chunk c of row r is stored at chunk position
// c ^ ((r >> 1) & 7), so the 16 rows a fragment read touches map to 16 distinct
// 4-bank groups.
// The n-range of a wave lies inside one 128-row weight block, so every lane needs
// one weight scale and 4 token scales per K block.
// Workgroup ids are remapped so that the tiles each XCD receives are contiguous in
// a grouped (8 tile-rows) raster order: tiles that share q rows or w rows then
// share an XCD's L2.
#include "device_common.h"
#include "launch.h"

namespace fp8bs {

constexpr int kBM = 128, kBN = 128;
constexpr int kPrefillThreads = 256;
constexpr int kTileBytes = 128 * 128;
constexpr int kGroupRows = 8;
constexpr int kXcds = 8;

struct PrefillArgs {
    const uint8_t* w;
    const float* ws;
    const uint8_t* x;
    const float* xs;
    uint16_t* y;
    int64_t M, N, K, KB;
    int64_t tiles_m, tiles_n;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int row, int g) {
    const v4i lo = *reinterpret_cast<const v4i*>(tile + swz(row, g));
    const v4i hi = *reinterpret_cast<const v4i*>(tile + swz(row, g + 4));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

__global__ __launch_bounds__(kPrefillThreads, 2) void gemm_prefill_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];   // [stage][w, x]

    // ---- tile selection: XCD-contiguous, grouped raster
    const int64_t T = a.tiles_m * a.tiles_n;
    const int64_t b = blockIdx.x;
    const int64_t xcd = b % kXcds, j = b / kXcds;
    const int64_t per = T / kXcds, extra = T % kXcds;
    const int64_t t = xcd * per + (xcd < extra ? xcd : extra) + j;
    const int64_t group_span = kGroupRows * a.tiles_n;
    const int64_t grp = t / group_span;
    const int64_t first_m = grp * kGroupRows;
    const int64_t gm = (a.tiles_m - first_m) < kGroupRows ? (a.tiles_m - first_m) : kGroupRows;
    const int64_t in_grp = t - grp * group_span;
    const int64_t tm = first_m + in_grp % gm;
    const int64_t tn = in_grp / gm;
    const int64_t m0 = tm * kBM, n0 = tn * kBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int g = lane >> 4, r = lane & 15;

    // ---- global -> register assignment: chunk id tid + 256 i, 8 chunks per row
    const uint8_t* wsrc[4];
    const uint8_t* xsrc[4];
    bool xok[4];
    int ldst[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int cid = tid + 256 * i;
        const int row = cid >> 3, c = cid & 7;
        wsrc[i] = a.w + (n0 + row) * a.K + c * 16;
        xok[i] = (m0 + row) < a.M;
        xsrc[i] = a.x + (xok[i] ? (m0 + row) : 0) * a.K + c * 16;
        ldst[i] = swz(row, c);
    }
    v4i wreg[4], xreg[4];
    auto gload = [&](int64_t kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wreg[i] = *reinterpret_cast<const v4i*>(wsrc[i] + kb * kGroup);
            xreg[i] = xok[i] ? *reinterpret_cast<const v4i*>(xsrc[i] + kb * kGroup) : v4i{0, 0, 0, 0};
        }
    };
    auto lstore = [&](int stage) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<v4i*>(&lds[stage][0][ldst[i]]) = wreg[i];
            *reinterpret_cast<v4i*>(&lds[stage][1][ldst[i]]) = xreg[i];
        }
    };

    // ---- scales: token rows of this lane's 4 B fragments, and the weight block row
    const float* xs_row[4];
    bool mok[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int64_t m = m0 + wm * 64 + 16 * jj + r;
        mok[jj] = m < a.M;
        xs_row[jj] = a.xs + (mok[jj] ? m : 0) * a.KB;
    }
    const float* ws_row = a.ws + (n0 / kGroup) * a.KB;
    float xsc[4], wsc;
    float xsc_n[4], wsc_n;
    auto sload = [&](int64_t kb, float (&xs_)[4], float& ws_) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) xs_[jj] = mok[jj] ? xs_row[jj][kb] : 0.0f;
        ws_ = ws_row[kb];
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    gload(0);
    sload(0, xsc, wsc);
    lstore(0);

    for (int64_t kb = 0; kb < a.KB; ++kb) {
        __syncthreads();
        const int stage = (int)(kb & 1);
        const bool more = kb + 1 < a.KB;
        if (more) {
            gload(kb + 1);
            sload(kb + 1, xsc_n, wsc_n);
        }
        const uint8_t* wt = lds[stage][0];
        const uint8_t* xt = lds[stage][1];
        v8i bf[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) bf[jj] = lds_frag(xt, wm * 64 + 16 * jj + r, g);
        float sc[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sc[jj] = xsc[jj] * wsc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v8i af = lds_frag(wt, wn * 64 + 16 * i + r, g);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[jj], zero, 0, 0, 0, 0, 0, 0);
                acc[i][jj][0] = fmaf(sc[jj], p[0], acc[i][jj][0]);
                acc[i][jj][1] = fmaf(sc[jj], p[1], acc[i][jj][1]);
                acc[i][jj][2] = fmaf(sc[jj], p[2], acc[i][jj][2]);
                acc[i][jj][3] = fmaf(sc[jj], p[3], acc[i][jj][3]);
            }
        }
        if (more) {
            lstore(stage ^ 1);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) xsc[jj] = xsc_n[jj];
            wsc = wsc_n;
        }
    }

    // ---- epilogue: lane holds y[m][n .. n + 3] for each (i, jj)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        if (!mok[jj]) continue;
        const int64_t m = m0 + wm * 64 + 16 * jj + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t n = n0 + wn * 64 + 16 * i + 4 * g;
            uint2 o;
            o.x = f32_to_bf16_rne(acc[i][jj][0]) | (f32_to_bf16_rne(acc[i][jj][1]) << 16);
            o.y = f32_to_bf16_rne(acc[i][jj][2]) | (f32_to_bf16_rne(acc[i][jj][3]) << 16);
            *reinterpret_cast<uint2*>(a.y + m * a.N + n) = o;
        }
    }
}

hipError_t launch_gemm_prefill(const void* q, const float* s, const void* w, const float* ws, void* y,
                               int64_t M, int64_t N, int64_t K, int cus, hipStream_t st) {
    (void)cus;
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
    a.tiles_m = (M + kBM - 1) / kBM;
    a.tiles_n = N / kBN;
    const int64_t T = a.tiles_m * a.tiles_n;
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_prefill_kernel, dim3((unsigned)T), dim3(kPrefillThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace fp8bs
