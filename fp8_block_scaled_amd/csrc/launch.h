// Host-side launchers of the gfx950 kernels (called by the C ABI in api.hip after
// validation; they assume valid shapes, aligned pointers and a gfx950 device).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace fp8bs {

// Raises `fn`'s dynamic-LDS limit to `bytes` on the current device, once per device.
// hipFuncSetAttribute acts on the current device only, so each launcher keeps one
// bit per device (devices 0..63; higher ones repeat the idempotent call every time).
inline hipError_t raise_lds_limit(const void* fn, std::atomic<uint64_t>& done, unsigned bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
    if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    done.fetch_or(bit, std::memory_order_relaxed);
    return hipSuccess;
}

hipError_t launch_quant_act(const void* x, void* q, float* s, int64_t M, int64_t K, hipStream_t st);
hipError_t launch_silu_mul_quant(const void* gu, void* q, float* s, int64_t M, int64_t I, hipStream_t st);
hipError_t launch_rmsnorm_quant(const void* x, const void* gamma, float eps, void* q, float* s, int64_t M, int64_t K,
                                hipStream_t st);
hipError_t launch_quant_weight(const void* w, void* qw, float* ws, int64_t N, int64_t K, hipStream_t st);

// ---- decode GEMM (M <= kDecodeMaxM): one workgroup per strip of `rows` columns, split-K over its waves
constexpr int kDecodeMaxM = 16;
// ... and K <= kDecodeMaxK: its per-lane weight offsets are 32-bit (below 17 K).  Longer
// rows take the mid-size kernel (64-bit addresses; rows past M repeat row M - 1).
constexpr int64_t kDecodeMaxK = int64_t{1} << 27;
// kDecodeMaxK, or a lower bound set by the FP8BS_DECODE_MAX_K test hook.
int64_t decode_max_k();

// Strips per workgroup for the weight-streaming decode kernels.  Workgroups go
// round-robin to the CUs and a CU's own bandwidth is limited, so the time follows
// what the busiest CU moves: ceil(workgroups / cus) workgroups, each NS strips of
// weights (`strip_bytes` each, from HBM) and one copy of the activations
// (`act_bytes`, from L2, counted at half weight).  Returns the NS in 1..max_ns that
// makes it smallest and, of equals, the largest (fewer workgroups).
inline int decode_strips_per_wg(int64_t strips, int cus, int64_t strip_bytes, int64_t act_bytes, int max_ns) {
    if (cus <= 0) cus = 1;
    int best = 1;
    double best_cost = 0.0;
    for (int ns = 1; ns <= max_ns; ++ns) {
        const int64_t wgs = (strips + ns - 1) / ns;
        const double cost = (double)((wgs + cus - 1) / cus) * ((double)ns * strip_bytes + 0.5 * act_bytes);
        if (ns == 1 || cost <= best_cost) {
            best_cost = cost;
            best = ns;
        }
    }
    return best;
}

struct DecodePlan {
    int rows;            // 4, 8 or 16: token rows per MFMA group = output columns per strip
    int strips_per_wg;   // 1..4 adjacent strips per workgroup
    int64_t strips;      // N / rows
    int64_t workgroups;  // ceil(strips / strips_per_wg)
    int64_t kblocks;     // K / 128
    int waves;           // waves per workgroup = K splits
    int batch;           // super blocks whose loads are issued together (1 or 2)
    int interleave;      // 1: wave w of S takes super blocks w, w + S, ...; 0: contiguous ranges
};

DecodePlan plan_decode(int64_t M, int64_t N, int64_t K, int cus);

hipError_t launch_gemm_decode(const DecodePlan& plan, const void* q, const float* s, const void* w,
                              const float* ws, void* y, int64_t M, int64_t N, int64_t K, hipStream_t st);

// ---- mid-size GEMM (kDecodeMaxM < M <= kMidMaxM): weight streaming, R token groups
// (above 64 rows the 128 x 128 prefill tiles are faster)
constexpr int kMidMaxM = 64;
// Above this many rows a split-K prefill schedule (given a workspace) is used instead.
constexpr int kSplitMinM = 32;

struct MidPlan {
    int groups;          // R: 16-token groups per weight fragment (2, 4 or 8)
    int strips_per_wg;   // 1 or 2 strips of 16 output columns per workgroup
    int64_t strips;      // N / 16
    int64_t workgroups;  // ceil(strips / strips_per_wg)
    int64_t kblocks;     // K / 128
    int waves;           // waves per workgroup = K splits
};

MidPlan plan_mid(int64_t M, int64_t N, int64_t K, int cus);

hipError_t launch_gemm_mid(const MidPlan& plan, const void* q, const float* s, const void* w, const float* ws,
                           void* y, int64_t M, int64_t N, int64_t K, hipStream_t st);

// ---- prefill GEMM (M > kMidMaxM): LDS-tiled FP8 MFMA; with a workspace, split-K
// for shapes whose tiles leave CUs idle
hipError_t launch_gemm_prefill(const void* q, const float* s, const void* w, const float* ws, void* y,
                               int64_t M, int64_t N, int64_t K, int cus, void* workspace, size_t workspace_bytes,
                               hipStream_t st);
size_t prefill_workspace_size(int64_t M, int64_t N, int64_t K);
// Split-K ways launch_gemm_prefill uses for this shape and workspace (0: none).
int prefill_plan_split(int64_t M, int64_t N, int64_t K, int cus, size_t workspace_bytes);

// ---- split-K reduce: y = BF16(g * sum over ks < ksplit of part[ks]), in order
// (part: FP32 [ksplit][mn], mn a multiple of 4; y: BF16 [mn])
hipError_t launch_splitk_reduce(const float* part, int ksplit, int64_t mn, float g, uint16_t* y, hipStream_t st);

// ---- NVFP4 weight-only linear (W4A16): weight streaming, R 16-token groups per
// dequantized fragment, M covered in chunks of 16 R rows (second grid dimension)
constexpr int64_t kW4MaxChunks = 65535;   // grid.y limit; larger M is split on the host

struct W4Plan {
    int groups;          // R: 16-token groups per weight fragment (1, 2 or 4)
    int strips_per_wg;   // 1 or 2 strips of 16 output columns per workgroup
    int64_t strips;      // N / 16
    int64_t strip_wgs;   // ceil(strips / strips_per_wg)
    int64_t m_chunks;    // ceil(M / (16 R))
    int64_t kblocks;     // K / 128
    int waves;           // waves per workgroup = K splits
    int decode_p;        // > 0: decode kernel (M <= 16) with strips of P columns
    int decode_ns;       //   strips per workgroup (1..4)
    int decode_ch;       //   super blocks per load batch (1 or 2)
    int64_t decode_wgs;
    int tile;            // > 0: LDS-tiled kernel, BM * 1000 + BN
    int ksplit;          // >= 2: split-K over workgroups, FP32 partials in the workspace
};

// Workspace bytes the split-K schedule can use (0 when it never applies).
size_t w4a16_workspace_size(int64_t M, int64_t N, int64_t K);

W4Plan plan_w4a16(int64_t M, int64_t N, int64_t K, int cus, size_t workspace_bytes);

hipError_t launch_w4a16(const W4Plan& plan, const void* x, const void* w, const void* bs, float g, void* y,
                        int64_t M, int64_t N, int64_t K, void* workspace, hipStream_t st);

}  // namespace fp8bs
