// C ABI of libfp8bs.so (declared in include/fp8bs.h).
//
// Every entry point validates its arguments on the host before touching the HIP
// runtime, so argument errors are reported synchronously and identically with or
// without a GPU.  Then it checks (once per device, cached) that the current device
// is gfx950, and enqueues the kernels on the caller's stream.
#include <atomic>
#include <cstdint>
#include <cmath>
#include <cstring>

#include "fp8bs.h"
#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = not yet queried, > 0 = gfx950 with that many CUs, < 0 = not gfx950.
std::atomic<int> g_device_cus[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Sizes must be non-negative and every element/byte count must fit int64.
bool mul_ok(int64_t a, int64_t b) { return a == 0 || b <= INT64_MAX / a; }

int check_device(int* cus_out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FP8BS_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FP8BS_ERR_DEVICE;
    int v = g_device_cus[dev].load(std::memory_order_acquire);
    if (v == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8BS_ERR_HIP;
        const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        v = ok ? (prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1) : -1;
        g_device_cus[dev].store(v, std::memory_order_release);
    }
    if (v < 0) return FP8BS_ERR_DEVICE;
    if (cus_out) *cus_out = v;
    return FP8BS_OK;
}

int quant_shape_check(const void* in, const void* q, const float* s, int64_t M, int64_t K) {
    if (M < 0 || K < 0 || K % 128 != 0 || !mul_ok(M, K) || !mul_ok(M * K, 2)) return FP8BS_ERR_SHAPE;
    if (M == 0 || K == 0) return 1;   // nothing to do
    if (!in || !q || !s) return FP8BS_ERR_NULL;
    if (!aligned(in, 16) || !aligned(q, 16) || !aligned(s, 4)) return FP8BS_ERR_ALIGN;
    return FP8BS_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? FP8BS_OK : FP8BS_ERR_HIP; }

// Scratch of fp8_block_linear_noalloc: split-K partial sums (FP32 [split][M][N]),
// written completely by the tile kernel before the reduce kernel reads them, so
// nothing in it needs clearing between calls.  On a device of up to 256 CUs a split
// keeps split x tiles <= 256 tiles of 128 x 256 (or 128 x 128) partials, at most
// 32 MiB (16 MiB with 128 x 128 tiles).  Each GPU
// holds its own copy for the life of the process.  In host code `scratch` names a
// host-side stand-in: kernels get the device address from hipGetSymbolAddress.
constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
static_assert(kNoAllocScratchBytes == FP8BS_NOALLOC_SCRATCH_BYTES, "header and library disagree");
__device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];

// The current device's scratch address, looked up once per device (with that device
// current) and kept.
int device_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FP8BS_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FP8BS_ERR_DEVICE;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP8BS_ERR_HIP;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return FP8BS_OK;
}

}  // namespace

extern "C" {

int fp8bs_abi_version(void) { return FP8BS_ABI_VERSION; }

const char* fp8bs_status_string(int status) {
    switch (status) {
        case FP8BS_OK: return "ok";
        case FP8BS_ERR_NULL: return "a required pointer is NULL";
        case FP8BS_ERR_SHAPE: return "invalid shape (negative size, K or N not a multiple of 128, or overflow)";
        case FP8BS_ERR_ALIGN: return "misaligned pointer (tensors need 16-byte, scales 4-byte alignment)";
        case FP8BS_ERR_DEVICE: return "the current HIP device is not gfx950 (MI355X)";
        case FP8BS_ERR_HIP: return "HIP runtime call or kernel launch failed";
        case FP8BS_ERR_WORKSPACE:
            return "workspace must be 256-byte aligned (no-allocation call: the shape needs more than the static "
                   "scratch)";
        case FP8BS_ERR_VALUE:
            return "scalar argument out of range (RMSNorm eps must be finite and > 0, the NVFP4 global scale finite)";
        default: return "unknown fp8bs status";
    }
}

int fp8_quant_act(const void* x_bf16, void* q_e4m3, float* s_f32, int64_t M, int64_t K, hipStream_t stream) {
    int rc = quant_shape_check(x_bf16, q_e4m3, s_f32, M, K);
    if (rc != FP8BS_OK) return rc > 0 ? FP8BS_OK : rc;
    if ((rc = check_device(nullptr)) != FP8BS_OK) return rc;
    return hip_status(fp8bs::launch_quant_act(x_bf16, q_e4m3, s_f32, M, K, stream));
}

int fp8_quant_weight(const void* w_bf16, void* qw_e4m3, float* ws_f32, int64_t N, int64_t K, hipStream_t stream) {
    if (N < 0 || N % 128 != 0) return FP8BS_ERR_SHAPE;
    int rc = quant_shape_check(w_bf16, qw_e4m3, ws_f32, N, K);
    if (rc != FP8BS_OK) return rc > 0 ? FP8BS_OK : rc;
    if ((rc = check_device(nullptr)) != FP8BS_OK) return rc;
    return hip_status(fp8bs::launch_quant_weight(w_bf16, qw_e4m3, ws_f32, N, K, stream));
}

int fp8_silu_mul_quant(const void* gu_bf16, void* q_e4m3, float* s_f32, int64_t M, int64_t I, hipStream_t stream) {
    if (I < 0 || !mul_ok(I, 2)) return FP8BS_ERR_SHAPE;
    int rc = quant_shape_check(gu_bf16, q_e4m3, s_f32, M, I);
    if (rc == FP8BS_OK && !mul_ok(M, 2 * I)) rc = FP8BS_ERR_SHAPE;
    if (rc != FP8BS_OK) return rc > 0 ? FP8BS_OK : rc;
    if ((rc = check_device(nullptr)) != FP8BS_OK) return rc;
    return hip_status(fp8bs::launch_silu_mul_quant(gu_bf16, q_e4m3, s_f32, M, I, stream));
}

int fp8_rmsnorm_quant(const void* x_bf16, const void* gamma_bf16, float eps, void* q_e4m3, float* s_f32,
                      int64_t M, int64_t K, hipStream_t stream) {
    int rc = quant_shape_check(x_bf16, q_e4m3, s_f32, M, K);
    if (rc != FP8BS_OK) return rc > 0 ? FP8BS_OK : rc;
    if (!gamma_bf16) return FP8BS_ERR_NULL;
    if (!aligned(gamma_bf16, 16)) return FP8BS_ERR_ALIGN;
    if (!(eps > 0.0f) || !std::isfinite(eps)) return FP8BS_ERR_VALUE;
    if ((rc = check_device(nullptr)) != FP8BS_OK) return rc;
    return hip_status(fp8bs::launch_rmsnorm_quant(x_bf16, gamma_bf16, eps, q_e4m3, s_f32, M, K, stream));
}

size_t fp8_block_linear_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K <= 0 || N % 128 || K % 128 || !mul_ok(N, K) || !mul_ok(M, K) || !mul_ok(M, N))
        return 0;
    if (!mul_ok(M * N, 32)) return 0;
    return fp8bs::prefill_workspace_size(M, N, K);     // split-K partial sums (0 when unused)
}

namespace {

int linear_check(const void* q_e4m3, const float* s_f32, const void* w_e4m3, const float* ws_f32, void* y_bf16,
                 int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return FP8BS_ERR_SHAPE;
    if (!mul_ok(N, K) || !mul_ok(M, K) || !mul_ok(M, N) || !mul_ok(M * N, 2)) return FP8BS_ERR_SHAPE;
    if (M == 0 || N == 0) return 1;                      // nothing to do
    if (!q_e4m3 || !s_f32 || !w_e4m3 || !ws_f32 || !y_bf16) return FP8BS_ERR_NULL;
    if (!aligned(q_e4m3, 16) || !aligned(w_e4m3, 16) || !aligned(y_bf16, 16) || !aligned(s_f32, 4) ||
        !aligned(ws_f32, 4))
        return FP8BS_ERR_ALIGN;
    return FP8BS_OK;
}

// Schedule choice and launches of a validated call on a gfx950 device with `cus` CUs.
int linear_dispatch(const void* q_e4m3, const float* s_f32, const void* w_e4m3, const float* ws_f32, void* y_bf16,
                    int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes, int cus,
                    hipStream_t stream) {
    if (M <= fp8bs::kDecodeMaxM && K <= fp8bs::decode_max_k()) {
        const fp8bs::DecodePlan plan = fp8bs::plan_decode(M, N, K, cus);
        return hip_status(
            fp8bs::launch_gemm_decode(plan, q_e4m3, s_f32, w_e4m3, ws_f32, y_bf16, M, N, K, stream));
    }
    // 32 < M <= 64 with a workspace: split-K tiles beat weight streaming.
    if (M <= fp8bs::kMidMaxM &&
        !(M > fp8bs::kSplitMinM && workspace && fp8bs::prefill_plan_split(M, N, K, cus, workspace_bytes) >= 2)) {
        const fp8bs::MidPlan plan = fp8bs::plan_mid(M, N, K, cus);
        return hip_status(fp8bs::launch_gemm_mid(plan, q_e4m3, s_f32, w_e4m3, ws_f32, y_bf16, M, N, K, stream));
    }
    return hip_status(fp8bs::launch_gemm_prefill(q_e4m3, s_f32, w_e4m3, ws_f32, y_bf16, M, N, K, cus, workspace,
                                                 workspace ? workspace_bytes : 0, stream));
}

}  // namespace

int fp8_block_linear(const void* q_e4m3, const float* s_f32, const void* w_e4m3, const float* ws_f32,
                     void* y_bf16, int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    int rc = linear_check(q_e4m3, s_f32, w_e4m3, ws_f32, y_bf16, M, N, K);
    if (rc != FP8BS_OK) return rc > 0 ? FP8BS_OK : rc;
    if (workspace && !aligned(workspace, 256)) return FP8BS_ERR_WORKSPACE;
    int cus = 0;
    if ((rc = check_device(&cus)) != FP8BS_OK) return rc;
    return linear_dispatch(q_e4m3, s_f32, w_e4m3, ws_f32, y_bf16, M, N, K, workspace, workspace_bytes, cus, stream);
}

int fp8_block_linear_noalloc(const void* q_e4m3, const float* s_f32, const void* w_e4m3, const float* ws_f32,
                             void* y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    int rc = linear_check(q_e4m3, s_f32, w_e4m3, ws_f32, y_bf16, M, N, K);
    if (rc != FP8BS_OK) return rc > 0 ? FP8BS_OK : rc;
    if (fp8_block_linear_workspace_size(M, N, K) > kNoAllocScratchBytes) return FP8BS_ERR_WORKSPACE;
    int cus = 0;
    if ((rc = check_device(&cus)) != FP8BS_OK) return rc;
    void* ws = nullptr;
    if ((rc = device_scratch(&ws)) != FP8BS_OK) return rc;
    return linear_dispatch(q_e4m3, s_f32, w_e4m3, ws_f32, y_bf16, M, N, K, ws, kNoAllocScratchBytes, cus, stream);
}

int nvfp4_w4a16_linear(const void* x_bf16, const void* w_fp4, const void* bs_e4m3, float g, void* y_bf16,
                       int64_t M, int64_t N, int64_t K, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    if (M < 0 || N < 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return FP8BS_ERR_SHAPE;
    if (!mul_ok(N, K) || !mul_ok(M, K) || !mul_ok(M * K, 2) || !mul_ok(M, N) || !mul_ok(M * N, 4))
        return FP8BS_ERR_SHAPE;
    if (M > INT32_MAX) return FP8BS_ERR_SHAPE;             // token rows are 32-bit in the kernels
    if (!std::isfinite(g)) return FP8BS_ERR_VALUE;
    if (M == 0 || N == 0) return FP8BS_OK;
    if (!x_bf16 || !w_fp4 || !bs_e4m3 || !y_bf16) return FP8BS_ERR_NULL;
    if (!aligned(x_bf16, 16) || !aligned(w_fp4, 16) || !aligned(bs_e4m3, 16) || !aligned(y_bf16, 16))
        return FP8BS_ERR_ALIGN;
    if (workspace && !aligned(workspace, 256)) return FP8BS_ERR_WORKSPACE;
    int cus = 0;
    int rc = check_device(&cus);
    if (rc != FP8BS_OK) return rc;
    const fp8bs::W4Plan plan = fp8bs::plan_w4a16(M, N, K, cus, workspace ? workspace_bytes : 0);
    if (plan.ksplit >= 2)                                  // one launch: M is at most a few hundred rows
        return hip_status(fp8bs::launch_w4a16(plan, x_bf16, w_fp4, bs_e4m3, g, y_bf16, M, N, K, workspace, stream));
    // The grid covers at most kW4MaxChunks chunks of token rows per launch.
    const int64_t rows_per_launch = fp8bs::kW4MaxChunks * 16 * plan.groups;
    for (int64_t m0 = 0; m0 < M; m0 += rows_per_launch) {
        const int64_t mm = M - m0 < rows_per_launch ? M - m0 : rows_per_launch;
        fp8bs::W4Plan p = plan;
        p.m_chunks = (mm + 16 * p.groups - 1) / (16 * p.groups);
        const hipError_t e = fp8bs::launch_w4a16(p, (const uint16_t*)x_bf16 + m0 * K, w_fp4, bs_e4m3, g,
                                                 (uint16_t*)y_bf16 + m0 * N, mm, N, K, nullptr, stream);
        if (e != hipSuccess) return FP8BS_ERR_HIP;
    }
    return FP8BS_OK;
}

size_t nvfp4_w4a16_workspace_size(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K <= 0 || N % 128 != 0 || K % 128 != 0) return 0;
    if (!mul_ok(M, N) || !mul_ok(M * N, 32)) return 0;
    return fp8bs::w4a16_workspace_size(M, N, K);
}

}  // extern "C"
