/*
 * fp8bs.h -- C ABI of libfp8bs.so, the MI355X (gfx950) W8A8 FP8 block-scaled linear.
 *
 * The operation is the linear layer of the "Nanbeige4.3-33B FP8" model card
 * (ProCreations; introduction and section "Recipe and calibration"): weights in
 * OCP E4M3 with one scale per 128x128 block ("standard minmax"), activations
 * quantized dynamically per token in groups of 128, the GEMM accumulated in FP32
 * and written as BF16 (the model is served with --dtype bfloat16, section
 * "Serving").  The card fixes no API; these calls are this library's own.
 *
 * Conventions shared by every call:
 *   - All tensors are dense, row-major and live in device memory of the current
 *     HIP device.  The caller owns every buffer; the library allocates no memory
 *     and keeps no per-call state.
 *   - BF16 tensors are passed as raw 16-bit patterns, E4M3 tensors as bytes.
 *   - Shapes: K (and N) must be multiples of 128; M >= 0 (M == 0 is a no-op).
 *   - Alignment: BF16 and E4M3 tensors 16-byte aligned, FP32 scale tensors 4-byte
 *     aligned.
 *   - Calls only enqueue work on `stream` (NULL = the device's null stream) and
 *     never synchronize.  Validation happens on the host before any launch and is
 *     reported synchronously; a fault inside a kernel surfaces at the caller's
 *     next synchronization, as for any HIP library.
 *   - Inputs must be finite.  NaN or infinity in an input is outside the contract.
 *   - Return value: FP8BS_OK (0) or a negative fp8bs_status code.
 *   - The device must be gfx950; other devices get FP8BS_ERR_DEVICE.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8BS_OK = 0,
    FP8BS_ERR_NULL = -1,      /* a required pointer is NULL                       */
    FP8BS_ERR_SHAPE = -2,     /* negative size, K or N not a multiple of 128, or  */
                              /* an index range that overflows int64            */
    FP8BS_ERR_ALIGN = -3,     /* a pointer violates the alignment rule above      */
    FP8BS_ERR_DEVICE = -4,    /* the current device is not gfx950                 */
    FP8BS_ERR_HIP = -5,       /* a HIP runtime call or a kernel launch failed     */
    FP8BS_ERR_WORKSPACE = -6, /* workspace given but misaligned; or, without      */
                              /* allocation, more scratch needed than the library holds */
    FP8BS_ERR_VALUE = -7      /* a scalar argument out of range (eps <= 0, non-finite g) */
} fp8bs_status;

/*
 * Dynamic per-token, group-128 activation quantization.
 * Defined by the "Nanbeige4.3-33B FP8" model card: its introduction gives E4M3 codes
 * with dynamic activation scales per token and group of 128, and its section
 * "Recipe and calibration" calls the scales standard minmax (data independent).
 * The scale type (FP32), the scale formula amax / 448, the float32 quotient, the
 * rounding and the zero-group rule below are this library's readings of that text.
 *   x_bf16 [M, K]      BF16 input (in).
 *   q_e4m3 [M, K]      E4M3 codes (out).
 *   s_f32  [M, K/128]  scales (out); s[m, g] covers x[m, 128 g .. 128 g + 127].
 * For every group: s = fl32(amax / 448) with amax the largest |x| of the group
 * (IEEE float32 division, round to nearest even, subnormals kept);
 * q = E4M3(fl32(x / s)) rounded to nearest even and saturated at +-448.  A group
 * whose amax is 0 gets s = +0.0 and codes 0x00.  Bit-exact and deterministic.
 * Ownership: x is read only; q and s are written completely (every element).
 * Errors: FP8BS_ERR_SHAPE (K not a multiple of 128, M < 0, overflow),
 * FP8BS_ERR_NULL, FP8BS_ERR_ALIGN, FP8BS_ERR_DEVICE, FP8BS_ERR_HIP; on an error
 * nothing is enqueued.
 */
int fp8_quant_act(const void* x_bf16, void* q_e4m3, float* s_f32,
                  int64_t M, int64_t K, hipStream_t stream);

/*
 * 128x128 block weight quantization (offline step; same rounding as above).
 * "Nanbeige4.3-33B FP8" card, "Recipe and calibration": one scale per 128x128 weight
 * block from standard minmax quantization, which needs no calibration data.
 *   w_bf16  [N, K]            BF16 weights, row n = output channel n (in).
 *   qw_e4m3 [N, K]            E4M3 codes (out).
 *   ws_f32  [N/128, K/128]    scales (out); ws[i, j] covers rows 128 i .. 128 i + 127
 *                             and columns 128 j .. 128 j + 127.
 * N and K must be multiples of 128.
 */
int fp8_quant_weight(const void* w_bf16, void* qw_e4m3, float* ws_f32,
                     int64_t N, int64_t K, hipStream_t stream);

/*
 * Input of the down projection: h = BF16(silu(gate) * up), then the activation
 * quantization above applied to h ("Nanbeige4.3-33B DFlash2" card, "Architecture and
 * checkpoint format": separate gate and up tensors, MLP width 8192).
 *   gu_bf16 [M, 2 I]    fused gate/up output: gate = columns [0, I), up = [I, 2 I).
 *   q_e4m3  [M, I]      E4M3 codes of h (out).
 *   s_f32   [M, I/128]  scales of h (out).
 * silu(g) = g / (1 + exp(-g)); the product is evaluated in FP64 and rounded to
 * BF16 once (nearest even).  I must be a multiple of 128.
 */
int fp8_silu_mul_quant(const void* gu_bf16, void* q_e4m3, float* s_f32,
                       int64_t M, int64_t I, hipStream_t stream);

/*
 * Input of the q/k/v projection: h = BF16(RMSNorm(x) * gamma), then the activation
 * quantization above applied to h ("Nanbeige4.3-33B DMS sidecar" card, "Format and
 * hipEngine compatibility": the normalized stage before the q projection;
 * "Nanbeige4.3-33B DFlash2" card, architecture table: RMS epsilon 1e-5).
 *   x_bf16     [M, K]      hidden states (in).
 *   gamma_bf16 [K]         RMSNorm weight (in), 16-byte aligned.
 *   eps                    added to the mean square; finite and > 0, else
 *                          FP8BS_ERR_VALUE.
 *   q_e4m3     [M, K]      E4M3 codes of h (out).
 *   s_f32      [M, K/128]  scales of h (out).
 * h[m, k] = x[m, k] / sqrt(mean_k x[m, k]^2 + eps) * gamma[k], evaluated in FP64
 * (eps widened exactly; the reciprocal square root within a few FP64 ulps) and
 * rounded to BF16 once (nearest even).  K must be a multiple of 128.  Deterministic.
 */
int fp8_rmsnorm_quant(const void* x_bf16, const void* gamma_bf16, float eps,
                      void* q_e4m3, float* s_f32, int64_t M, int64_t K, hipStream_t stream);

/*
 * Block-scaled FP8 GEMM: y = (q * s) @ (w * ws)^T, accumulated in FP32, stored BF16.
 * Defined by the "Nanbeige4.3-33B FP8" model card: introduction and "Recipe and
 * calibration" (E4M3 weights with one scale per 128x128 block, activations with
 * dynamic per-token group-128 scales), "Serving" (the model runs with --dtype
 * bfloat16, hence a BF16 output) and "Compatibility and limitations" (results are
 * not promised bit-identical across kernel geometries, hence a tolerance rather than
 * one summation order).
 *   q_e4m3  [M, K]            activation codes; s_f32 [M, K/128] their scales.
 *   w_e4m3  [N, K]            weight codes;     ws_f32 [N/128, K/128] block scales.
 *   y_bf16  [M, N]            output (out), rounded to BF16 (nearest even) once.
 *   workspace / workspace_bytes
 *       Optional device scratch, sized by fp8_block_linear_workspace_size.  With it,
 *       a batch too small to give every CU a tile (32 < M up to a few hundred tokens)
 *       splits K over the workgroups of each tile: FP32 partial sums go to the
 *       workspace and a second kernel adds them in a fixed order.  NULL / 0, or a
 *       smaller workspace, selects a schedule that fits (never an error); it must be
 *       256-byte aligned (else FP8BS_ERR_WORKSPACE).  Calls that share one must not
 *       overlap.
 * Per 128-wide K block the FP32 partial product is multiplied by s[m, kb] *
 * ws[n/128, kb] and added to an FP32 accumulator.  The summation order is fixed
 * for a given (M, N, K, device, workspace size), so repeated calls give
 * bitwise-identical outputs.  Accuracy: |y - ref| <= 4e-3 |ref| + 1e-3 rms(ref)
 * against the exact dequantize-and-matmul.
 * Ownership: q, s, w, ws are read only; y is written completely; the workspace
 * is scratch the call may overwrite.  Errors: FP8BS_ERR_SHAPE (K <= 0, K or N not a
 * multiple of 128, overflow), FP8BS_ERR_NULL, FP8BS_ERR_ALIGN, FP8BS_ERR_WORKSPACE,
 * FP8BS_ERR_DEVICE, FP8BS_ERR_HIP; on an error nothing is enqueued.
 */
int fp8_block_linear(const void* q_e4m3, const float* s_f32,
                     const void* w_e4m3, const float* ws_f32,
                     void* y_bf16, int64_t M, int64_t N, int64_t K,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fp8_block_linear for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and schedules as fp8_block_linear with a workspace of
 * FP8BS_NOALLOC_SCRATCH_BYTES, except that the split-K partial sums go to a static
 * device array inside the library (one per GPU, held until the process ends); the
 * call allocates nothing.  The caller still passes inputs and outputs.  Shapes whose
 * workspace size (fp8_block_linear_workspace_size) exceeds that array get
 * FP8BS_ERR_WORKSPACE; on devices of up to 256 CUs no valid shape does.  Every call
 * on one GPU shares its array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialized by the caller.  Nothing in the array needs
 * clearing: each call writes every partial it reads.
 */
#define FP8BS_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int fp8_block_linear_noalloc(const void* q_e4m3, const float* s_f32,
                             const void* w_e4m3, const float* ws_f32,
                             void* y_bf16, int64_t M, int64_t N, int64_t K, hipStream_t stream);

/* Bytes of workspace the fastest schedule of fp8_block_linear can use for this shape
 * on devices of up to 256 CUs (0 if none: M <= 32, and prefill shapes with enough
 * tiles; 0 for invalid shapes as well). */
size_t fp8_block_linear_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * NVFP4 weight-only linear (W4A16): y = x @ W^T with BF16 activations and
 *   W[n, k] = e2m1(code[n, k]) * e4m3(bs[n, k/16]) * g.
 * The scheme of the "Nanbeige4.3-33B-NVFP4-A16" model card (paragraph on the base
 * revision and calibration): FP4 E2M1 weights in groups of 16 along K, an E4M3
 * scale per group and a global weight scale; activations are not quantized.  The
 * card's serving layout keeps packed FP4 values and block scales and stores the
 * global scale as a multiplier.
 *   x_bf16   [M, K]     BF16 activations (in).
 *   w_fp4    [N, K/2]   packed codes (in): byte j of row n holds element 2j in bits
 *                       0-3 and element 2j+1 in bits 4-7.  A code is OCP MX E2M1 (sign,
 *                       2 exponent bits with bias 1, 1 mantissa bit: +-{0, 0.5, 1, 1.5,
 *                       2, 3, 4, 6}).
 *   bs_e4m3  [N, K/16]  group scales (in), OCP E4M3 bytes; the NaN codes 0x7F / 0xFF
 *                       are outside the contract.
 *   g                   global scale, any finite float32 (else FP8BS_ERR_VALUE).
 *   y_bf16   [M, N]     output (out): fl32(g * acc) rounded to BF16 (nearest even).
 *   workspace / workspace_bytes
 *       Optional device scratch, sized by nvfp4_w4a16_workspace_size.  With it, a
 *       batch too small to give every CU a tile (a few hundred tokens) splits K over
 *       workgroups: FP32 partial sums go to the workspace and a second kernel adds
 *       them in a fixed order.  NULL / 0, or a smaller workspace, selects a schedule
 *       that fits (never an error); a workspace must be 256-byte aligned
 *       (else FP8BS_ERR_WORKSPACE).  The caller owns it; calls that share one must
 *       not overlap.
 * Shapes follow the shared rule (K and N multiples of 128).  Alignment: x, w, y and
 * bs 16-byte aligned.  Each product e2m1 * e4m3 is exact in BF16 and each product
 * with x exact in FP32; acc is their FP32 sum in an order fixed for a given
 * (M, N, K, device, workspace size), so repeated calls give bitwise-identical
 * outputs.  Accuracy: |y - ref| <= 4e-3 |ref| + 1e-3 rms(ref) against the exact
 * dequantize-and-matmul.
 */
int nvfp4_w4a16_linear(const void* x_bf16, const void* w_fp4, const void* bs_e4m3, float g,
                       void* y_bf16, int64_t M, int64_t N, int64_t K,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace the fastest schedule of nvfp4_w4a16_linear can use for this shape
 * on devices of up to 256 CUs (0 if none: decode shapes and large M; 0 for invalid
 * shapes as well). */
size_t nvfp4_w4a16_workspace_size(int64_t M, int64_t N, int64_t K);

/* Static, human-readable text for a status code. */
const char* fp8bs_status_string(int status);

/* ABI version of this header: major * 10000 + minor * 100 + patch. */
int fp8bs_abi_version(void);

#define FP8BS_ABI_VERSION 10400

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
