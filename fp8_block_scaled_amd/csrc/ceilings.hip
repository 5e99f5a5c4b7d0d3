// Measured ceilings of this GPU, for the bench (not part of the product ABI, not
// declared in include/fp8bs.h; built into libfp8bs_ceilings.so):
//   * a plain streaming read of a device buffer: the best HBM read rate a kernel
//     reaches at a given byte count, next to the published 8 TB/s;
//   * a loop of FP8 MFMAs (16x16x128, E4M3 x E4M3 -> FP32) on register operands,
//     alone and with the per-K-block promotion of the block-scaled GEMM (four FP32
//     FMAs per MFMA result): the MFMA rate reached, next to the published 5 PFLOP/s,
//     and the rate the promotion leaves;
//   * the shader clock while that loop runs: s_memtime (shader clock counter) over
//     s_memrealtime (constant-rate counter) read by one lane at its start and end.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Each workgroup reads one contiguous range of the buffer, U 16-byte loads in
// flight per lane; the loaded words are folded into one value that is stored only
// if it equals a value the buffer never produces here, so the loads stay and no
// write traffic is added.
template <int U, bool NT>
__global__ __launch_bounds__(1024) void stream_read_kernel(const v4i* __restrict__ buf, int64_t n16, int64_t per_wg,
                                                           int* __restrict__ sink) {
    const int64_t begin = (int64_t)blockIdx.x * per_wg;
    int64_t end = begin + per_wg;
    end = end < n16 ? end : n16;
    v4i acc = {0, 0, 0, 0};
    const int64_t stride = (int64_t)blockDim.x * U;
    for (int64_t i = begin + threadIdx.x; i < end; i += stride) {
        v4i v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = i + (int64_t)u * blockDim.x;
            const int64_t jj = j < end ? j : begin;
            v[u] = NT ? __builtin_nontemporal_load(buf + jj) : buf[jj];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    const int folded = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (folded == 0x7F3A5C11) sink[blockIdx.x * blockDim.x + threadIdx.x] = folded;
}

// CH independent chains of v_mfma_f32_16x16x128_f8f6f4 per wave.  PROMOTE: each MFMA
// starts from zero and its result is folded into an accumulator by four FMAs, as the
// GEMM does per 128-wide K block; otherwise the MFMA accumulates in place.  An
// operand is made opaque before every MFMA, so none is merged or hoisted.
// Two waves per SIMD, as in the GEMM: 256 registers per wave, so the MFMA results stay
// in the VGPRs the FMAs read (no AGPR copies).
template <bool PROMOTE, int CH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_loop_kernel(int iters, float* __restrict__ out,
                                                        unsigned long long* __restrict__ clk) {
    const int lane = threadIdx.x & 63;
    v8i a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = 0x38383838 ^ (lane * 0x01010101 & 0x07070707);   // E4M3 values near 1
        b[i] = 0x30303030 ^ (i * 0x01010101);
    }
    v4f acc[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    const float sc = 1.0f + 1e-7f * lane;
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
    unsigned long long t0 = 0, r0 = 0;
    if (timer) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            asm volatile("" : "+v"(a));          // every MFMA sees a new operand: no CSE, no hoisting
            if (PROMOTE) {
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
                acc[c][0] = fmaf(sc, p[0], acc[c][0]);
                acc[c][1] = fmaf(sc, p[1], acc[c][1]);
                acc[c][2] = fmaf(sc, p[2], acc[c][2]);
                acc[c][3] = fmaf(sc, p[3], acc[c][3]);
            } else {
                acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
            }
        }
    }
    if (timer) {
        // The wave's MFMAs have retired once their results are read below; read the
        // counters after that.
        float s0 = 0.0f;
#pragma unroll
        for (int c = 0; c < CH; ++c) s0 += acc[c][0];
        asm volatile("" : "+v"(s0));
        const unsigned long long t1 = __builtin_amdgcn_s_memtime();
        const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
        clk[0] = t1 - t0;
        clk[1] = r1 - r0;
        acc[0][0] = s0;
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a multiple of 16, 16-byte aligned) from `buf` with
// `wgs` workgroups of `threads` threads (64..1024, a multiple of 64), `unroll` in
// {2, 4, 8} loads in flight per lane, nontemporal loads if `nt`.  `sink` must hold
// wgs * threads ints (never written in practice).  Returns a hipError_t.
int fp8bs_ceil_stream_read(const void* buf, int64_t bytes, int* sink, int wgs, int threads, int unroll, int nt,
                           hipStream_t st) {
    if (!buf || !sink || bytes <= 0 || bytes % 16 || wgs <= 0 || threads < 64 || threads > 1024 || threads % 64)
        return (int)hipErrorInvalidValue;
    const int64_t n16 = bytes / 16;
    const int64_t per_wg = (n16 + wgs - 1) / wgs;
    const v4i* b = (const v4i*)buf;
#define FP8BS_SR(U, NT)                                                                                   \
    hipLaunchKernelGGL((stream_read_kernel<U, NT>), dim3((unsigned)wgs), dim3(threads), 0, st, b, n16, per_wg, sink)
    if (unroll <= 2) {
        if (nt) FP8BS_SR(2, true); else FP8BS_SR(2, false);
    } else if (unroll <= 4) {
        if (nt) FP8BS_SR(4, true); else FP8BS_SR(4, false);
    } else {
        if (nt) FP8BS_SR(8, true); else FP8BS_SR(8, false);
    }
#undef FP8BS_SR
    return (int)hipGetLastError();
}

// `wgs` workgroups of 4 waves, each wave `iters` x 8 chains of FP8 MFMAs (65,536 flop
// each), with the promotion FMAs if `promote`.  `out` holds wgs * 256 floats, `clk`
// two counts (shader clock ticks, constant-rate ticks) of workgroup 0's first wave.
int fp8bs_ceil_mfma(int wgs, int iters, int promote, float* out, unsigned long long* clk, hipStream_t st) {
    if (!out || !clk || wgs <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
    if (promote)
        hipLaunchKernelGGL((mfma_loop_kernel<true, 8>), dim3((unsigned)wgs), dim3(256), 0, st, iters, out, clk);
    else
        hipLaunchKernelGGL((mfma_loop_kernel<false, 8>), dim3((unsigned)wgs), dim3(256), 0, st, iters, out, clk);
    return (int)hipGetLastError();
}

// Rate of the constant-rate counter read by s_memrealtime, in kHz (0 on error).
int fp8bs_ceil_wallclock_khz(void) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return v;
}

}  // extern "C"
