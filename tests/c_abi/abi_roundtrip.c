/* A plain C caller of libfp8bs (no Python, no torch): it fills BF16 activations and
 * weights from a fixed-seed generator, quantizes both, runs the block-scaled GEMM
 * through the C ABI with the workspace the size query asks for, and writes every
 * input and output to a binary file for the test to check against the oracle.
 *
 * usage: abi_roundtrip M N K SEED OUT.bin
 * file:  int64 M, N, K; then x bf16[M*K], w bf16[N*K], q u8[M*K], s f32[M*K/128],
 *        qw u8[N*K], ws f32[N/128*K/128], y bf16[M*N].  Exit status 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8bs.h"

static uint64_t state;
static double uniform01(void) {            /* 64-bit LCG, top 53 bits */
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(state >> 11) * (1.0 / 9007199254740992.0);
}
static float normal(void) {                /* Box-Muller */
    double u1 = uniform01(), u2 = uniform01();
    if (u1 < 1e-300) u1 = 1e-300;
    return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}
static uint16_t to_bf16(float f) {         /* nearest even, finite inputs */
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

#define HIP_OK(call)                                                        \
    do {                                                                    \
        hipError_t e_ = (call);                                             \
        if (e_ != hipSuccess) {                                             \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_)); \
            return 2;                                                       \
        }                                                                   \
    } while (0)
#define FB_OK(call)                                                         \
    do {                                                                    \
        int s_ = (call);                                                    \
        if (s_ != FP8BS_OK) {                                               \
            fprintf(stderr, "%s: %s\n", #call, fp8bs_status_string(s_));    \
            return 3;                                                       \
        }                                                                   \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 6) {
        fprintf(stderr, "usage: %s M N K SEED OUT.bin\n", argv[0]);
        return 1;
    }
    const int64_t M = atoll(argv[1]), N = atoll(argv[2]), K = atoll(argv[3]);
    state = strtoull(argv[4], NULL, 10);
    if (M <= 0 || N <= 0 || K <= 0 || N % 128 || K % 128) return 1;
    printf("abi version %d\n", fp8bs_abi_version());

    const size_t nx = (size_t)(M * K), nw = (size_t)(N * K), ns = nx / 128, nws = nw / (128 * 128),
                 ny = (size_t)(M * N);
    uint16_t* x = malloc(nx * 2);
    uint16_t* w = malloc(nw * 2);
    uint8_t* q = malloc(nx);
    float* s = malloc(ns * 4);
    uint8_t* qw = malloc(nw);
    float* ws = malloc(nws * 4);
    uint16_t* y = malloc(ny * 2);
    if (!x || !w || !q || !s || !qw || !ws || !y) return 4;
    for (size_t i = 0; i < nx; ++i) x[i] = to_bf16(normal());
    for (size_t i = 0; i < nw; ++i) w[i] = to_bf16(0.02f * normal());

    void *dx, *dw, *dq, *dqw, *dy, *dwk = NULL;
    float *ds, *dws;
    HIP_OK(hipMalloc(&dx, nx * 2));
    HIP_OK(hipMalloc(&dw, nw * 2));
    HIP_OK(hipMalloc(&dq, nx));
    HIP_OK(hipMalloc((void**)&ds, ns * 4));
    HIP_OK(hipMalloc(&dqw, nw));
    HIP_OK(hipMalloc((void**)&dws, nws * 4));
    HIP_OK(hipMalloc(&dy, ny * 2));
    const size_t wk = fp8_block_linear_workspace_size(M, N, K);
    if (wk) HIP_OK(hipMalloc(&dwk, wk));
    printf("workspace %zu bytes\n", wk);

    hipStream_t st;
    HIP_OK(hipStreamCreate(&st));
    HIP_OK(hipMemcpyAsync(dx, x, nx * 2, hipMemcpyHostToDevice, st));
    HIP_OK(hipMemcpyAsync(dw, w, nw * 2, hipMemcpyHostToDevice, st));
    FB_OK(fp8_quant_act(dx, dq, ds, M, K, st));
    FB_OK(fp8_quant_weight(dw, dqw, dws, N, K, st));
    FB_OK(fp8_block_linear(dq, ds, dqw, dws, dy, M, N, K, dwk, wk, st));
    HIP_OK(hipMemcpyAsync(q, dq, nx, hipMemcpyDeviceToHost, st));
    HIP_OK(hipMemcpyAsync(s, ds, ns * 4, hipMemcpyDeviceToHost, st));
    HIP_OK(hipMemcpyAsync(qw, dqw, nw, hipMemcpyDeviceToHost, st));
    HIP_OK(hipMemcpyAsync(ws, dws, nws * 4, hipMemcpyDeviceToHost, st));
    HIP_OK(hipMemcpyAsync(y, dy, ny * 2, hipMemcpyDeviceToHost, st));
    HIP_OK(hipStreamSynchronize(st));

    FILE* f = fopen(argv[5], "wb");
    if (!f) return 5;
    const int64_t dims[3] = {M, N, K};
    fwrite(dims, 8, 3, f);
    fwrite(x, 2, nx, f);
    fwrite(w, 2, nw, f);
    fwrite(q, 1, nx, f);
    fwrite(s, 4, ns, f);
    fwrite(qw, 1, nw, f);
    fwrite(ws, 4, nws, f);
    fwrite(y, 2, ny, f);
    fclose(f);

    hipStreamDestroy(st);
    hipFree(dx);
    hipFree(dw);
    hipFree(dq);
    hipFree(ds);
    hipFree(dqw);
    hipFree(dws);
    hipFree(dy);
    if (dwk) hipFree(dwk);
    free(x);
    free(w);
    free(q);
    free(s);
    free(qw);
    free(ws);
    free(y);
    printf("ok\n");
    return 0;
}
