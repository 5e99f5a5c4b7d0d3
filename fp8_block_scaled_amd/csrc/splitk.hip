// Split-K reduce shared by the FP8 prefill GEMM (g = 1) and the NVFP4 tiles (g = the
// global weight scale): y = BF16(g * sum over ks of part[ks]), summed in the order
// ks = 0, 1, ..., so a given split gives the same bits on every call.  Four
// neighbouring elements per thread; M N is a multiple of 4 (N is a multiple of 128
// in both callers).  HBM-bound: 4 ksplit + 2 bytes per output element.
#include "device_common.h"
#include "launch.h"

namespace fp8bs {

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* part, int ksplit, int64_t mn, float g,
                                                                 uint16_t* y) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= mn) return;
    v4f sum = *reinterpret_cast<const v4f*>(part + i);
    for (int ks = 1; ks < ksplit; ++ks) {
        const v4f v = *reinterpret_cast<const v4f*>(part + (int64_t)ks * mn + i);
        sum[0] += v[0];
        sum[1] += v[1];
        sum[2] += v[2];
        sum[3] += v[3];
    }
    const uint32_t lo = f32_to_bf16_rne(g * sum[0]) | (f32_to_bf16_rne(g * sum[1]) << 16);
    const uint32_t hi = f32_to_bf16_rne(g * sum[2]) | (f32_to_bf16_rne(g * sum[3]) << 16);
    *reinterpret_cast<uint2*>(y + i) = make_uint2(lo, hi);
}

hipError_t launch_splitk_reduce(const float* part, int ksplit, int64_t mn, float g, uint16_t* y, hipStream_t st) {
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0, st, part, ksplit, mn,
                       g, y);
    return hipGetLastError();
}

}  // namespace fp8bs
