// The unfused order of the layer, built only to measure what the fusion saves.
//
// ZeroQuant reading notes, kernel-fusion figure: before fusion the LayerNorm
// (or GeLU) writes an FP16 tensor, a separate kernel quantizes it per token,
// the INT8 GEMM writes its INT32 accumulators, and a separate kernel
// dequantizes them; after fusion the quantizer lives in the LN/GeLU kernel
// and the dequantization in the GEMM's epilogue ("探秘Transformer系列之（36）---
// 大模型量化方案" 1.2.2 describes the fused form).  The unfused layer here reuses
// the library's own kernels for the op (fp16 output mode), the quantizer
// (no op) and the GEMM (int32 output mode); this file adds the dequantizer.
#include "zq_device.h"
#include "zq_kernels.h"

#include <algorithm>

namespace zq {
namespace {

// Y[m, n] = fp16(s_x[m] s_w[n / G] acc[m, n] + bias[n]), optional GeLU, with
// the same expression as the fused epilogues.  One thread per 4 outputs
// (N % 4 == 0): a 16-byte int32 load and an 8-byte fp16 store.
__global__ __launch_bounds__(256) void k_dequant(const int32_t *__restrict__ acc,
                                                 const float *__restrict__ sx,
                                                 const float *__restrict__ sw, int G,
                                                 const float *__restrict__ bias, int act, int M,
                                                 int N, _Float16 *__restrict__ Y)
{
    const int64_t quads = (int64_t)M * (N / 4);
    for (int64_t q = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; q < quads;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = q / (N / 4);
        const int n = (int)(q % (N / 4)) * 4;
        const v4i a = *reinterpret_cast<const v4i *>(acc + m * N + n);
        const float sxm = sx[m];
        h4 o;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float v = fmaf((float)a[i], sxm * sw[(n + i) / G], bias ? bias[n + i] : 0.0f);
            if (act == 1)
                v = gelu_fast(v);
            o[i] = (_Float16)v;
        }
        *reinterpret_cast<h4 *>(Y + m * N + n) = o;
    }
}

}  // namespace

hipError_t launch_dequant(const int32_t *acc, const float *x_scales, const float *w_scales,
                          int64_t G, const float *bias, int act, int64_t M, int64_t N, void *Y,
                          hipStream_t stream)
{
    const int64_t quads = M * (N / 4);
    const int64_t blocks = std::min<int64_t>((quads + 255) / 256, 4096);
    hipLaunchKernelGGL(k_dequant, dim3((unsigned)blocks), dim3(256), 0, stream, acc, x_scales,
                       w_scales, (int)G, bias, act, (int)M, (int)N, static_cast<_Float16 *>(Y));
    return hipGetLastError();
}

}  // namespace zq
