// Weight-streaming int8 GEMM for few tokens (M <= 32), the decode shape (gfx950).
//
// Same result as the tiled kernel: Y[m, n] = fp16(s_x[m] s_w[n/G] acc[m, n] + bias[n]),
// optional GeLU ("探秘Transformer系列之（36）--- 大模型量化方案" 1.2.2 and 1.1.2;
// ZeroQuant reading notes, "GeMM + DeQuantize").  With a handful of tokens
// the int8 weight stream dominates: the layer is bound by HBM bandwidth
// ("Integer Quantization: Deep Dive": decoding is memory-bandwidth bound).
//
// Design for CDNA4:
//  - v_mfma_i32_16x16x64_i8 with W as the A operand (16 output rows) and X as
//    the B operand (16 tokens): one instruction consumes 16 rows x 64 bytes
//    of W, so the matrix cores absorb the whole 16-token product and the VALU
//    stays idle.
//  - W is read straight from HBM into registers (no LDS): each lane loads
//    16 bytes of one row; a wave's UNROLL loads cover 16 rows x 64*UNROLL
//    contiguous bytes, i.e. whole cache lines.  X (M x K int8, at most
//    896 KB) is re-read from L2.
//  - A workgroup owns 16 output rows; its NWAVE waves split K into contiguous
//    ranges so that many 16-byte loads per CU are in flight.  Partial int32
//    sums are combined through LDS in a fixed order (deterministic, no atomics).
#include "zq_device.h"
#include "zq_kernels.h"

namespace zq {
namespace {

template <int MT, int NWAVE, int UNROLL, bool OUT_I32>
__global__ __launch_bounds__(NWAVE *kWave) void k_gemm_skinny(
    const int8_t *__restrict__ Xq, const float *__restrict__ sx, const int8_t *__restrict__ Wq,
    const float *__restrict__ sw, int G, const float *__restrict__ bias, int act, int M, int N,
    int K, void *__restrict__ Y)
{
    __shared__ v4i part[NWAVE][MT][kWave];

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int n0 = blockIdx.x * 16;
    const int r16 = lane & 15;   // operand row within the 16-row block
    const int kq = lane >> 4;    // which 16-byte quarter of a 64-byte k block

    const int n = min(n0 + r16, N - 1);  // ragged N: re-read the last row, never stored
    const int8_t *wrow = Wq + (int64_t)n * K + kq * 16;
    const int8_t *xrow[MT];
#pragma unroll
    for (int t = 0; t < MT; t++)
        xrow[t] = Xq + (int64_t)min(16 * t + r16, M - 1) * K + kq * 16;

    // Contiguous k-block range of this wave (64-byte blocks, last one may be partial).
    const int nkb = (K + 63) / 64;
    const int per = (nkb + NWAVE - 1) / NWAVE;
    const int kb_begin = wave * per;
    const int kb_end = min(nkb, kb_begin + per);

    v4i acc[MT];
#pragma unroll
    for (int t = 0; t < MT; t++)
        acc[t] = v4i{0, 0, 0, 0};

    for (int kb = kb_begin; kb < kb_end; kb += UNROLL) {
        v4i w[UNROLL], x[UNROLL][MT];
#pragma unroll
        for (int u = 0; u < UNROLL; u++) {
            const int k = (kb + u) * 64 + kq * 16;
            const bool ok = (kb + u < kb_end) && (k < K);
            w[u] = ok ? *reinterpret_cast<const v4i *>(wrow + (int64_t)(kb + u) * 64) : v4i{0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < MT; t++)
                x[u][t] = ok ? *reinterpret_cast<const v4i *>(xrow[t] + (int64_t)(kb + u) * 64)
                             : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < UNROLL; u++)
#pragma unroll
            for (int t = 0; t < MT; t++)
                acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[u], x[u][t], acc[t], 0, 0, 0);
    }

#pragma unroll
    for (int t = 0; t < MT; t++)
        part[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int t = 0; t < MT; t++) {
        v4i s = part[0][t][lane];
#pragma unroll
        for (int w = 1; w < NWAVE; w++)
            s += part[w][t][lane];
        acc[t] = s;
    }

    // Accumulator register r holds token m = 16 t + lane % 16 and
    // output row n = n0 + 4 * (lane / 16) + r.
#pragma unroll
    for (int t = 0; t < MT; t++) {
        const int m = 16 * t + r16;
        const int nn = n0 + 4 * kq;
        if (m >= M || nn >= N)
            continue;
        if constexpr (OUT_I32) {
            *reinterpret_cast<v4i *>(static_cast<int32_t *>(Y) + (int64_t)m * N + nn) = acc[t];
        } else {
            const float sxm = sx[m];
            h4 o;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float v = (float)acc[t][i] * (sxm * sw[(nn + i) / G]);
                if (bias)
                    v += bias[nn + i];
                if (act == 1)
                    v = gelu_erf(v);
                o[i] = (_Float16)v;
            }
            *reinterpret_cast<h4 *>(static_cast<_Float16 *>(Y) + (int64_t)m * N + nn) = o;
        }
    }
}

template <int MT, int NWAVE, int UNROLL>
hipError_t launch_cfg(const int8_t *Xq, const float *sx, const int8_t *Wq, const float *sw,
                      int64_t G, const float *bias, int act, int64_t M, int64_t N, int64_t K,
                      void *Y, bool out_i32, hipStream_t stream)
{
    const dim3 grid((unsigned)((N + 15) / 16));
    const dim3 block(NWAVE * kWave);
    if (out_i32)
        hipLaunchKernelGGL((k_gemm_skinny<MT, NWAVE, UNROLL, true>), grid, block, 0, stream, Xq,
                           sx, Wq, sw, (int)G, bias, act, (int)M, (int)N, (int)K, Y);
    else
        hipLaunchKernelGGL((k_gemm_skinny<MT, NWAVE, UNROLL, false>), grid, block, 0, stream, Xq,
                           sx, Wq, sw, (int)G, bias, act, (int)M, (int)N, (int)K, Y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_skinny(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                              const float *w_scales, int64_t G, const float *bias, int act,
                              int64_t M, int64_t N, int64_t K, void *Y, bool out_i32,
                              hipStream_t stream)
{
    if (M <= 16)
        return launch_cfg<1, 8, 4>(Xq, x_scales, Wq, w_scales, G, bias, act, M, N, K, Y, out_i32,
                                   stream);
    return launch_cfg<2, 8, 4>(Xq, x_scales, Wq, w_scales, G, bias, act, M, N, K, Y, out_i32,
                               stream);
}

}  // namespace zq
