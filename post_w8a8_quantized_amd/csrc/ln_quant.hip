// Fused prologue for gfx950: LayerNorm or GeLU (or nothing) in fp32 registers,
// then dynamic per-token symmetric absmax quantization to int8.
//
// Pages: ZeroQuant reading notes, kernel-fusion flowchart (LN/GeLU + Quantize
// in one kernel); "探秘Transformer系列之（36）--- 大模型量化方案" 1.2.2 (token-wise
// scales computed at run time; fusing the quantizer with the preceding
// LayerNorm removes a round trip through HBM) and 1.1.2 (absmax to [-127, 127]).
//
// Layout: one token row of X is read once with 16-byte loads (8 fp16 or 2x4
// fp32 per chunk), kept in registers, reduced across the wave (and across
// waves through LDS for long rows), quantized and written back as 8-byte
// groups of codes.  The kernel is HBM-bound: per token it moves
// K * sizeof(x) bytes in, K + 4 bytes out.
#include "zq_device.h"
#include "zq_kernels.h"

namespace zq {
namespace {

// One 16-byte piece of a row: 8 fp16 (one load) or 8 fp32 (two loads), kept
// in its storage type so that a lane holds long rows in few registers.
template <typename T>
struct Chunk;

template <>
struct Chunk<_Float16> {
    h8 h;
    __device__ __forceinline__ void load(const _Float16 *p) { h = *reinterpret_cast<const h8 *>(p); }
    __device__ __forceinline__ void zero() { h = h8{0, 0, 0, 0, 0, 0, 0, 0}; }
    __device__ __forceinline__ float operator[](int i) const { return (float)h[i]; }
};

template <>
struct Chunk<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p)
    {
        a = *reinterpret_cast<const float4 *>(p);
        b = *reinterpret_cast<const float4 *>(p + 4);
    }
    __device__ __forceinline__ void zero() { a = b = float4{0.f, 0.f, 0.f, 0.f}; }
    __device__ __forceinline__ float operator[](int i) const
    {
        switch (i) {
        case 0: return a.x; case 1: return a.y; case 2: return a.z; case 3: return a.w;
        case 4: return b.x; case 5: return b.y; case 6: return b.z; default: return b.w;
        }
    }
};

__device__ __forceinline__ void load8(const float *p, float (&v)[8])
{
    float4 a = *reinterpret_cast<const float4 *>(p);
    float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// The fused op applied to the 8 elements of chunk c (c < K/8).
template <typename T>
__device__ __forceinline__ void pre_op(const Chunk<T> &x, int c, int pre, float mean, float rstd,
                                       const float *__restrict__ gamma,
                                       const float *__restrict__ beta, float (&y)[8])
{
    if (pre == 1) {
        float g[8], b[8];
        if (gamma) {
            load8(gamma + c * 8, g);
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++) g[e] = 1.0f;
        }
        if (beta) {
            load8(beta + c * 8, b);
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++) b[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; e++)
            y[e] = (x[e] - mean) * rstd * g[e] + b[e];
    } else if (pre == 2) {
#pragma unroll
        for (int e = 0; e < 8; e++)
            y[e] = gelu_erf(x[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
            y[e] = x[e];
    }
}

// Block = TPB tokens x WPT waves per token.  Thread t of a token owns chunks
// t, t + 64*WPT, ... (NCH of them) so that consecutive lanes read consecutive
// 16-byte pieces of the row.  The row is read from HBM once; y is recomputed
// from the registers for the absmax pass and again for the quantize pass.
template <typename T, int NCH, int WPT, int TPB>
__global__ __launch_bounds__(kWave * WPT * TPB) void k_ln_quant(
    const T *__restrict__ X, int M, int K, int pre, const float *__restrict__ gamma,
    const float *__restrict__ beta, float eps, int8_t *__restrict__ Xq, float *__restrict__ sx)
{
    constexpr int TT = kWave * WPT;  // threads per token
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int tok_in_blk = wave / WPT;
    const int t = (wave % WPT) * kWave + lane;
    const int64_t m = (int64_t)blockIdx.x * TPB + tok_in_blk;
    const bool live = m < M;
    const int nchunks = K / 8;

    __shared__ float red[TPB][WPT > 1 ? WPT : 1];

    // Combine one value per thread over the token's threads; every thread of
    // the token gets the same result (fixed order, so deterministic).
    auto token_reduce = [&](float v, bool is_max) -> float {
        v = is_max ? wave_max(v) : wave_sum(v);
        if constexpr (WPT > 1) {
            if (lane == 0)
                red[tok_in_blk][wave % WPT] = v;
            __syncthreads();
            float r = red[tok_in_blk][0];
#pragma unroll
            for (int w = 1; w < WPT; w++)
                r = is_max ? fmaxf(r, red[tok_in_blk][w]) : r + red[tok_in_blk][w];
            __syncthreads();
            v = r;
        }
        return v;
    };

    Chunk<T> x[NCH];
    const T *xrow = X + m * (int64_t)K;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int c = t + TT * i;
        if (live && c < nchunks)
            x[i].load(xrow + (int64_t)c * 8);
        else
            x[i].zero();
    }

    float mean = 0.0f, rstd = 0.0f;
    if (pre == 1) {  // LayerNorm statistics, two passes over the registers
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; i++)
#pragma unroll
            for (int e = 0; e < 8; e++)
                s += x[i][e];
        mean = token_reduce(s, false) / (float)K;
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            if (t + TT * i < nchunks) {
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float d = x[i][e] - mean;
                    ss += d * d;
                }
            }
        }
        const float var = token_reduce(ss, false) / (float)K;
        rstd = 1.0f / sqrtf(var + eps);
    }

    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int c = t + TT * i;
        if (c < nchunks) {
            float y[8];
            pre_op(x[i], c, pre, mean, rstd, gamma, beta, y);
#pragma unroll
            for (int e = 0; e < 8; e++)
                a = fmaxf(a, fabsf(y[e]));
        }
    }
    a = token_reduce(a, true);
    const float scale = a / 127.0f;

    if (!live)
        return;
    int8_t *qrow = Xq + m * (int64_t)K;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int c = t + TT * i;
        if (c < nchunks) {
            float y[8];
            pre_op(x[i], c, pre, mean, rstd, gamma, beta, y);
            uint2 packed;
            packed.x = pack4_i8(quant_code(y[0], scale), quant_code(y[1], scale),
                                quant_code(y[2], scale), quant_code(y[3], scale));
            packed.y = pack4_i8(quant_code(y[4], scale), quant_code(y[5], scale),
                                quant_code(y[6], scale), quant_code(y[7], scale));
            *reinterpret_cast<uint2 *>(qrow + (int64_t)c * 8) = packed;
        }
    }
    if (t == 0)
        sx[m] = scale;
}

template <typename T, int WPT, int TPB>
hipError_t launch_cfg(const T *X, int64_t M, int64_t K, int pre, const float *gamma,
                      const float *beta, float eps, int8_t *Xq, float *sx, hipStream_t stream)
{
    const int64_t nchunks = K / 8;
    const int64_t per = (nchunks + kWave * WPT - 1) / (kWave * WPT);
    const dim3 grid((unsigned)((M + TPB - 1) / TPB));
    const dim3 block(kWave * WPT * TPB);
#define ZQ_LNQ_CASE(n)                                                                          \
    if (per <= n) {                                                                             \
        hipLaunchKernelGGL((k_ln_quant<T, n, WPT, TPB>), grid, block, 0, stream, X, (int)M,     \
                           (int)K, pre, gamma, beta, eps, Xq, sx);                              \
        return hipGetLastError();                                                               \
    }
    ZQ_LNQ_CASE(1)
    ZQ_LNQ_CASE(2)
    ZQ_LNQ_CASE(3)
    ZQ_LNQ_CASE(4)
    ZQ_LNQ_CASE(6)
    ZQ_LNQ_CASE(8)
    ZQ_LNQ_CASE(10)
    ZQ_LNQ_CASE(12)
    ZQ_LNQ_CASE(16)
#undef ZQ_LNQ_CASE
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_typed(const T *X, int64_t M, int64_t K, int pre, const float *gamma,
                        const float *beta, float eps, int8_t *Xq, float *sx, hipStream_t stream)
{
    // Rows up to 64 lanes x 16 chunks x 8 = 8192 elements: one wave per token,
    // four tokens per block.  Longer rows: 16 waves per token.
    if (K <= 8192)
        return launch_cfg<T, 1, 4>(X, M, K, pre, gamma, beta, eps, Xq, sx, stream);
    return launch_cfg<T, 16, 1>(X, M, K, pre, gamma, beta, eps, Xq, sx, stream);
}

}  // namespace

hipError_t launch_ln_quant(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                           const float *gamma, const float *beta, float eps, int8_t *Xq,
                           float *x_scales, hipStream_t stream)
{
    if (x_f16)
        return launch_typed(static_cast<const _Float16 *>(X), M, K, pre, gamma, beta, eps, Xq,
                            x_scales, stream);
    return launch_typed(static_cast<const float *>(X), M, K, pre, gamma, beta, eps, Xq, x_scales,
                        stream);
}

}  // namespace zq
