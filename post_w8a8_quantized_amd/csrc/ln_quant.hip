// Fused prologue for gfx950: LayerNorm or GeLU (or nothing) in fp32 registers,
// then dynamic per-token symmetric absmax quantization to int8.
//
// Pages: ZeroQuant reading notes, kernel-fusion flowchart (LN/GeLU + Quantize
// in one kernel); "探秘Transformer系列之（36）--- 大模型量化方案" 1.2.2 (token-wise
// scales computed at run time; fusing the quantizer with the preceding
// LayerNorm removes a round trip through HBM) and 1.1.2 (absmax to [-127, 127]).
//
// The kernel is HBM-bound: per token it reads K * sizeof(x) bytes and writes
// K + 4.  A token row is read once with 16-byte loads (8 fp16 or 2 x 4 fp32
// per chunk; consecutive lanes take consecutive chunks), the fused op's
// result y stays in registers, the reductions (sum, sum of squares about the
// mean, absmax) run on DPP without touching LDS (and through LDS only across
// the waves of one token), and codes go out as 8-byte groups.
//
// Rows longer than 8192 without LayerNorm (the decode shape) are split over
// many workgroups when a workspace is available: one kernel writes the
// absmax of each 2048-element segment, a second reads a token's segment
// maxima in a fixed order and quantizes its segment.
#include "zq_device.h"
#include "zq_kernels.h"

namespace zq {
namespace {

// One 16-byte piece of a row: 8 fp16 (one load) or 8 fp32 (two loads).
template <typename T>
struct Chunk;

template <>
struct Chunk<_Float16> {
    static __device__ __forceinline__ void load(const _Float16 *p, float (&v)[8])
    {
        const h8 h = *reinterpret_cast<const h8 *>(p);
#pragma unroll
        for (int i = 0; i < 8; i++)
            v[i] = (float)h[i];
    }
};

template <>
struct Chunk<float> {
    static __device__ __forceinline__ void load(const float *p, float (&v)[8])
    {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

__device__ __forceinline__ void load8(const float *p, float (&v)[8])
{
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Codes of 8 values with scale s (rs = fl32(1/s), fast = rcp_quant_ok(s)).
__device__ __forceinline__ uint2 quant8(const float (&y)[8], float s, float rs, bool fast)
{
    int q[8];
    if (fast) {
#pragma unroll
        for (int e = 0; e < 8; e++)
            q[e] = quant_code_rcp(y[e], s, rs);
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
            q[e] = quant_code(y[e], s);
    }
    uint2 packed;
    packed.x = pack4_i8(q[0], q[1], q[2], q[3]);
    packed.y = pack4_i8(q[4], q[5], q[6], q[7]);
    return packed;
}

// Block = TPB tokens x WPT waves per token.  Thread t of a token owns chunks
// t, t + 64*WPT, ... (NCH of them).
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

    float y[NCH][8];
    const T *xrow = X + m * (int64_t)K;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int c = t + TT * i;
        if (live && c < nchunks) {
            Chunk<T>::load(xrow + (int64_t)c * 8, y[i]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++)
                y[i][e] = 0.0f;
        }
    }

    if (pre == 1) {  // LayerNorm: mean, then biased variance about the mean
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; i++)
#pragma unroll
            for (int e = 0; e < 8; e++)
                s += y[i][e];
        const float mean = token_reduce(s, false) / (float)K;
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            if (t + TT * i < nchunks) {
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float d = y[i][e] - mean;
                    ss += d * d;
                }
            }
        }
        const float rstd = 1.0f / sqrtf(token_reduce(ss, false) / (float)K + eps);
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int c = t + TT * i;
            if (c < nchunks) {
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
                for (int e = 0; e < 8; e++) {
                    const float a = rstd * g[e];          // y = (x - mean) * rstd * g + b
                    y[i][e] = fmaf(y[i][e], a, fmaf(-mean, a, b[e]));
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    y[i][e] = 0.0f;
            }
        }
    } else if (pre == 2) {  // exact GeLU (gelu(0) = 0 keeps the padding at 0)
#pragma unroll
        for (int i = 0; i < NCH; i++)
#pragma unroll
            for (int e = 0; e < 8; e++)
                y[i][e] = gelu_erf(y[i][e]);
    }

    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; i++)
#pragma unroll
        for (int e = 0; e < 8; e++)
            a = fmaxf(a, fabsf(y[i][e]));
    a = token_reduce(a, true);
    const float scale = a / 127.0f;
    const bool fast = rcp_quant_ok(scale);
    const float rs = fast ? 1.0f / scale : 0.0f;

    if (!live)
        return;
    int8_t *qrow = Xq + m * (int64_t)K;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int c = t + TT * i;
        if (c < nchunks)
            *reinterpret_cast<uint2 *>(qrow + (int64_t)c * 8) = quant8(y[i], scale, rs, fast);
    }
    if (t == 0)
        sx[m] = scale;
}

// ---- Split path for long rows without LayerNorm ----

constexpr int kSegThreads = 256;
constexpr int kSegChunks = 1;                          // 8-element chunks per thread
constexpr int kSegElems = kSegThreads * kSegChunks * 8;  // 2048 elements per segment

template <typename T>
__device__ __forceinline__ void seg_load(const T *xrow, int K, int seg, int pre, float (&y)[8],
                                         int &c)
{
    c = seg * (kSegElems / 8) + threadIdx.x;
    if (c < K / 8) {
        Chunk<T>::load(xrow + (int64_t)c * 8, y);
        if (pre == 2) {
#pragma unroll
            for (int e = 0; e < 8; e++)
                y[e] = gelu_erf(y[e]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
            y[e] = 0.0f;
    }
}

__device__ __forceinline__ float block_max(float v)
{
    __shared__ float red[kSegThreads / kWave];
    v = wave_max(v);
    if (threadIdx.x % kWave == 0)
        red[threadIdx.x / kWave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kSegThreads / kWave; w++)
        r = fmaxf(r, red[w]);
    return r;
}

// Grid (segments, M): partial[m * nseg + seg] = max |pre(x)| over the segment.
template <typename T>
__global__ __launch_bounds__(kSegThreads) void k_seg_absmax(const T *__restrict__ X, int K, int pre,
                                                            float *__restrict__ partial)
{
    const int seg = blockIdx.x, nseg = gridDim.x;
    const int64_t m = blockIdx.y;
    float y[8];
    int c;
    seg_load(X + m * K, K, seg, pre, y, c);
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e++)
        a = fmaxf(a, fabsf(y[e]));
    a = block_max(a);
    if (threadIdx.x == 0)
        partial[m * nseg + seg] = a;
}

// Grid (segments, M): token scale from the segment maxima (fixed order), then
// the segment's codes; segment 0 stores the scale.
template <typename T>
__global__ __launch_bounds__(kSegThreads) void k_seg_quant(const T *__restrict__ X, int K, int pre,
                                                           const float *__restrict__ partial,
                                                           int8_t *__restrict__ Xq,
                                                           float *__restrict__ sx)
{
    const int seg = blockIdx.x, nseg = gridDim.x;
    const int64_t m = blockIdx.y;
    float a = 0.0f;
    for (int j = 0; j < nseg; j++)
        a = fmaxf(a, partial[m * nseg + j]);
    const float scale = a / 127.0f;
    const bool fast = rcp_quant_ok(scale);
    const float rs = fast ? 1.0f / scale : 0.0f;
    float y[8];
    int c;
    seg_load(X + m * K, K, seg, pre, y, c);
    if (c < K / 8)
        *reinterpret_cast<uint2 *>(Xq + m * K + (int64_t)c * 8) = quant8(y, scale, rs, fast);
    if (seg == 0 && threadIdx.x == 0)
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
                        const float *beta, float eps, int8_t *Xq, float *sx, float *partial,
                        hipStream_t stream)
{
    // Rows up to 64 lanes x 16 chunks x 8 = 8192 elements: one wave per token,
    // four tokens per block.
    if (K <= 8192)
        return launch_cfg<T, 1, 4>(X, M, K, pre, gamma, beta, eps, Xq, sx, stream);
    // Longer rows without LayerNorm, with room for the segment maxima: split.
    if (pre != 1 && partial) {
        const dim3 grid((unsigned)((K + kSegElems - 1) / kSegElems), (unsigned)M);
        hipLaunchKernelGGL(k_seg_absmax<T>, grid, dim3(kSegThreads), 0, stream, X, (int)K, pre,
                           partial);
        hipLaunchKernelGGL(k_seg_quant<T>, grid, dim3(kSegThreads), 0, stream, X, (int)K, pre,
                           partial, Xq, sx);
        return hipGetLastError();
    }
    // Otherwise 16 waves per token.
    return launch_cfg<T, 16, 1>(X, M, K, pre, gamma, beta, eps, Xq, sx, stream);
}

}  // namespace

int64_t ln_quant_partials(int64_t K)
{
    return (K + kSegElems - 1) / kSegElems;
}

hipError_t launch_ln_quant(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                           const float *gamma, const float *beta, float eps, int8_t *Xq,
                           float *x_scales, float *partial, hipStream_t stream)
{
    if (x_f16)
        return launch_typed(static_cast<const _Float16 *>(X), M, K, pre, gamma, beta, eps, Xq,
                            x_scales, partial, stream);
    return launch_typed(static_cast<const float *>(X), M, K, pre, gamma, beta, eps, Xq, x_scales,
                        partial, stream);
}

}  // namespace zq
