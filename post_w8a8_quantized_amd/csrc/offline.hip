// Offline preparation kernels (gfx950): group-wise weight quantization and the
// SmoothQuant factors with their LayerNorm fold.  Not on the per-token path.
//
// Pages: ZeroQuant reading notes, group-wise quantization of W (one scale per
// group); "探秘Transformer系列之（36）--- 大模型量化方案" 1.2.2 (group-wise weight
// quantization); "SmoothQuant技术解析：大模型INT8量化的突破与实践" 2.2 (per-channel
// factor s with Y = (X diag(s)^-1)(diag(s) W)) and 3.2 (offline: compute s,
// scale W, quantize; online: divide X by s, quantize).
//
// Reductions over a group or a channel use an unsigned atomic max on the
// bits of non-negative floats, which gives the exact maximum whatever the
// arrival order.  Buffers that receive atomics are cleared with a fill
// kernel on the same stream.
#include "zq_device.h"
#include "zq_kernels.h"

namespace zq {
namespace {

constexpr int kThreads = 256;

__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = v;
}

// Element j of row n of W, times smooth[j] when given (rounded to fp32 once).
template <typename T>
__device__ __forceinline__ float w_elem(const T *W, const float *smooth, int64_t n, int K, int j)
{
    float v = (float)W[n * K + j];
    if (smooth)
        v = v * smooth[j];
    return v;
}

// One block covers up to kThreads * 4 consecutive elements of one row.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_wgroup_absmax(const T *__restrict__ W,
                                                            const float *__restrict__ smooth,
                                                            int K, int G, int blocks_per_row,
                                                            uint32_t *__restrict__ amax)
{
    const int64_t n = blockIdx.x / blocks_per_row;
    const int j0 = (blockIdx.x % blocks_per_row) * kThreads * 4;
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int j = j0 + i * kThreads + threadIdx.x;
        if (j < K)
            a = fmaxf(a, fabsf(w_elem(W, smooth, n, K, j)));
    }
    a = wave_max(a);
    __shared__ float red[kThreads / kWave];
    if (threadIdx.x % kWave == 0)
        red[threadIdx.x / kWave] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = red[0];
        for (int w = 1; w < kThreads / kWave; w++)
            r = fmaxf(r, red[w]);
        atomic_max_nonneg(&amax[n / G], r);
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_wgroup_quant(const T *__restrict__ W,
                                                           const float *__restrict__ smooth,
                                                           int K, int G, int blocks_per_row,
                                                           const uint32_t *__restrict__ amax,
                                                           int8_t *__restrict__ Wq)
{
    const int64_t n = blockIdx.x / blocks_per_row;
    const int j0 = (blockIdx.x % blocks_per_row) * kThreads * 4;
    const float s = __uint_as_float(amax[n / G]) / 127.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int j = j0 + i * kThreads + threadIdx.x;
        if (j < K)
            Wq[n * K + j] = (int8_t)quant_code(w_elem(W, smooth, n, K, j), s);
    }
}

// FP8 codes of the group: power-of-two scale 2^e from the group's absmax.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_wgroup_quant_fp8(const T *__restrict__ W,
                                                               const float *__restrict__ smooth,
                                                               int K, int G, int blocks_per_row,
                                                               const uint32_t *__restrict__ amax,
                                                               uint8_t *__restrict__ Wq)
{
    const int64_t n = blockIdx.x / blocks_per_row;
    const int j0 = (blockIdx.x % blocks_per_row) * kThreads * 4;
    int e;
    const float s = fp8_scale(__uint_as_float(amax[n / G]), e);
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int j = j0 + i * kThreads + threadIdx.x;
        if (j < K) {
            const float v = w_elem(W, smooth, n, K, j);
            Wq[n * K + j] = s == 0.0f ? 0 : (uint8_t)(fp8x4(v, 0.0f, 0.0f, 0.0f, e) & 0xff);
        }
    }
}

__global__ void k_wgroup_scales_fp8(const uint32_t *__restrict__ amax, float *__restrict__ s_w,
                                    int64_t ng)
{
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < ng) {
        int e;
        s_w[g] = fp8_scale(__uint_as_float(amax[g]), e);
    }
}

__global__ void k_wgroup_scales(const uint32_t *__restrict__ amax, float *__restrict__ s_w, int64_t ng)
{
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < ng)
        s_w[g] = __uint_as_float(amax[g]) / 127.0f;
}

template <typename T>
hipError_t quantize_typed(const T *W, const float *smooth, int64_t N, int64_t K, int64_t G,
                          int8_t *Wq, float *w_scales, hipStream_t stream, bool fp8)
{
    const int64_t ng = N / G;
    // The scale array doubles as the group-max scratch: bits of |W'|max.
    uint32_t *amax = reinterpret_cast<uint32_t *>(w_scales);
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0, stream, amax,
                       ng, 0u);
    const int bpr = (int)((K + kThreads * 4 - 1) / (kThreads * 4));
    const dim3 grid((unsigned)(N * bpr));
    hipLaunchKernelGGL(k_wgroup_absmax<T>, grid, dim3(kThreads), 0, stream, W, smooth, (int)K,
                       (int)G, bpr, amax);
    if (fp8) {
        hipLaunchKernelGGL(k_wgroup_quant_fp8<T>, grid, dim3(kThreads), 0, stream, W, smooth,
                           (int)K, (int)G, bpr, amax, reinterpret_cast<uint8_t *>(Wq));
        hipLaunchKernelGGL(k_wgroup_scales_fp8, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0,
                           stream, amax, w_scales, ng);
    } else {
        hipLaunchKernelGGL(k_wgroup_quant<T>, grid, dim3(kThreads), 0, stream, W, smooth, (int)K,
                           (int)G, bpr, amax, Wq);
        hipLaunchKernelGGL(k_wgroup_scales, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0,
                           stream, amax, w_scales, ng);
    }
    return hipGetLastError();
}

// ---- SmoothQuant statistics ----

// Per-token LayerNorm statistics (gamma = 1, beta = 0): mean and 1/sqrt(var + eps),
// fp32, two passes, one wave per token.  The summation order need not match the
// prologue's: the factors feed an offline fold, not a code decision.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_ln_stats(const T *__restrict__ X, int M, int K,
                                                       float eps, float *__restrict__ stats)
{
    const int64_t m = (int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    if (m >= M)
        return;
    const T *row = X + m * K;
    float s = 0.0f;
    for (int j = lane; j < K; j += kWave)
        s += (float)row[j];
    const float mean = wave_sum(s) / (float)K;
    float ss = 0.0f;
    for (int j = lane; j < K; j += kWave) {
        const float d = (float)row[j] - mean;
        ss += d * d;
    }
    const float var = wave_sum(ss) / (float)K;
    if (lane == 0) {
        stats[2 * m] = mean;
        stats[2 * m + 1] = 1.0f / sqrtf(var + eps);
    }
}

// Column maxima of LN(X): thread owns channel j, walks a slab of tokens.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_col_absmax_ln(const T *__restrict__ X, int M, int K,
                                                            const float *__restrict__ stats,
                                                            int rows_per_blk,
                                                            uint32_t *__restrict__ amax)
{
    const int j = blockIdx.x * kThreads + threadIdx.x;
    const int r0 = blockIdx.y * rows_per_blk;
    const int r1 = min(M, r0 + rows_per_blk);
    if (j >= K)
        return;
    float a = 0.0f;
    for (int m = r0; m < r1; m++) {
        const float y = ((float)X[(int64_t)m * K + j] - stats[2 * m]) * stats[2 * m + 1];
        a = fmaxf(a, fabsf(y));
    }
    atomic_max_nonneg(&amax[j], a);
}

// Column maxima of W [N x K].
template <typename T>
__global__ __launch_bounds__(kThreads) void k_col_absmax_w(const T *__restrict__ W, int N, int K,
                                                           int rows_per_blk,
                                                           uint32_t *__restrict__ amax)
{
    const int j = blockIdx.x * kThreads + threadIdx.x;
    const int r0 = blockIdx.y * rows_per_blk;
    const int r1 = min(N, r0 + rows_per_blk);
    if (j >= K)
        return;
    float a = 0.0f;
    for (int n = r0; n < r1; n++)
        a = fmaxf(a, fabsf((float)W[(int64_t)n * K + j]));
    atomic_max_nonneg(&amax[j], a);
}

// s_j = fl32(sqrt(a_j / w_j)) (1 if either is 0); gamma' = gamma / s, beta' = beta / s.
// The square root is taken in fp64 and rounded once, as is the ratio.
__global__ void k_smooth_finalize(const uint32_t *__restrict__ amax_x,
                                  const uint32_t *__restrict__ amax_w, int K,
                                  const float *__restrict__ gamma, const float *__restrict__ beta,
                                  float *__restrict__ smooth, float *__restrict__ gamma_out,
                                  float *__restrict__ beta_out)
{
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= K)
        return;
    const double a = (double)__uint_as_float(amax_x[j]);
    const double w = (double)__uint_as_float(amax_w[j]);
    const float s = (a > 0.0 && w > 0.0) ? (float)sqrt(a / w) : 1.0f;
    smooth[j] = s;
    gamma_out[j] = (gamma ? gamma[j] : 1.0f) / s;
    beta_out[j] = (beta ? beta[j] : 0.0f) / s;
}

template <typename TX, typename TW>
hipError_t smooth_typed(const TX *X, int64_t M, int64_t K, float eps, const TW *W, int64_t N,
                        const float *gamma, const float *beta, float *smooth, float *gamma_out,
                        float *beta_out, void *ws, hipStream_t stream)
{
    float *stats = static_cast<float *>(ws);
    uint32_t *amax_x = reinterpret_cast<uint32_t *>(stats + 2 * M);
    uint32_t *amax_w = amax_x + K;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((2 * K + 255) / 256)), dim3(256), 0, stream,
                       amax_x, 2 * K, 0u);
    hipLaunchKernelGGL(k_ln_stats<TX>, dim3((unsigned)((M + 3) / 4)), dim3(kThreads), 0, stream, X,
                       (int)M, (int)K, eps, stats);
    const int rows = 64;
    hipLaunchKernelGGL(k_col_absmax_ln<TX>,
                       dim3((unsigned)((K + kThreads - 1) / kThreads), (unsigned)((M + rows - 1) / rows)),
                       dim3(kThreads), 0, stream, X, (int)M, (int)K, stats, rows, amax_x);
    hipLaunchKernelGGL(k_col_absmax_w<TW>,
                       dim3((unsigned)((K + kThreads - 1) / kThreads), (unsigned)((N + rows - 1) / rows)),
                       dim3(kThreads), 0, stream, W, (int)N, (int)K, rows, amax_w);
    hipLaunchKernelGGL(k_smooth_finalize, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, stream,
                       amax_x, amax_w, (int)K, gamma, beta, smooth, gamma_out, beta_out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_weights(const void *W, bool w_f16, const float *smooth, int64_t N,
                                   int64_t K, int64_t G, int8_t *Wq, float *w_scales,
                                   hipStream_t stream, bool fp8)
{
    if (w_f16)
        return quantize_typed(static_cast<const _Float16 *>(W), smooth, N, K, G, Wq, w_scales,
                              stream, fp8);
    return quantize_typed(static_cast<const float *>(W), smooth, N, K, G, Wq, w_scales, stream,
                          fp8);
}

hipError_t launch_smooth_factors(const void *X, bool x_f16, int64_t M, int64_t K, float eps,
                                 const void *W, bool w_f16, int64_t N, const float *gamma,
                                 const float *beta, float *smooth, float *gamma_out,
                                 float *beta_out, void *ws, hipStream_t stream)
{
    if (x_f16) {
        if (w_f16)
            return smooth_typed(static_cast<const _Float16 *>(X), M, K, eps,
                                static_cast<const _Float16 *>(W), N, gamma, beta, smooth,
                                gamma_out, beta_out, ws, stream);
        return smooth_typed(static_cast<const _Float16 *>(X), M, K, eps,
                            static_cast<const float *>(W), N, gamma, beta, smooth, gamma_out,
                            beta_out, ws, stream);
    }
    if (w_f16)
        return smooth_typed(static_cast<const float *>(X), M, K, eps,
                            static_cast<const _Float16 *>(W), N, gamma, beta, smooth, gamma_out,
                            beta_out, ws, stream);
    return smooth_typed(static_cast<const float *>(X), M, K, eps, static_cast<const float *>(W), N,
                        gamma, beta, smooth, gamma_out, beta_out, ws, stream);
}

}  // namespace zq
