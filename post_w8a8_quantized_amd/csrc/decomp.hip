// Outlier-column bookkeeping and the fp16 weight copy of the mixed-precision
// decomposition (LLM.int8() in "探秘Transformer系列之（36）--- 大模型量化方案"
// 1.1, "方案" and "混合精度分解": columns whose activations exceed the threshold
// stay in fp16 on both sides, the rest go through the int8 GEMM).
//
// The set O is a property of the whole batch, so it is found in its own pass
// (k_ln_quant with DEC = 1 marks slot[col] = 1 after a clear; for few tokens
// without a LayerNorm, k_mark_cols writes every mark, 1 or 0, itself) and a
// one-workgroup compaction turns the marks into
//   cols[0] = |O|, cols[1 + p] = the p-th outlier column (ascending),
//   slot[j] = p for an outlier column j, -1 otherwise.
// Both arrays are O(K) and stay in L2 for the passes that read them.
//
// The fp16 weights of the outlier columns are read by column: W16t is the
// fp16 copy of W laid out [K x N] (input channel major), so one outlier
// column is one contiguous run of N halves and the GEMM epilogue reads the
// 32 columns of a fragment as 64 contiguous bytes.
#include "zq_device.h"
#include "zq_kernels.h"

#include <algorithm>

namespace zq {
namespace {

__global__ __launch_bounds__(256) void k_fill_i32(int32_t *__restrict__ p, int64_t n, int32_t v)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

constexpr int kCompactThreads = 1024;
constexpr int kTileCols = 4 * kCompactThreads;  // one 16-byte piece of marks per thread
constexpr int kTilesLoaded = 8;                 // tiles whose marks are loaded together

// One workgroup.  The marks go in tiles of 4096 columns: thread t owns
// columns 4 t .. 4 t + 3 of a tile, so every load and store instruction is one
// contiguous 1 KB run per wave.  kTilesLoaded tiles are loaded together; then,
// tile by tile, an inclusive scan of the per-thread counts over the threads
// (by shuffles within each wave, then over the wave totals in LDS) gives each
// thread the position of its first outlier column, and it rewrites its own
// four columns.  No column is read by one thread and written by another.
__global__ __launch_bounds__(kCompactThreads) void k_outlier_compact(int32_t *__restrict__ slot,
                                                                     int K,
                                                                     int32_t *__restrict__ cols)
{
    constexpr int kWaves = kCompactThreads / kWave;
    __shared__ int wsum[kWaves];
    const int t = threadIdx.x;
    const int lane = t % kWave, wave = t / kWave;
    int base = 0;
    for (int t0 = 0; t0 < K; t0 += kTileCols * kTilesLoaded) {
        // K % 16 == 0, so each group of four columns is wholly inside or past K.
        int4 v[kTilesLoaded];
#pragma unroll
        for (int i = 0; i < kTilesLoaded; i++) {
            const int j = t0 + i * kTileCols + 4 * t;
            v[i] = j < K ? *reinterpret_cast<const int4 *>(slot + j) : make_int4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kTilesLoaded; i++) {
            if (t0 + i * kTileCols >= K)  // the same for every thread: no barrier is skipped alone
                break;
            const int cnt = (v[i].x != 0) + (v[i].y != 0) + (v[i].z != 0) + (v[i].w != 0);
            int incl = cnt;
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const int up = __shfl_up(incl, d);
                if (lane >= d)
                    incl += up;
            }
            if (lane == kWave - 1)
                wsum[wave] = incl;
            __syncthreads();
            int before = 0, tile_total = 0;
#pragma unroll
            for (int w = 0; w < kWaves; w++) {
                const int x = wsum[w];
                before += w < wave ? x : 0;
                tile_total += x;
            }
            const int j = t0 + i * kTileCols + 4 * t;
            if (j < K) {
                int p = base + before + incl - cnt;
                const int in[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                int out[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    if (in[e] != 0) {
                        out[e] = p;
                        cols[1 + p] = j + e;
                        p++;
                    } else {
                        out[e] = -1;
                    }
                }
                *reinterpret_cast<int4 *>(slot + j) = make_int4(out[0], out[1], out[2], out[3]);
            }
            base += tile_total;
            __syncthreads();  // wsum[] is reused by the next tile
        }
    }
    if (t == 0)
        cols[0] = base;
}

// W [N x K] (fp32 or fp16) -> W16t [K x N] fp16 (round to nearest even), through
// a 64 x 64 LDS tile so that both the reads (along K) and the writes (along N)
// are coalesced.  Block (x, y) covers rows n0 = 64 x .. n0 + 63 and columns
// k0 = 64 y .. k0 + 63.
template <typename T>
__global__ __launch_bounds__(256) void k_transpose_to_f16(const T *__restrict__ W, int N, int K,
                                                          _Float16 *__restrict__ Wt)
{
    __shared__ _Float16 tile[64][64 + 2];
    const int n0 = blockIdx.x * 64;
    const int k0 = blockIdx.y * 64;
    const int tx = threadIdx.x % 64;
    const int ty = threadIdx.x / 64;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int r = ty + 4 * i;
        const int n = n0 + r, k = k0 + tx;
        tile[r][tx] = (n < N && k < K) ? (_Float16)W[(int64_t)n * K + k] : (_Float16)0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int r = ty + 4 * i;
        const int k = k0 + r, n = n0 + tx;
        if (k < K && n < N)
            Wt[(int64_t)k * N + n] = tile[tx][r];
    }
}

}  // namespace

hipError_t launch_outlier_columns(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                                  const float *gamma, const float *beta, float eps, float alpha,
                                  int32_t *slot, int32_t *cols, hipStream_t stream)
{
    hipError_t e;
    if (!outlier_detect_writes_all(M, K, pre)) {
        const int64_t blocks = std::min<int64_t>((K + 255) / 256, 1024);
        hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)blocks), dim3(256), 0, stream, slot, K, 0);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (M > 0) {
        e = launch_outlier_detect(X, x_f16, M, K, pre, gamma, beta, eps, alpha, slot, stream);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(k_outlier_compact, dim3(1), dim3(kCompactThreads), 0, stream, slot, (int)K,
                       cols);
    return hipGetLastError();
}

hipError_t launch_pack_outlier_weights(const void *W, bool w_f16, int64_t N, int64_t K,
                                       _Float16 *Wt, hipStream_t stream)
{
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((K + 63) / 64));
    if (w_f16)
        hipLaunchKernelGGL(k_transpose_to_f16<_Float16>, grid, dim3(256), 0, stream,
                           static_cast<const _Float16 *>(W), (int)N, (int)K, Wt);
    else
        hipLaunchKernelGGL(k_transpose_to_f16<float>, grid, dim3(256), 0, stream,
                           static_cast<const float *>(W), (int)N, (int)K, Wt);
    return hipGetLastError();
}

}  // namespace zq
