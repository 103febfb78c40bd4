// Tiled int8 MFMA GEMM with the dequantization fused into its epilogue (gfx950).
//
// Pages: "探秘Transformer系列之（36）--- 大模型量化方案" 1.2.2 (INT8 GEMM accumulating
// in INT32; the accumulation is scaled by the activation and weight scales
// before the FP16 result is written) and 1.1.2 vector-wise (the scaling is
// the outer product of per-row and per-column scales); ZeroQuant reading
// notes, kernel-fusion flowchart ("GeMM + DeQuantize" is one kernel);
// "Integer Quantization: Deep Dive", MAC unit (the bias joins the sum).
//
// Y[m, n] = fp16( s_x[m] * s_w[n / G] * sum_k Xq[m, k] Wq[n, k] + bias[n] ), optional GeLU.
//
// Design for CDNA4:
//  - v_mfma_i32_32x32x32_i8: one instruction multiplies a 32x32 block of
//    W rows by a 32x32 block of X rows over 32 k.  W is the A operand and X
//    the B operand, so each lane's 16 accumulators hold 4 runs of 4
//    consecutive output columns n of one token m: the epilogue writes 8-byte
//    fp16 groups straight from registers.
//  - Both operands are K-contiguous in HBM, so every lane's MFMA operand is
//    one 16-byte run of k; tiles are staged through LDS with 16-byte global
//    loads and ds_read_b128, double-buffered so that the next k-slab's global
//    loads are in flight while the current slab feeds the MFMAs.
//  - LDS rows are 64 bytes (one k-slab); the 16-byte chunk index is XORed
//    with (row / 4) % 4, which makes both the row-wise writes and the
//    column-wise MFMA operand reads free of bank conflicts.
//  - Output tiles are ordered so that consecutive workgroups, which the
//    dispatcher spreads round-robin over the 8 XCDs, land on the same XCD in
//    groups that share W (and X) panels in that XCD's L2.
#include "zq_device.h"
#include "zq_kernels.h"

namespace zq {
namespace {

constexpr int BK = 64;  // k bytes per LDS slab

__device__ __forceinline__ int swz(int row, int chunk)
{
    return chunk ^ ((row >> 2) & 3);
}

template <int BM, int BN, int WM, int WN>
struct TileCfg {
    static constexpr int NT = WM * WN * kWave;        // threads per block
    static constexpr int TWM = BM / WM;               // tokens per wave
    static constexpr int TWN = BN / WN;               // output columns per wave
    static constexpr int FM = TWM / 32;               // X fragments per wave
    static constexpr int FN = TWN / 32;               // W fragments per wave
    static constexpr int LX = BM * 4 / NT;            // 16-byte X loads per thread per slab
    static constexpr int LW = BN * 4 / NT;            // 16-byte W loads per thread per slab
    static_assert(BM % (32 * WM) == 0 && BN % (32 * WN) == 0, "wave tile must be 32-aligned");
    static_assert((BM * 4) % NT == 0 && (BN * 4) % NT == 0, "loads must divide evenly");
};

// Map the linear workgroup id to an output tile.  Workgroup b runs on XCD
// b % 8; regrouping makes workgroups that share an XCD take neighbouring
// tiles along M within one N column band, so they reuse the same W panel.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int total = tiles_m * tiles_n;
    int t = bid;
    if ((total & 7) == 0) {
        const int per_xcd = total >> 3;
        t = (bid & 7) * per_xcd + (bid >> 3);
    }
    tn = t / tiles_m;
    tm = t % tiles_m;
}

template <int BM, int BN, int WM, int WN, bool OUT_I32>
__global__ __launch_bounds__(WM *WN *kWave) void k_gemm_tiled(
    const int8_t *__restrict__ Xq, const float *__restrict__ sx, const int8_t *__restrict__ Wq,
    const float *__restrict__ sw, int G, const float *__restrict__ bias, int act, int M, int N,
    int K, void *__restrict__ Y, int tiles_m, int tiles_n)
{
    using C = TileCfg<BM, BN, WM, WN>;
    __shared__ __attribute__((aligned(16))) int8_t lds_x[2][BM * BK];
    __shared__ __attribute__((aligned(16))) int8_t lds_w[2][BN * BK];

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int wm = wave % WM;
    const int wn = wave / WM;

    // Global load assignment: chunk u = tid + NT*j covers row u/4, 16-byte chunk u%4.
    const int8_t *gx[C::LX];
    const int8_t *gw[C::LW];
    int lds_off_x[C::LX], lds_off_w[C::LW];
    int kchunk_x[C::LX], kchunk_w[C::LW];
#pragma unroll
    for (int j = 0; j < C::LX; j++) {
        const int u = tid + C::NT * j;
        const int r = u >> 2, c = u & 3;
        const int m = min(m0 + r, M - 1);  // ragged M: re-read the last row, never stored
        gx[j] = Xq + (int64_t)m * K + c * 16;
        kchunk_x[j] = c * 16;
        lds_off_x[j] = r * BK + swz(r, c) * 16;
    }
#pragma unroll
    for (int j = 0; j < C::LW; j++) {
        const int u = tid + C::NT * j;
        const int r = u >> 2, c = u & 3;
        const int n = min(n0 + r, N - 1);
        gw[j] = Wq + (int64_t)n * K + c * 16;
        kchunk_w[j] = c * 16;
        lds_off_w[j] = r * BK + swz(r, c) * 16;
    }

    v4i rx[C::LX], rw[C::LW];
    auto gload = [&](int k0) {
#pragma unroll
        for (int j = 0; j < C::LX; j++)
            rx[j] = (k0 + kchunk_x[j] < K) ? *reinterpret_cast<const v4i *>(gx[j] + k0) : v4i{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < C::LW; j++)
            rw[j] = (k0 + kchunk_w[j] < K) ? *reinterpret_cast<const v4i *>(gw[j] + k0) : v4i{0, 0, 0, 0};
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < C::LX; j++)
            *reinterpret_cast<v4i *>(&lds_x[buf][lds_off_x[j]]) = rx[j];
#pragma unroll
        for (int j = 0; j < C::LW; j++)
            *reinterpret_cast<v4i *>(&lds_w[buf][lds_off_w[j]]) = rw[j];
    };

    v16i acc[C::FN][C::FM];
#pragma unroll
    for (int a = 0; a < C::FN; a++)
#pragma unroll
        for (int b = 0; b < C::FM; b++)
            acc[a][b] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

    // MFMA operand rows of this lane.
    const int frow = lane & 31;
    const int fhalf = lane >> 5;
    int xrow[C::FM], wrow[C::FN];
#pragma unroll
    for (int b = 0; b < C::FM; b++)
        xrow[b] = wm * C::TWM + b * 32 + frow;
#pragma unroll
    for (int a = 0; a < C::FN; a++)
        wrow[a] = wn * C::TWN + a * 32 + frow;

    const int nk = (K + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        if (kt + 1 < nk)
            gload((kt + 1) * BK);
#pragma unroll
        for (int ks = 0; ks < BK / 32; ks++) {
            const int chunk = ks * 2 + fhalf;
            v4i fx[C::FM], fw[C::FN];
#pragma unroll
            for (int b = 0; b < C::FM; b++)
                fx[b] = *reinterpret_cast<const v4i *>(&lds_x[cur][xrow[b] * BK + swz(xrow[b], chunk) * 16]);
#pragma unroll
            for (int a = 0; a < C::FN; a++)
                fw[a] = *reinterpret_cast<const v4i *>(&lds_w[cur][wrow[a] * BK + swz(wrow[a], chunk) * 16]);
#pragma unroll
            for (int a = 0; a < C::FN; a++)
#pragma unroll
                for (int b = 0; b < C::FM; b++)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[a], fx[b], acc[a][b], 0, 0, 0);
        }
        if (kt + 1 < nk)
            lstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Accumulator register r of fragment (a, b) holds
    // token  m = m0 + wm*TWM + b*32 + lane%32 and
    // column n = n0 + wn*TWN + a*32 + 8*(r/4) + 4*(lane/32) + r%4.
#pragma unroll
    for (int b = 0; b < C::FM; b++) {
        const int m = m0 + wm * C::TWM + b * 32 + frow;
        if (m >= M)
            continue;
        const float sxm = OUT_I32 ? 0.0f : sx[m];
#pragma unroll
        for (int a = 0; a < C::FN; a++) {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int n = n0 + wn * C::TWN + a * 32 + 8 * q + 4 * fhalf;
                if (n >= N)
                    continue;
                if constexpr (OUT_I32) {
                    v4i o = {acc[a][b][4 * q + 0], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2],
                             acc[a][b][4 * q + 3]};
                    *reinterpret_cast<v4i *>(static_cast<int32_t *>(Y) + (int64_t)m * N + n) = o;
                } else {
                    h4 o;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const float scale = sxm * sw[(n + i) / G];
                        float v = (float)acc[a][b][4 * q + i] * scale;
                        if (bias)
                            v += bias[n + i];
                        if (act == 1)
                            v = gelu_erf(v);
                        o[i] = (_Float16)v;
                    }
                    *reinterpret_cast<h4 *>(static_cast<_Float16 *>(Y) + (int64_t)m * N + n) = o;
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const int8_t *Xq, const float *sx, const int8_t *Wq, const float *sw,
                      int64_t G, const float *bias, int act, int64_t M, int64_t N, int64_t K,
                      void *Y, bool out_i32, hipStream_t stream)
{
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    const dim3 block(WM * WN * kWave);
    if (out_i32)
        hipLaunchKernelGGL((k_gemm_tiled<BM, BN, WM, WN, true>), grid, block, 0, stream, Xq, sx,
                           Wq, sw, (int)G, bias, act, (int)M, (int)N, (int)K, Y, tiles_m, tiles_n);
    else
        hipLaunchKernelGGL((k_gemm_tiled<BM, BN, WM, WN, false>), grid, block, 0, stream, Xq, sx,
                           Wq, sw, (int)G, bias, act, (int)M, (int)N, (int)K, Y, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_tiled(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                             const float *w_scales, int64_t G, const float *bias, int act,
                             int64_t M, int64_t N, int64_t K, void *Y, bool out_i32,
                             hipStream_t stream)
{
    return launch_cfg<128, 128, 2, 2>(Xq, x_scales, Wq, w_scales, G, bias, act, M, N, K, Y,
                                      out_i32, stream);
}

}  // namespace zq
