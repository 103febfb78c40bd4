// Weight-streaming int8 GEMM for few tokens (M <= 32), the decode shape (gfx950).
//
// Same result as the tiled kernel: Y[m, n] = fp16(s_x[m] s_w[n/G] acc[m, n] + bias[n]),
// optional GeLU ("探秘Transformer系列之（36）--- 大模型量化方案" 1.2.2 and 1.1.2;
// ZeroQuant reading notes, "GeMM + DeQuantize").  With a handful of tokens
// the int8 weight stream dominates: the layer is bound by HBM bandwidth
// ("Integer Quantization: Deep Dive": decoding is memory-bandwidth bound).
//
// Design for CDNA4:
//  - A workgroup owns 16*RG output rows over all of K (one workgroup per CU
//    at the decode shape).  Slabs of BKB bytes of those rows (and of the
//    <= 32 token rows of X) move HBM -> LDS with global_load_lds_dwordx4;
//    every wave-wide DMA reads 1 KB of ONE row, i.e. fully contiguous,
//    streaming memory, which is what HBM rewards.  Two slabs are in flight.
//  - In LDS, 16-byte chunk c of row r sits at slot c ^ (r % 16) (the DMA
//    lane fetching a slot picks the matching chunk), so the MFMA operand
//    reads -- 16 rows, one chunk each -- hit 16 different bank groups.
//  - v_mfma_i32_16x16x64_i8 with W as the A operand (16 rows) and X as the
//    B operand (16 tokens) absorbs the whole product; the four waves take
//    alternate 64-byte k blocks of each slab and their int32 partial sums
//    are added through LDS in a fixed order (deterministic, no atomics).
#include "zq_device.h"
#include "zq_kernels.h"

namespace zq {
namespace {

// 16 zero bytes: the DMA source for lanes whose chunk lies past the end of K.
__device__ __attribute__((aligned(16))) int8_t zero16[16];

constexpr int kThreads = 256;  // 4 waves

__device__ __forceinline__ void dma16(const int8_t *src, int8_t *lds_base)
{
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int MT, int RG, int BKB, bool OUT_I32>
__global__ __launch_bounds__(kThreads) void k_gemm_skinny(
    const int8_t *__restrict__ Xq, const float *__restrict__ sx, const int8_t *__restrict__ Wq,
    const float *__restrict__ sw, int G, const float *__restrict__ bias, int act, int M, int N,
    int K, void *__restrict__ Y)
{
    constexpr int WR = 16 * RG;            // weight rows per workgroup
    constexpr int XR = 16 * MT;            // token rows (padded to 16s)
    constexpr int ROWS = WR + XR;
    constexpr int PIECES = BKB / 1024;     // 1 KB DMA pieces per row per slab
    constexpr int DMAS = ROWS * PIECES;    // wave-wide DMAs per slab
    static_assert(DMAS % 4 == 0, "DMAs split evenly over the four waves");
    constexpr int PER_WAVE = DMAS / 4;
    constexpr int STAGE = ROWS * BKB;
    constexpr int KB = BKB / 64;           // 64-byte MFMA k blocks per slab

    __shared__ __attribute__((aligned(1024))) int8_t buf0[STAGE];
    __shared__ __attribute__((aligned(1024))) int8_t buf1[STAGE];
    __shared__ v4i part[4][RG][MT][kWave];

    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int n0 = blockIdx.x * WR;

    // DMA j of this wave: row (wave + 4 j) / PIECES, piece (wave + 4 j) % PIECES.
    // Row index < WR is a weight row, otherwise a token row.
    const int8_t *src[PER_WAVE];
    int kc[PER_WAVE];          // byte offset of this lane's chunk within the slab
    int slot_bytes[PER_WAVE];  // LDS destination of the DMA
#pragma unroll
    for (int j = 0; j < PER_WAVE; j++) {
        const int d = wave + 4 * j;
        const int r = d / PIECES, q = d % PIECES;
        const int chunk = (64 * q + lane) ^ (r & 15);   // global chunk for this lane's slot
        const int8_t *row = r < WR ? Wq + (int64_t)min(n0 + r, N - 1) * K
                                   : Xq + (int64_t)min(r - WR, M - 1) * K;
        src[j] = row + 16 * chunk;
        kc[j] = 16 * chunk;
        slot_bytes[j] = r * BKB + q * 1024;
    }
    auto issue = [&](int slab, int8_t *buf) {
        const int k0 = slab * BKB;
#pragma unroll
        for (int j = 0; j < PER_WAVE; j++)
            dma16(k0 + kc[j] < K ? src[j] + k0 : zero16, buf + slot_bytes[j]);
    };

    // MFMA operand rows: lane (r16, kq) reads row r16 of a 16-row group at
    // chunk 4 kb + kq, stored at slot (4 kb + kq) ^ r16.
    const int r16 = lane & 15;
    const int kq = lane >> 4;

    v4i acc[RG][MT];
#pragma unroll
    for (int g = 0; g < RG; g++)
#pragma unroll
        for (int t = 0; t < MT; t++)
            acc[g][t] = v4i{0, 0, 0, 0};

    auto compute = [&](const int8_t *buf) {
#pragma unroll
        for (int kb = wave; kb < KB; kb += 4) {
            const int off = 16 * ((4 * kb + kq) ^ r16);
            v4i a[RG], b[MT];
#pragma unroll
            for (int g = 0; g < RG; g++)
                a[g] = *reinterpret_cast<const v4i *>(buf + (16 * g + r16) * BKB + off);
#pragma unroll
            for (int t = 0; t < MT; t++)
                b[t] = *reinterpret_cast<const v4i *>(buf + (WR + 16 * t + r16) * BKB + off);
#pragma unroll
            for (int g = 0; g < RG; g++)
#pragma unroll
                for (int t = 0; t < MT; t++)
                    acc[g][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[g], b[t], acc[g][t], 0, 0, 0);
        }
    };
    auto barrier = [] {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
    };

    // Slabs alternate between buf0 and buf1; the slab count is padded to even
    // (a padding slab lies past K and reads zeros).
    const int ns = (K + BKB - 1) / BKB;
    const int nsp = (ns + 1) & ~1;
    issue(0, buf0);
    issue(1, buf1);
    for (int s = 0; s < nsp; s += 2) {
        wait_vmcnt<PER_WAVE>();   // slab s landed (slab s+1 may be in flight)
        barrier();
        compute(buf0);
        barrier();                // every wave is done with buf0
        issue(s + 2, buf0);
        wait_vmcnt<PER_WAVE>();   // slab s+1 landed (slab s+2 may be in flight)
        barrier();
        compute(buf1);
        barrier();
        issue(s + 3, buf1);
    }
    wait_vmcnt<0>();  // drain the zero-filled refills before LDS is released

#pragma unroll
    for (int g = 0; g < RG; g++)
#pragma unroll
        for (int t = 0; t < MT; t++)
            part[wave][g][t][lane] = acc[g][t];
    __syncthreads();

    // Wave w finishes row groups w, w+4, ...: fixed-order sum of the four
    // partials, then the epilogue.  Accumulator register i of (g, t) holds
    // token m = 16 t + lane % 16 and output row n = n0 + 16 g + 4 (lane / 16) + i.
#pragma unroll
    for (int g = 0; g < RG; g++) {
        if (g % 4 != wave)
            continue;
#pragma unroll
        for (int t = 0; t < MT; t++) {
            const v4i sum = part[0][g][t][lane] + part[1][g][t][lane] + part[2][g][t][lane] +
                            part[3][g][t][lane];
            const int m = 16 * t + r16;
            const int nn = n0 + 16 * g + 4 * kq;
            if (m >= M || nn >= N)
                continue;
            if constexpr (OUT_I32) {
                *reinterpret_cast<v4i *>(static_cast<int32_t *>(Y) + (int64_t)m * N + nn) = sum;
            } else {
                const float sxm = sx[m];
                h4 o;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    float v = (float)sum[i] * (sxm * sw[(nn + i) / G]);
                    if (bias)
                        v += bias[nn + i];
                    if (act == 1)
                        v = gelu_fast(v);
                    o[i] = (_Float16)v;
                }
                *reinterpret_cast<h4 *>(static_cast<_Float16 *>(Y) + (int64_t)m * N + nn) = o;
            }
        }
    }
}

template <int MT, int RG, int BKB>
hipError_t launch_cfg(const int8_t *Xq, const float *sx, const int8_t *Wq, const float *sw,
                      int64_t G, const float *bias, int act, int64_t M, int64_t N, int64_t K,
                      void *Y, bool out_i32, hipStream_t stream)
{
    const dim3 grid((unsigned)((N + 16 * RG - 1) / (16 * RG)));
    const dim3 block(kThreads);
    if (out_i32)
        hipLaunchKernelGGL((k_gemm_skinny<MT, RG, BKB, true>), grid, block, 0, stream, Xq, sx, Wq,
                           sw, (int)G, bias, act, (int)M, (int)N, (int)K, Y);
    else
        hipLaunchKernelGGL((k_gemm_skinny<MT, RG, BKB, false>), grid, block, 0, stream, Xq, sx, Wq,
                           sw, (int)G, bias, act, (int)M, (int)N, (int)K, Y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_skinny(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                              const float *w_scales, int64_t G, const float *bias, int act,
                              int64_t M, int64_t N, int64_t K, void *Y, bool out_i32,
                              hipStream_t stream)
{
    // 32 weight rows per workgroup (two row groups) fills 256 CUs at N = 8192.
    if (M <= 16)
        return launch_cfg<1, 2, 1024>(Xq, x_scales, Wq, w_scales, G, bias, act, M, N, K, Y,
                                      out_i32, stream);
    return launch_cfg<2, 2, 1024>(Xq, x_scales, Wq, w_scales, G, bias, act, M, N, K, Y, out_i32,
                                  stream);
}

}  // namespace zq
