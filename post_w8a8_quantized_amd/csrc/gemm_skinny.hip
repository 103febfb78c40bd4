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
//    streaming memory, which is what HBM rewards.  NS slabs are in flight
//    (four 512-byte slabs at the shapes used); the weights are read with
//    the non-temporal policy, since each byte is used once.
//  - In LDS, 16-byte chunk c of row r sits at slot c ^ (r % 16) (the DMA
//    lane fetching a slot picks the matching chunk), so the MFMA operand
//    reads -- 16 rows, one chunk each -- hit 16 different bank groups.
//  - v_mfma_i32_16x16x64_i8 with W as the A operand (16 rows) and X as the
//    B operand (16 tokens) absorbs the whole product; the four waves take
//    alternate 64-byte k blocks of each slab and their int32 partial sums
//    are added through LDS in a fixed order (deterministic, no atomics).
#include "zq_device.h"
#include "zq_kernels.h"

#include <algorithm>

#include <type_traits>

namespace zq {
namespace {

// 16 zero bytes: the DMA source for lanes whose chunk lies past the end of K.
__device__ __attribute__((aligned(16))) int8_t zero16[16];

constexpr int kThreads = 256;  // 4 waves
constexpr int kPackRows = 32;   // weight rows per packed block
constexpr int kPackBytes = 512; // bytes of each row per packed block

// F8: the operands are OCP E4M3 codes and the product is
// v_mfma_scale_f32_16x16x128_f8f6f4 (unit block scales), accumulating in fp32;
// OUT_I32 then writes the raw fp32 accumulators.
//
// ODEC (fp16 output): the mixed-precision decomposition's fp16 part joins the
// epilogue, sum_p XO[m, p] W16t[O_p, n] by fp32 FMAs per output (a handful of
// outlier columns against a K-long weight stream).  The outlier count and the
// first kOutCols columns are fetched into LDS at the start, so the epilogue's
// loads depend on nothing in flight.
template <int MT, int RG, int BKB, int NS, bool PACKED, bool OUT_I32, bool F8 = false,
          bool ODEC = false>
__global__ __launch_bounds__(kThreads) void k_gemm_skinny(
    const int8_t *__restrict__ Xq, const float *__restrict__ sx, const int8_t *__restrict__ Wq,
    const float *__restrict__ sw, int G, const float *__restrict__ bias, int act, int M, int N,
    int K, void *__restrict__ Y, float *__restrict__ row_part, OutlierOperands dec)
{
    constexpr int WR = 16 * RG;            // weight rows per workgroup
    constexpr int XR = 16 * MT;            // token rows (padded to 16s)
    constexpr int ROWS = WR + XR;
    constexpr int CPR = BKB / 16;          // 16-byte chunks per row and slab
    constexpr int LW = WR * CPR / 256;     // wave-wide DMAs per wave and slab, weights
    constexpr int LX = XR * CPR / 256;     // the same, tokens
    static_assert(CPR >= 16 && (XR * CPR) % 256 == 0, "DMAs split evenly over the four waves");
    constexpr int PER_WAVE = LW + LX;
    constexpr int STAGE = ROWS * BKB;
    constexpr int KB = BKB / (F8 ? 128 : 64);  // MFMA k blocks per slab (64 or 128 bytes)
    static_assert(KB % 4 == 0, "the four waves share each slab's k blocks evenly");
    using Acc = std::conditional_t<F8, v4f, v4i>;
    using Frag = std::conditional_t<F8, v8i, v4i>;
    static_assert(NS >= 2 && NS <= 8, "pipeline depth");
    static_assert(4 * RG * MT * 64 * 16 <= STAGE, "partial sums fit in one slab buffer");
    static_assert(!PACKED || (WR == kPackRows && BKB == kPackBytes), "packed blocks are slabs");

    // One LDS object per slab buffer, referenced statically from the unrolled
    // loop, so the compiler can tell the buffers apart from in-flight DMAs.
    __shared__ __attribute__((aligned(1024))) int8_t buf0[STAGE];
    __shared__ __attribute__((aligned(1024))) int8_t buf1[STAGE];
    __shared__ __attribute__((aligned(1024))) int8_t buf2[NS > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) int8_t buf3[NS > 3 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) int8_t buf4[NS > 4 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) int8_t buf5[NS > 5 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) int8_t buf6[NS > 6 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) int8_t buf7[NS > 7 ? STAGE : 16];
    int8_t *const bufs[8] = {buf0, buf1, buf2, buf3, buf4, buf5, buf6, buf7};
    constexpr int kOutCols = 64;
    __shared__ int out_cols[ODEC ? kOutCols + 1 : 1];
    // ODEC with at most kPanelP outlier columns and N % 8 == 0: the epilogue's
    // operands, the fp16 weights of the outlier columns for this workgroup's
    // WR output rows (pw[p][n - n0]) and the tokens' outlier values
    // (px[m][p]), are loaded as one 16-byte piece per thread right after the
    // first slab DMAs, held in registers through the main loop and stored to
    // LDS at its final drain, so the epilogue waits for no memory.
    constexpr int kPanelP = 32;
    constexpr int kPW = kPanelP * (WR / 8);  // weight-panel pieces
    constexpr int kPX = XR * (kPanelP / 8);  // activation-panel pieces
    static_assert(!ODEC || kPW + kPX <= kThreads, "one piece per thread");
    __shared__ __attribute__((aligned(16))) _Float16 pw[ODEC ? kPanelP * WR : 8];
    __shared__ __attribute__((aligned(16))) _Float16 px[ODEC ? XR * kPanelP : 8];
    int n_out = 0, pcol = 0;
    if constexpr (ODEC) {
        if (threadIdx.x <= kOutCols && threadIdx.x <= K)  // cols holds K + 1 entries
            out_cols[threadIdx.x] = dec.cols[threadIdx.x];
        n_out = dec.cols[0];
        const int p = threadIdx.x / (WR / 8);
        if (threadIdx.x < kPW && p < K)
            pcol = dec.cols[1 + p];
    }
    const bool use_panel = ODEC && n_out <= kPanelP && (N & 7) == 0;

    // Wave index as a scalar: the DMA split, k blocks and row groups below
    // are uniform per wave.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int n0 = blockIdx.x * WR;

    // Wave-wide DMA d of a row block fills LDS bytes [1024 d, 1024 d + 1024)
    // of that block: lane l lands at flat chunk position f = 64 d + l, i.e.
    // slot f % CPR of row f / CPR, and fetches the chunk stored there.
    // Wave w issues DMAs w, w + 4, ... of the weight block and of the token block.
    // Packed weights: the workgroup's slab s is one contiguous block of WR
    // rows x BKB bytes at ((blockIdx.x * ns) + s) * WR * BKB, zero padded.
    const int ns = (K + BKB - 1) / BKB;
    const int8_t *src_w[LW], *src_x[LX];
    int kc_w[LW], kc_x[LX];    // byte offset of this lane's chunk within the slab
#pragma unroll
    for (int j = 0; j < LW; j++) {
        const int f = 64 * (wave + 4 * j) + lane;
        const int r = f / CPR;
        const int chunk = (f % CPR) ^ (r & 15);
        if constexpr (PACKED)
            src_w[j] = Wq + (int64_t)blockIdx.x * ns * (WR * BKB) + r * BKB + 16 * chunk;
        else
            src_w[j] = Wq + (int64_t)min(n0 + r, N - 1) * K + 16 * chunk;
        kc_w[j] = 16 * chunk;
    }
#pragma unroll
    for (int j = 0; j < LX; j++) {
        const int f = 64 * (wave + 4 * j) + lane;
        const int r = f / CPR;
        const int chunk = (f % CPR) ^ (r & 15);
        src_x[j] = Xq + (int64_t)min(r, M - 1) * K + 16 * chunk;
        kc_x[j] = 16 * chunk;
    }
    // Lanes whose chunk lies past K (and every lane of a padding slab) fetch
    // the zero block instead.
    auto issue = [&](int slab, int8_t *buf) {
        const int k0 = slab * BKB;
#pragma unroll
        for (int j = 0; j < LW; j++) {
            const int8_t *p;
            if constexpr (PACKED)
                p = slab < ns ? src_w[j] + (int64_t)slab * (WR * BKB) : zero16;
            else
                p = k0 + kc_w[j] < K ? src_w[j] + k0 : zero16;
            dma16<2>(p, buf + 1024 * (wave + 4 * j));  // streamed once: non-temporal
        }
#pragma unroll
        for (int j = 0; j < LX; j++)
            dma16<0>(k0 + kc_x[j] < K ? src_x[j] + k0 : zero16,
                     buf + WR * BKB + 1024 * (wave + 4 * j));
    };

    // MFMA operand rows: lane (r16, kq) reads row r16 of a 16-row group at
    // chunk 4 kb + kq, stored at slot (4 kb + kq) ^ r16.
    const int r16 = lane & 15;
    const int kq = lane >> 4;

    Acc acc[RG][MT];
#pragma unroll
    for (int g = 0; g < RG; g++)
#pragma unroll
        for (int t = 0; t < MT; t++)
            acc[g][t] = Acc{};

    // Wave w takes k blocks w, w + 4, ... of each slab.
    auto compute = [&](const int8_t *buf) {
#pragma unroll
        for (int i = 0; i < KB / 4; i++) {
            const int kb = wave + 4 * i;
            Frag a[RG], b[MT];
            if constexpr (F8) {
                // lane (r16, kq) holds bytes 32 kq .. +32 of the 128-byte block: chunks
                // 8 kb + 2 kq and the next, each at its own swizzled slot
                const int c0 = 8 * kb + 2 * kq;
                const int off0 = 16 * (c0 ^ r16), off1 = 16 * ((c0 + 1) ^ r16);
                auto two = [&](const int8_t *row) {
                    const v4i lo = *reinterpret_cast<const v4i *>(row + off0);
                    const v4i hi = *reinterpret_cast<const v4i *>(row + off1);
                    return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                };
#pragma unroll
                for (int g = 0; g < RG; g++)
                    a[g] = two(buf + (16 * g + r16) * BKB);
#pragma unroll
                for (int t = 0; t < MT; t++)
                    b[t] = two(buf + (WR + 16 * t + r16) * BKB);
            } else {
                const int off = 16 * ((4 * kb + kq) ^ r16);
#pragma unroll
                for (int g = 0; g < RG; g++)
                    a[g] = *reinterpret_cast<const v4i *>(buf + (16 * g + r16) * BKB + off);
#pragma unroll
                for (int t = 0; t < MT; t++)
                    b[t] = *reinterpret_cast<const v4i *>(buf + (WR + 16 * t + r16) * BKB + off);
            }
#pragma unroll
            for (int g = 0; g < RG; g++)
#pragma unroll
                for (int t = 0; t < MT; t++) {
                    if constexpr (F8)
                        acc[g][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            a[g], b[t], acc[g][t], 0, 0, 0, 127, 0, 127);
                    else
                        acc[g][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[g], b[t], acc[g][t], 0,
                                                                          0, 0);
                }
        }
    };
    auto barrier = [] {
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
    };

    // Slab s lives in buffer s % NS; NS - 1 slabs are in flight while one is
    // multiplied.  Step s: wait for slab s, barrier (every wave is done with
    // slab s - 1), refill slab s - 1's buffer with slab s + NS - 1, multiply.
    // The slab count is padded to a multiple of NS (padding slabs read zeros
    // and add 0), so the loop has no branches and every wait the same count.
    const int nsp = (ns + NS - 1) / NS * NS;
#pragma unroll
    for (int j = 0; j < NS - 1; j++)
        issue(j, bufs[j]);
    h8 piece = {};
    if constexpr (ODEC) {
        const int t = threadIdx.x;
        if (use_panel && t < kPW) {
            const int p = t / (WR / 8), c = t % (WR / 8);
            if (p < n_out && n0 + 8 * c + 8 <= N)
                piece = *reinterpret_cast<const h8 *>(dec.wt + (int64_t)pcol * N + n0 + 8 * c);
        } else if (use_panel && t < kPW + kPX) {
            // 8 c < n_out <= K, both multiples of 8 up to K: the piece stays inside row tok.
            const int i = t - kPW;
            const int tok = i / (kPanelP / 8), c = i % (kPanelP / 8);
            if (tok < M && 8 * c < n_out)
                piece = *reinterpret_cast<const h8 *>(dec.xo + (int64_t)tok * K + 8 * c);
        }
    }
    auto step = [&](int s, auto J) {
        constexpr int j = decltype(J)::value;
        wait_vmcnt<(NS - 2) * PER_WAVE>();
        barrier();
        issue(s + NS - 1, bufs[(j + NS - 1) % NS]);
        compute(bufs[j]);
    };
    for (int s = 0; s < nsp; s += NS) {
        step(s, std::integral_constant<int, 0>{});
        step(s + 1, std::integral_constant<int, 1>{});
        if constexpr (NS > 2)
            step(s + 2, std::integral_constant<int, 2>{});
        if constexpr (NS > 3)
            step(s + 3, std::integral_constant<int, 3>{});
        if constexpr (NS > 4)
            step(s + 4, std::integral_constant<int, 4>{});
        if constexpr (NS > 5)
            step(s + 5, std::integral_constant<int, 5>{});
        if constexpr (NS > 6)
            step(s + 6, std::integral_constant<int, 6>{});
        if constexpr (NS > 7)
            step(s + 7, std::integral_constant<int, 7>{});
    }
    // The last NS - 1 refills lie past K and fill buffers nobody reads; drain
    // them, and let every wave finish its reads, before buf0 is reused.
    wait_vmcnt<0>();
    if constexpr (ODEC) {
        const int t = threadIdx.x;
        if (use_panel && t < kPW)
            *reinterpret_cast<h8 *>(pw + (t / (WR / 8)) * WR + 8 * (t % (WR / 8))) = piece;
        else if (use_panel && t < kPW + kPX)
            *reinterpret_cast<h8 *>(px + ((t - kPW) / (kPanelP / 8)) * kPanelP +
                                    8 * ((t - kPW) % (kPanelP / 8))) = piece;
    }
    barrier();

    // Partial sums of the four waves go through buf0 (free now).
    Acc *part = reinterpret_cast<Acc *>(buf0);   // [wave][g][t][lane]
#pragma unroll
    for (int g = 0; g < RG; g++)
#pragma unroll
        for (int t = 0; t < MT; t++)
            part[((wave * RG + g) * MT + t) * kWave + lane] = acc[g][t];
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
            Acc sum = part[((0 * RG + g) * MT + t) * kWave + lane];
#pragma unroll
            for (int w = 1; w < 4; w++)
                sum += part[((w * RG + g) * MT + t) * kWave + lane];
            const int m = 16 * t + r16;
            const int nn = n0 + 16 * g + 4 * kq;
            float r = 0.0f;  // max |fp16 output| of this lane's four outputs
            if (m < M && nn < N) {
                if constexpr (OUT_I32) {
                    *reinterpret_cast<Acc *>(static_cast<int32_t *>(Y) + (int64_t)m * N + nn) = sum;
                } else {
                    const float sxm = sx[m];
                    float outl[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    if constexpr (ODEC) {
                        // Eight outlier positions per step: one 16-byte load of XO
                        // (p0 + 8 <= K: p0 < P <= K, both multiples of 8), then
                        // four weights of each column (8 bytes: N % 4 == 0, nn % 4 == 0).
                        const int P = out_cols[0];
                        if (use_panel) {
                            // The same sum, in the same order, from the LDS panels.
                            const int ml = 16 * t + r16;
                            const int nl = nn - n0;
                            for (int p = 0; p < P; p++) {
                                const float xv = (float)px[ml * kPanelP + p];
                                const h4 wv = *reinterpret_cast<const h4 *>(pw + p * WR + nl);
#pragma unroll
                                for (int i = 0; i < 4; i++)
                                    outl[i] = fmaf(xv, (float)wv[i], outl[i]);
                            }
                        }
                        for (int p0 = 0; !use_panel && p0 < P; p0 += 8) {
                            const h8 xv =
                                *reinterpret_cast<const h8 *>(dec.xo + (int64_t)m * K + p0);
#pragma unroll
                            for (int j = 0; j < 8; j++) {
                                const int p = p0 + j;
                                if (p < P) {
                                    const int col =
                                        p < kOutCols ? out_cols[1 + p] : dec.cols[1 + p];
                                    const h4 wv = *reinterpret_cast<const h4 *>(
                                        dec.wt + (int64_t)col * N + nn);
#pragma unroll
                                    for (int i = 0; i < 4; i++)
                                        outl[i] = fmaf((float)xv[j], (float)wv[i], outl[i]);
                                }
                            }
                        }
                    }
                    h4 o;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        // The tiled kernel's expression, so both give the same bits.
                        float v;
                        if constexpr (ODEC)
                            v = fmaf((float)sum[i], sxm * sw[(nn + i) / G], outl[i]) +
                                (bias ? bias[nn + i] : 0.0f);
                        else
                            v = fmaf((float)sum[i], sxm * sw[(nn + i) / G],
                                     bias ? bias[nn + i] : 0.0f);
                        if (act == 1)
                            v = gelu_fast(v);
                        o[i] = (_Float16)v;
                    }
                    *reinterpret_cast<h4 *>(static_cast<_Float16 *>(Y) + (int64_t)m * N + nn) = o;
                    if (row_part)
                        r = fmaxf(fmaxf(fabsf((float)o[0]), fabsf((float)o[1])),
                                  fmaxf(fabsf((float)o[2]), fabsf((float)o[3])));
                }
            }
            if (!OUT_I32 && row_part) {
                // Partial max |fp16 output| of token m over this row group's 16
                // outputs (the four column quads of lanes r16 + 16 kq combined),
                // for a per-token quantizer downstream: a plain store per group.
                r = fmaxf(r, __shfl_xor(r, 16));
                r = fmaxf(r, __shfl_xor(r, 32));
                if (kq == 0 && m < M)
                    row_part[(int64_t)m * (gridDim.x * RG) + blockIdx.x * RG + g] = r;
            }
        }
    }
}

template <int MT, int RG, int BKB, int NS, bool PACKED = false, bool F8 = false,
          bool ODEC = false>
hipError_t launch_cfg(const int8_t *Xq, const float *sx, const int8_t *Wq, const float *sw,
                      int64_t G, const float *bias, int act, int64_t M, int64_t N, int64_t K,
                      void *Y, bool out_i32, hipStream_t stream, float *row_part = nullptr,
                      const OutlierOperands *dec = nullptr)
{
    const dim3 grid((unsigned)((N + 16 * RG - 1) / (16 * RG)));
    const dim3 block(kThreads);
    const OutlierOperands od = dec ? *dec : OutlierOperands{nullptr, nullptr, nullptr};
    if constexpr (ODEC)
        hipLaunchKernelGGL((k_gemm_skinny<MT, RG, BKB, NS, PACKED, false, F8, true>), grid,
                           block, 0, stream, Xq, sx, Wq, sw, (int)G, bias, act, (int)M, (int)N,
                           (int)K, Y, row_part, od);
    else if (out_i32)
        hipLaunchKernelGGL((k_gemm_skinny<MT, RG, BKB, NS, PACKED, true, F8>), grid, block, 0,
                           stream, Xq, sx, Wq, sw, (int)G, bias, act, (int)M, (int)N, (int)K, Y,
                           row_part, od);
    else
        hipLaunchKernelGGL((k_gemm_skinny<MT, RG, BKB, NS, PACKED, false, F8>), grid, block, 0,
                           stream, Xq, sx, Wq, sw, (int)G, bias, act, (int)M, (int)N, (int)K, Y,
                           row_part, od);
    return hipGetLastError();
}

// Packed weight layout: block b (rows 32 b .. 32 b + 31) and slab s (bytes
// 512 s .. 512 s + 511 of each row) form one contiguous 16 KB run at
// ((b * KS) + s) * 16384, rows 512 bytes apart; KS = ceil(K / 512).  Rows
// past N and bytes past K are zero.  One thread moves one 16-byte chunk.
__global__ __launch_bounds__(256) void k_pack_weights(const int8_t *__restrict__ Wq, int N, int K,
                                                      int KS, int64_t chunks,
                                                      int8_t *__restrict__ Wp)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < chunks;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int c = (int)(i % (kPackBytes / 16));
        const int r = (int)((i / (kPackBytes / 16)) % kPackRows);
        const int64_t bs = i / (kPackBytes / 16 * kPackRows);  // b * KS + s
        const int s = (int)(bs % KS);
        const int64_t n = bs / KS * kPackRows + r;
        const int64_t k = (int64_t)s * kPackBytes + 16 * c;
        v4i v = {0, 0, 0, 0};
        if (n < N && k < K)
            v = *reinterpret_cast<const v4i *>(Wq + n * K + k);
        *reinterpret_cast<v4i *>(Wp + 16 * i) = v;
    }
}

}  // namespace

hipError_t launch_gemm_skinny(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                              const float *w_scales, int64_t G, const float *bias, int act,
                              int64_t M, int64_t N, int64_t K, void *Y, bool out_i32,
                              hipStream_t stream, float *row_part)
{
#define ZQ_SK(MT, RG, BKB, NS)                                                                   \
    launch_cfg<MT, RG, BKB, NS>(Xq, x_scales, Wq, w_scales, G, bias, act, M, N, K, Y, out_i32,   \
                                stream, row_part)
    // 32 weight rows per workgroup (two row groups) fills 256 CUs at N = 8192;
    // 512-byte row pieces four slabs deep (measured against 256- and 1024-byte
    // pieces two to eight deep, and against cached weight loads).
    if (M <= 16)
        return ZQ_SK(1, 2, 512, 4);
    return ZQ_SK(2, 2, 512, 4);
#undef ZQ_SK
}

int64_t gemm_skinny_row_groups(int64_t N)
{
    return (N + 31) / 32 * 2;  // 32 output rows per workgroup, two row groups
}

hipError_t launch_gemm_skinny_packed(const int8_t *Xq, const float *x_scales, const int8_t *Wp,
                                     const float *w_scales, int64_t G, const float *bias, int act,
                                     int64_t M, int64_t N, int64_t K, void *Y, bool out_i32,
                                     hipStream_t stream)
{
    if (M <= 16)
        return launch_cfg<1, 2, kPackBytes, 4, true>(Xq, x_scales, Wp, w_scales, G, bias, act,
                                                           M, N, K, Y, out_i32, stream);
    return launch_cfg<2, 2, kPackBytes, 4, true>(Xq, x_scales, Wp, w_scales, G, bias, act, M,
                                                       N, K, Y, out_i32, stream);
}

hipError_t launch_gemm_skinny_fp8(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                                  const float *w_scales, int64_t G, const float *bias, int act,
                                  int64_t M, int64_t N, int64_t K, void *Y, bool out_raw,
                                  bool packed, hipStream_t stream)
{
#define ZQ_SK8(MT, P)                                                                             \
    launch_cfg<MT, 2, kPackBytes, 4, P, true>(Xq, x_scales, Wq, w_scales, G, bias, act, M, N, K, \
                                               Y, out_raw, stream)
    if (packed)
        return M <= 16 ? ZQ_SK8(1, true) : ZQ_SK8(2, true);
    return M <= 16 ? ZQ_SK8(1, false) : ZQ_SK8(2, false);
#undef ZQ_SK8
}

hipError_t launch_gemm_skinny_decomp(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                                     const float *w_scales, int64_t G, const float *bias, int act,
                                     int64_t M, int64_t N, int64_t K, const int32_t *cols,
                                     const _Float16 *XO, const _Float16 *W16t, void *Y,
                                     hipStream_t stream)
{
    const OutlierOperands dec{cols, XO, W16t};
    if (M <= 16)
        return launch_cfg<1, 2, 512, 4, false, false, true>(
            Xq, x_scales, Wq, w_scales, G, bias, act, M, N, K, Y, false, stream, nullptr, &dec);
    return launch_cfg<2, 2, 512, 4, false, false, true>(
        Xq, x_scales, Wq, w_scales, G, bias, act, M, N, K, Y, false, stream, nullptr, &dec);
}

int64_t packed_weights_bytes(int64_t N, int64_t K)
{
    return (N + kPackRows - 1) / kPackRows * kPackRows * ((K + kPackBytes - 1) / kPackBytes) *
           kPackBytes;
}

hipError_t launch_pack_weights(const int8_t *Wq, int64_t N, int64_t K, int8_t *Wp,
                               hipStream_t stream)
{
    const int64_t chunks = packed_weights_bytes(N, K) / 16;
    const int64_t blocks = std::min<int64_t>((chunks + 255) / 256, 8192);
    hipLaunchKernelGGL(k_pack_weights, dim3((unsigned)blocks), dim3(256), 0, stream, Wq, (int)N,
                       (int)K, (int)((K + kPackBytes - 1) / kPackBytes), chunks, Wp);
    return hipGetLastError();
}

}  // namespace zq
