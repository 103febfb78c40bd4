// Fused prologue for gfx950: LayerNorm or GeLU (or nothing) in fp32 registers,
// then dynamic per-token symmetric absmax quantization to int8.
//
// Pages: ZeroQuant reading notes, kernel-fusion flowchart (LN/GeLU + Quantize
// in one kernel); "探秘Transformer系列之（36）--- 大模型量化方案" 1.2.2 (token-wise
// scales computed at run time; fusing the quantizer with the preceding
// LayerNorm removes a round trip through HBM) and 1.1.2 (absmax to [-127, 127]).
//
// The kernel is HBM-bound: per token it reads K * sizeof(x) bytes and writes
// K + 4.  A token row is read once with non-temporal 16-byte loads (8 fp16 or
// 2 x 4 fp32 per chunk; consecutive lanes take consecutive chunks) by one,
// four or sixteen waves depending on its length (launch_rows), the fused
// op's result y stays in registers, the reductions (sum, sum of squares
// about the mean, absmax) run on DPP without touching LDS (and through LDS
// only across the waves of one token), and codes go out as 8-byte groups.
// The same kernel provides the fp16-output op of the unfused order, the FP8
// codes, and the two passes of the mixed-precision decomposition.  fp16 rows
// of at most 8192 elements quantized to int8 or FP8 (the prefill layers) take
// k_ln_quant_f16, the same arithmetic instantiated per op.
//
// A few tokens with long rows (the decode shape) are spread over many
// workgroups per row instead (see k_rowseg_quant).
#include "zq_device.h"
#include "zq_kernels.h"

#include <algorithm>
#include <type_traits>

namespace zq {
namespace {

// One 16-byte piece of a row: 8 fp16 (one load) or 8 fp32 (two loads).
template <typename T>
struct Chunk;

// load_nt: the same with the non-temporal hint, for data read exactly once.
template <>
struct Chunk<_Float16> {
    static __device__ __forceinline__ void load(const _Float16 *p, float (&v)[8])
    {
        const h8 h = *reinterpret_cast<const h8 *>(p);
#pragma unroll
        for (int i = 0; i < 8; i++)
            v[i] = (float)h[i];
    }
    static __device__ __forceinline__ void load_nt(const _Float16 *p, float (&v)[8])
    {
        const h8 h = __builtin_nontemporal_load(reinterpret_cast<const h8 *>(p));
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
    static __device__ __forceinline__ void load_nt(const float *p, float (&v)[8])
    {
        const v4f a = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
        const v4f b = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p + 4));
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
        v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    }
};

__device__ __forceinline__ void load8(const float *p, float (&v)[8])
{
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Codes of 8 values with scale s (rs = fl32(1/s), fast = rcp_quant_ok(s)),
// the values being elements of the vector whose absmax gave s.
//
// Reciprocal path, all 8 at once: u = fma(y, rs, 1.5 * 2^23) rounds y * rs to
// the nearest integer r (the spacing of floats in [2^23, 2^24) is 1), so the
// low byte of u's bits is r as a two's-complement int8 (|r| <= 127 leaves the
// upper bits at those of 1.5 * 2^23); r = u - 1.5 * 2^23 exactly, and
// |fma(y, rs, -r)| is y * rs's distance to r.  When every distance is at most
// 1/2 - 2^-13 (no value within 2^-13 of a half-integer), r is also the integer
// nearest to y / s (y * rs is within 2^-17 of y / s below 128), i.e. the same
// code as quant_code; otherwise, in about one group of 8 in 10^3, the group
// takes quant_code.  One test per group instead of a branch per value.
__device__ __forceinline__ uint2 quant8(const float (&y)[8], float s, float rs, bool fast)
{
    constexpr float kRound = 12582912.0f;  // 1.5 * 2^23
    if (fast) {
        uint32_t u[8];
        float far = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const float ru = fmaf(y[e], rs, kRound);
            u[e] = __float_as_uint(ru);
            far = fmaxf(far, fabsf(fmaf(y[e], rs, -(ru - kRound))));
        }
        if (far <= 0.4998779296875f) {
            uint2 packed;
            packed.x = __builtin_amdgcn_perm(__builtin_amdgcn_perm(u[3], u[2], 0x0c0c0400u),
                                             __builtin_amdgcn_perm(u[1], u[0], 0x0c0c0400u),
                                             0x05040100u);
            packed.y = __builtin_amdgcn_perm(__builtin_amdgcn_perm(u[7], u[6], 0x0c0c0400u),
                                             __builtin_amdgcn_perm(u[5], u[4], 0x0c0c0400u),
                                             0x05040100u);
            return packed;
        }
    }
    int q[8];
#pragma unroll
    for (int e = 0; e < 8; e++)
        q[e] = quant_code(y[e], s);
    uint2 packed;
    packed.x = pack4_i8(q[0], q[1], q[2], q[3]);
    packed.y = pack4_i8(q[4], q[5], q[6], q[7]);
    return packed;
}

// FP8 codes of 8 values with power-of-two scale 2^e (all 0 when the scale is 0).
__device__ __forceinline__ uint2 quant8_fp8(const float (&y)[8], float scale, int e)
{
    uint2 packed = {0u, 0u};
    if (scale != 0.0f) {
        packed.x = fp8x4(y[0], y[1], y[2], y[3], e);
        packed.y = fp8x4(y[4], y[5], y[6], y[7], e);
    }
    return packed;
}

// Block = TPB tokens x WPT waves per token.  Thread t of a token owns chunks
// t, t + 64*WPT, ... (NCH of them).  With OUT_F16 the kernel stops after the
// op and stores y as fp16 to Y16 (the unfused order, where a separate step
// quantizes that tensor); Xq and sx are then unused.
//
// DEC selects the two passes of the mixed-precision decomposition (outlier
// columns kept in fp16, LLM.int8() in "探秘Transformer系列之（36）" 1.1).  Both
// passes run this same code up to y, so they see the same bits:
//   DEC = 1: every column holding some |y| > alpha gets slot[col] = 1 (a
//            plain store of the same value from every writer); nothing else.
//   DEC = 2: slot[col] is the column's position p in the outlier list, or -1.
//            y of an outlier column goes to XO[m * K + p] as fp16 and is then
//            set to 0, so the absmax and the codes cover the other columns only
//            (their codes there are 0).
template <typename T, int NCH, int WPT, int TPB, bool OUT_F16 = false, bool FP8 = false,
          int DEC = 0>
__global__ __launch_bounds__(kWave * WPT * TPB) void k_ln_quant(
    const T *__restrict__ X, int M, int K, int pre, const float *__restrict__ gamma,
    const float *__restrict__ beta, float eps, int8_t *__restrict__ Xq, float *__restrict__ sx,
    _Float16 *__restrict__ Y16, float alpha,
    int32_t *__restrict__ slot, _Float16 *__restrict__ XO)
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

    // The row is read once, with the non-temporal hint (measured: 4096x768 7.15 ->
    // 6.53 us, 2048x4096 12.0 -> 11.0 us), except by the outlier-marking pass,
    // whose X the decomposition's second pass reads again right after.
    float y[NCH][8];
    const T *xrow = X + m * (int64_t)K;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int c = t + TT * i;
        if (live && c < nchunks) {
            if constexpr (DEC == 1)
                Chunk<T>::load(xrow + (int64_t)c * 8, y[i]);
            else
                Chunk<T>::load_nt(xrow + (int64_t)c * 8, y[i]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++)
                y[i][e] = 0.0f;
        }
    }

    if (pre == 1) {
        // LayerNorm: the mean, then the biased variance about the mean.  A row
        // of equal values c must give mean = c exactly (then y = beta).  fp16
        // rows of at most 8192 elements sum to K c exactly in fp32 (11
        // significant bits times at most 2^13), so they are summed as they are;
        // other rows are summed about their first element x0.
        constexpr bool kShift = !std::is_same<T, _Float16>::value || NCH * TT * 8 > 8192;
        const float x0 = kShift && live ? (float)xrow[0] : 0.0f;
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            if (!kShift || t + TT * i < nchunks) {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    s += kShift ? y[i][e] - x0 : y[i][e];
            }
        }
        const float mean = x0 + token_reduce(s, false) / (float)K;
        // y now holds x - mean, reused by the affine step below.
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            if (t + TT * i < nchunks) {
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float d = y[i][e] - mean;
                    ss = fmaf(d, d, ss);
                    y[i][e] = d;
                }
            }
        }
        // 1 / sqrt(var + eps) once per token in fp64, rounded once to fp32.
        const float rstd =
            (float)(1.0 / sqrt((double)(token_reduce(ss, false) / (float)K) + (double)eps));
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
                for (int e = 0; e < 8; e++)               // y = (x - mean) * rstd * g + b
                    y[i][e] = fmaf(y[i][e], rstd * g[e], b[e]);
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

    if constexpr (DEC == 1) {
        if (!live)
            return;
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int c = t + TT * i;
            if (c < nchunks) {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    if (fabsf(y[i][e]) > alpha)
                        slot[c * 8 + e] = 1;
            }
        }
        return;
    }
    if constexpr (DEC == 2) {
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int c = t + TT * i;
            if (c < nchunks) {
                const int4 s0 = *reinterpret_cast<const int4 *>(slot + c * 8);
                const int4 s1 = *reinterpret_cast<const int4 *>(slot + c * 8 + 4);
                const int sl[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    if (sl[e] >= 0) {
                        if (live)
                            XO[m * (int64_t)K + sl[e]] = (_Float16)y[i][e];
                        y[i][e] = 0.0f;
                    }
                }
            }
        }
    }

    if constexpr (OUT_F16) {
        if (!live)
            return;
        _Float16 *yrow = Y16 + m * (int64_t)K;
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int c = t + TT * i;
            if (c < nchunks) {
                h8 h;
#pragma unroll
                for (int e = 0; e < 8; e++)
                    h[e] = (_Float16)y[i][e];
                *reinterpret_cast<h8 *>(yrow + (int64_t)c * 8) = h;
            }
        }
        return;
    }

    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; i++)
#pragma unroll
        for (int e = 0; e < 8; e++)
            a = fmaxf(a, fabsf(y[i][e]));
    a = token_reduce(a, true);
    if constexpr (FP8) {
        int e;
        const float scale = fp8_scale(a, e);
        if (!live)
            return;
        int8_t *qrow = Xq + m * (int64_t)K;
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int c = t + TT * i;
            if (c < nchunks)
                *reinterpret_cast<uint2 *>(qrow + (int64_t)c * 8) = quant8_fp8(y[i], scale, e);
        }
        if (t == 0)
            sx[m] = scale;
        return;
    }
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

// ---- fp16 rows of at most 8192 elements, int8 or FP8 codes: the main path ----
//
// The arithmetic of k_ln_quant for these rows (the same bits), built once per
// op so each instantiation holds only its own registers (LayerNorm with 3
// pieces per lane: 52 VGPRs; k_ln_quant, whose op is chosen at run time,
// carries GeLU's registers into its LayerNorm code: 67).  Each cross-wave reduction
// writes its own LDS entries, so one barrier per reduction suffices, and the
// barrier waits for LDS traffic only (no drain of outstanding stores).
// Measured on the 4096 x 5120 LayerNorm prologue: 21.2 us against 23.0 us for
// k_ln_quant; 4096 x 8192: 31.0 against 35.0 us.  Giving each token group two
// or four tokens at once (shared reductions and gamma / beta loads) was
// slower (22.9 and 30.5 us), as were two waves per token (21.1 us, with a
// different summation order) and a persistent form that streams rows into an
// LDS ring by DMA (24.3 us).
template <int NCH, int WPT, int TPB, int PRE, bool FP8>
__global__ __launch_bounds__(kWave * WPT * TPB) void k_ln_quant_f16(
    const _Float16 *__restrict__ X, int M, int K, const float *__restrict__ gamma,
    const float *__restrict__ beta, float eps, int8_t *__restrict__ Xq, float *__restrict__ sx)
{
    constexpr int TT = kWave * WPT;  // threads per token
    static_assert(NCH * TT * 8 <= 8192, "fp16 rows summed unshifted have at most 8192 elements");
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int tok = wave / WPT;
    const int wig = wave % WPT;
    const int t = wig * kWave + lane;
    const int64_t m = (int64_t)blockIdx.x * TPB + tok;
    const bool live = m < M;
    const int nchunks = K / 8;

    // [0] sum, [1] sum of squares, [2] absmax: each entry is written once.
    __shared__ float red[3][TPB][WPT > 1 ? WPT : 1];
    auto token_reduce = [&](float v, int k, bool is_max) -> float {
        v = is_max ? wave_max(v) : wave_sum(v);
        if constexpr (WPT > 1) {
            if (lane == 0)
                red[k][tok][wig] = v;
            lds_barrier();
            float r = red[k][tok][0];
#pragma unroll
            for (int w = 1; w < WPT; w++)
                r = is_max ? fmaxf(r, red[k][tok][w]) : r + red[k][tok][w];
            v = r;
        }
        return v;
    };

    float y[NCH][8];
    const _Float16 *xrow = X + m * (int64_t)K;
#pragma unroll
    for (int i = 0; i < NCH; i++) {
        const int c = t + TT * i;
        if (live && c < nchunks) {
            Chunk<_Float16>::load_nt(xrow + (int64_t)c * 8, y[i]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++)
                y[i][e] = 0.0f;
        }
    }

    if constexpr (PRE == 1) {
        // Summed unshifted (exact for a row of equal values), the variance
        // about the mean with x - mean kept, rstd once per token in fp64.
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; i++)
#pragma unroll
            for (int e = 0; e < 8; e++)
                s += y[i][e];
        const float mean = 0.0f + token_reduce(s, 0, false) / (float)K;
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            if (t + TT * i < nchunks) {
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float d = y[i][e] - mean;
                    ss = fmaf(d, d, ss);
                    y[i][e] = d;
                }
            }
        }
        const float rstd =
            (float)(1.0 / sqrt((double)(token_reduce(ss, 1, false) / (float)K) + (double)eps));
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
                for (int e = 0; e < 8; e++)
                    y[i][e] = fmaf(y[i][e], rstd * g[e], b[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++)
                    y[i][e] = 0.0f;
            }
        }
    } else if constexpr (PRE == 2) {
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
    a = token_reduce(a, 2, true);
    if (!live)
        return;

    int8_t *qrow = Xq + m * (int64_t)K;
    if constexpr (FP8) {
        int e;
        const float scale = fp8_scale(a, e);
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int c = t + TT * i;
            if (c < nchunks)
                *reinterpret_cast<uint2 *>(qrow + (int64_t)c * 8) = quant8_fp8(y[i], scale, e);
        }
        if (t == 0)
            sx[m] = scale;
    } else {
        const float scale = a / 127.0f;
        const bool fast = rcp_quant_ok(scale);
        const float rs = fast ? 1.0f / scale : 0.0f;
#pragma unroll
        for (int i = 0; i < NCH; i++) {
            const int c = t + TT * i;
            if (c < nchunks)
                *reinterpret_cast<uint2 *>(qrow + (int64_t)c * 8) = quant8(y[i], scale, rs, fast);
        }
        if (t == 0)
            sx[m] = scale;
    }
}

// ---- Few tokens with long rows (the decode shape): a row over many workgroups ----
//
// Workgroup (seg, m) quantizes chunks [256 seg, 256 seg + 256) of token m.
// The token's scale needs a statistic of the whole row; every workgroup of
// the token computes it itself, over the whole row (from L2 after the first
// touch), in the same fixed order, so all of them reach the same bits and no
// workgroup waits for another.  That costs little because the statistic
// needs no GeLU per element: GeLU(x) = x Phi(x) increases on [x0, inf) and
// decreases on (-inf, x0], x0 = -0.7517915 its minimum, where it is -0.16997.
// So when max_k x_k >= 0.3 (GeLU(0.3) = 0.185), max_k |GeLU(x_k)| is
// GeLU(max_k x_k); otherwise it is the largest of |GeLU| at max_k x_k, at
// L = the largest x_k <= x0 and at R = the smallest x_k > x0, found by a
// second pass.  Without an op the statistic is max(max x, -min x); max and
// min of fp16 rows run on packed fp16 pairs (exact).  LayerNorm needs the
// mean, the variance about it and max |y_k|, three passes of a few flops per
// element.

constexpr int kSegThreads = 256;
constexpr int kSegElems = kSegThreads * 8;  // elements per workgroup

constexpr float kGeluArgMin = -0.75179152f;
constexpr float kGeluPosBound = 0.3f;   // GeLU(x) > max over x < 0 of |GeLU(x)| for x >= 0.3
constexpr int64_t kRowSegMaxM = 64;     // token counts that leave most CUs idle otherwise
constexpr int64_t kRowSegMinK = 4096;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Running max and min of a row, loaded RB chunks per thread at a time.
template <typename T>
struct RowMinMax;

template <>
struct RowMinMax<_Float16> {
    static constexpr int RB = 16;
    using Raw = h8;
    h2 mx = {-(_Float16)__builtin_inff(), -(_Float16)__builtin_inff()};
    h2 mn = {(_Float16)__builtin_inff(), (_Float16)__builtin_inff()};
    static __device__ __forceinline__ Raw load(const _Float16 *p)
    {
        return *reinterpret_cast<const h8 *>(p);
    }
    __device__ __forceinline__ void add(const Raw &v)
    {
        mx = __builtin_elementwise_max(mx, v.s01);
        mx = __builtin_elementwise_max(mx, v.s23);
        mx = __builtin_elementwise_max(mx, v.s45);
        mx = __builtin_elementwise_max(mx, v.s67);
        mn = __builtin_elementwise_min(mn, v.s01);
        mn = __builtin_elementwise_min(mn, v.s23);
        mn = __builtin_elementwise_min(mn, v.s45);
        mn = __builtin_elementwise_min(mn, v.s67);
    }
    __device__ __forceinline__ float max() const { return fmaxf((float)mx.x, (float)mx.y); }
    __device__ __forceinline__ float min() const { return fminf((float)mn.x, (float)mn.y); }
};

template <>
struct RowMinMax<float> {
    static constexpr int RB = 8;
    struct Raw {
        float4 a, b;
    };
    float mx = -__builtin_inff(), mn = __builtin_inff();
    static __device__ __forceinline__ Raw load(const float *p)
    {
        return Raw{*reinterpret_cast<const float4 *>(p), *reinterpret_cast<const float4 *>(p + 4)};
    }
    __device__ __forceinline__ void add(const Raw &v)
    {
        mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(v.a.x, v.a.y), fmaxf(v.a.z, v.a.w)),
                             fmaxf(fmaxf(v.b.x, v.b.y), fmaxf(v.b.z, v.b.w))));
        mn = fminf(mn, fminf(fminf(fminf(v.a.x, v.a.y), fminf(v.a.z, v.a.w)),
                             fminf(fminf(v.b.x, v.b.y), fminf(v.b.z, v.b.w))));
    }
    __device__ __forceinline__ float max() const { return mx; }
    __device__ __forceinline__ float min() const { return mn; }
};

template <bool IS_MAX>
__device__ __forceinline__ float block_reduce(float v, float *red)
{
    v = IS_MAX ? wave_max(v) : wave_sum(v);
    __syncthreads();  // red is reused by consecutive reductions
    if (threadIdx.x % kWave == 0)
        red[threadIdx.x / kWave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kSegThreads / kWave; w++)
        r = IS_MAX ? fmaxf(r, red[w]) : r + red[w];
    return r;
}

// 1-D grid of 8 * ceil(M / 8) * nseg workgroups.  Workgroup b runs on XCD
// b % 8; token m's workgroups all get b % 8 == m % 8, so the token's row is
// fetched into one L2 and re-read from there.
template <typename T, int PRE, bool FP8>
__global__ __launch_bounds__(kSegThreads) void k_rowseg_quant(
    const T *__restrict__ X, int M, int K, int nseg, const float *__restrict__ gamma,
    const float *__restrict__ beta, float eps, int8_t *__restrict__ Xq, float *__restrict__ sx)
{
    __shared__ float red[kSegThreads / kWave];
    const int j = blockIdx.x / 8;
    const int seg = j % nseg;
    const int64_t m = (int64_t)(j / nseg) * 8 + blockIdx.x % 8;
    if (m >= M)
        return;
    const T *xrow = X + m * (int64_t)K;
    const int nch = K / 8;
    const int own = seg * kSegThreads + threadIdx.x;  // this thread's chunk
    const float inf = __builtin_inff();

    float mine[8];
    if (own < nch) {
        Chunk<T>::load(xrow + (int64_t)own * 8, mine);
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++)
            mine[e] = 0.0f;
    }

    float a, mean = 0.0f, rstd = 0.0f;
    if constexpr (PRE == 1) {
        // Mean about the row's first element (exact for a row of equal values).
        const float x0 = (float)xrow[0];
        float s = 0.0f;
#pragma unroll 4
        for (int c = threadIdx.x; c < nch; c += kSegThreads) {
            float v[8];
            Chunk<T>::load(xrow + (int64_t)c * 8, v);
#pragma unroll
            for (int e = 0; e < 8; e++)
                s += v[e] - x0;
        }
        mean = x0 + block_reduce<false>(s, red) / (float)K;
        float ss = 0.0f;
#pragma unroll 4
        for (int c = threadIdx.x; c < nch; c += kSegThreads) {
            float v[8];
            Chunk<T>::load(xrow + (int64_t)c * 8, v);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float d = v[e] - mean;
                ss += d * d;
            }
        }
        rstd = (float)(1.0 / sqrt((double)(block_reduce<false>(ss, red) / (float)K) + (double)eps));
        float amax = 0.0f;
#pragma unroll 2
        for (int c = threadIdx.x; c < nch; c += kSegThreads) {
            float v[8], g[8], b[8];
            Chunk<T>::load(xrow + (int64_t)c * 8, v);
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
                amax = fmaxf(amax, fabsf(fmaf(v[e] - mean, rstd * g[e], b[e])));
        }
        a = block_reduce<true>(amax, red);
    } else {
        // Max and min of the row, RB chunks per thread in flight at a time.
        using MM = RowMinMax<T>;
        MM mm;
        for (int base = threadIdx.x; base < nch; base += kSegThreads * MM::RB) {
            typename MM::Raw raw[MM::RB];
#pragma unroll
            for (int i = 0; i < MM::RB; i++)
                if (base + kSegThreads * i < nch)
                    raw[i] = MM::load(xrow + (int64_t)(base + kSegThreads * i) * 8);
#pragma unroll
            for (int i = 0; i < MM::RB; i++)
                if (base + kSegThreads * i < nch)
                    mm.add(raw[i]);
        }
        const float xmax = block_reduce<true>(mm.max(), red);
        if constexpr (PRE == 0) {
            const float xmin = -block_reduce<true>(-mm.min(), red);
            a = fmaxf(xmax, -xmin);
        } else {
            a = fabsf(gelu_erf(xmax));
            if (!(xmax >= kGeluPosBound)) {
                // The negative side may win: find L and R (uniform per token).
                float lo = -inf, hi = inf;
#pragma unroll 4
                for (int c = threadIdx.x; c < nch; c += kSegThreads) {
                    float v[8];
                    Chunk<T>::load(xrow + (int64_t)c * 8, v);
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        lo = fmaxf(lo, v[e] <= kGeluArgMin ? v[e] : -inf);
                        hi = fminf(hi, v[e] > kGeluArgMin ? v[e] : inf);
                    }
                }
                const float L = block_reduce<true>(lo, red);
                const float R = -block_reduce<true>(-hi, red);
                if (L > -inf)
                    a = fmaxf(a, fabsf(gelu_erf(L)));
                if (R < inf)
                    a = fmaxf(a, fabsf(gelu_erf(R)));
            }
        }
    }

    int e = 0;
    const float scale = FP8 ? fp8_scale(a, e) : a / 127.0f;
    const bool fast = !FP8 && rcp_quant_ok(scale);
    const float rs = fast ? 1.0f / scale : 0.0f;
    if (own < nch) {
        float y[8];
        if constexpr (PRE == 2) {
#pragma unroll
            for (int e = 0; e < 8; e++)
                y[e] = gelu_erf(mine[e]);
        } else if constexpr (PRE == 1) {
            float g[8], b[8];
            if (gamma) {
                load8(gamma + own * 8, g);
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++) g[e] = 1.0f;
            }
            if (beta) {
                load8(beta + own * 8, b);
            } else {
#pragma unroll
                for (int e = 0; e < 8; e++) b[e] = 0.0f;
            }
#pragma unroll
            for (int e = 0; e < 8; e++)
                y[e] = fmaf(mine[e] - mean, rstd * g[e], b[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++)
                y[e] = mine[e];
        }
        *reinterpret_cast<uint2 *>(Xq + m * K + (int64_t)own * 8) =
            FP8 ? quant8_fp8(y, scale, e) : quant8(y, scale, rs, fast);
    }
    if (seg == 0 && threadIdx.x == 0)
        sx[m] = scale;
}

// ---- The mixed-precision decomposition's two passes for few tokens ----
//
// Outlier marks without a LayerNorm (y of an element depends on that element
// alone): workgroup c decides columns [128 c, 128 c + 128) over every token
// and writes slot[col] = 1 or 0 for each, so the marks need no clearing first
// and the erf GeLU of a few long rows is spread over many CUs.  Thread (r, q)
// takes 8-column chunk q of the workgroup's columns for tokens r, r + 16, ...;
// the 16 partial masks meet in LDS.  Same test as the one-pass kernel's
// marking mode: |y| > alpha.
constexpr int kMarkChunks = 16;  // 8-column chunks per workgroup
constexpr int kMarkRows = kSegThreads / kMarkChunks;

template <typename T, int PRE>
__global__ __launch_bounds__(kSegThreads) void k_mark_cols(const T *__restrict__ X, int M, int K,
                                                           float alpha,
                                                           int32_t *__restrict__ slot)
{
    __shared__ uint32_t part[kSegThreads];
    const int q = threadIdx.x % kMarkChunks;
    const int r = threadIdx.x / kMarkChunks;
    const int c = blockIdx.x * kMarkChunks + q;
    const int nch = K / 8;
    uint32_t mask = 0;  // bit e: column 8 c + e
    if (c < nch) {
        for (int m = r; m < M; m += kMarkRows) {
            float v[8];
            Chunk<T>::load(X + (int64_t)m * K + (int64_t)c * 8, v);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float y = PRE == 2 ? gelu_erf(v[e]) : v[e];
                if (fabsf(y) > alpha)
                    mask |= 1u << e;
            }
        }
    }
    part[threadIdx.x] = mask;
    __syncthreads();
    if (r == 0 && c < nch) {
        uint32_t all = 0;
#pragma unroll
        for (int i = 0; i < kMarkRows; i++)
            all |= part[i * kMarkChunks + q];
        const int4 lo = make_int4(all & 1, (all >> 1) & 1, (all >> 2) & 1, (all >> 3) & 1);
        const int4 hi = make_int4((all >> 4) & 1, (all >> 5) & 1, (all >> 6) & 1, (all >> 7) & 1);
        *reinterpret_cast<int4 *>(slot + (int64_t)c * 8) = lo;
        *reinterpret_cast<int4 *>(slot + (int64_t)c * 8 + 4) = hi;
    }
}

// The INT8 part's prologue for few tokens with long rows, laid out as
// k_rowseg_quant: workgroup (seg, m) codes chunks [256 seg, 256 seg + 256) of
// token m, after taking the row statistic over the whole row itself.  The
// statistic is max |y| over the columns outside O (slot < 0), as in the
// one-pass kernel's mode 2 (whose zeroed outlier values add nothing to it):
// for LayerNorm a third pass over y with the mask; otherwise the masked max
// and min of x (and, for GeLU, the masked L and R of k_rowseg_quant's rule),
// so GeLU is evaluated on the workgroup's own chunk only.  An empty set
// outside O gives 0.  Outlier values of the own chunk go to XO[m * K + p] as
// fp16 and are then coded as 0.
template <typename T, int PRE>
__global__ __launch_bounds__(kSegThreads) void k_rowseg_decomp(
    const T *__restrict__ X, int M, int K, int nseg, const float *__restrict__ gamma,
    const float *__restrict__ beta, float eps, const int32_t *__restrict__ slot,
    int8_t *__restrict__ Xq, float *__restrict__ sx, _Float16 *__restrict__ XO)
{
    __shared__ float red[kSegThreads / kWave];
    const int j = blockIdx.x / 8;
    const int seg = j % nseg;
    const int64_t m = (int64_t)(j / nseg) * 8 + blockIdx.x % 8;
    if (m >= M)
        return;
    const T *xrow = X + m * (int64_t)K;
    const int nch = K / 8;
    const int own = seg * kSegThreads + threadIdx.x;
    const float inf = __builtin_inff();
    auto load_slot = [&](int c, int (&sl)[8]) {
        const int4 s0 = *reinterpret_cast<const int4 *>(slot + (int64_t)c * 8);
        const int4 s1 = *reinterpret_cast<const int4 *>(slot + (int64_t)c * 8 + 4);
        sl[0] = s0.x; sl[1] = s0.y; sl[2] = s0.z; sl[3] = s0.w;
        sl[4] = s1.x; sl[5] = s1.y; sl[6] = s1.z; sl[7] = s1.w;
    };
    auto load_affine = [&](int c, float (&g)[8], float (&b)[8]) {
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
    };

    float mine[8];
    int osl[8];
    if (own < nch) {
        Chunk<T>::load(xrow + (int64_t)own * 8, mine);
        load_slot(own, osl);
    } else {
#pragma unroll
        for (int e = 0; e < 8; e++) {
            mine[e] = 0.0f;
            osl[e] = -1;
        }
    }

    float a = 0.0f, mean = 0.0f, rstd = 0.0f;
    if constexpr (PRE == 1) {
        // Mean about the row's first element (exact for a row of equal values).
        const float x0 = (float)xrow[0];
        float s = 0.0f;
#pragma unroll 4
        for (int c = threadIdx.x; c < nch; c += kSegThreads) {
            float v[8];
            Chunk<T>::load(xrow + (int64_t)c * 8, v);
#pragma unroll
            for (int e = 0; e < 8; e++)
                s += v[e] - x0;
        }
        mean = x0 + block_reduce<false>(s, red) / (float)K;
        float ss = 0.0f;
#pragma unroll 4
        for (int c = threadIdx.x; c < nch; c += kSegThreads) {
            float v[8];
            Chunk<T>::load(xrow + (int64_t)c * 8, v);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float d = v[e] - mean;
                ss += d * d;
            }
        }
        rstd = (float)(1.0 / sqrt((double)(block_reduce<false>(ss, red) / (float)K) + (double)eps));
        float amax = 0.0f;
#pragma unroll 2
        for (int c = threadIdx.x; c < nch; c += kSegThreads) {
            float v[8], g[8], b[8];
            int sl[8];
            Chunk<T>::load(xrow + (int64_t)c * 8, v);
            load_slot(c, sl);
            load_affine(c, g, b);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float y = fmaf(v[e] - mean, rstd * g[e], b[e]);
                if (sl[e] < 0)
                    amax = fmaxf(amax, fabsf(y));
            }
        }
        a = block_reduce<true>(amax, red);
    } else {
        // Masked max and min of x, kBatch chunks per thread loaded at a time.
        constexpr int kBatch = 8;
        float mx = -inf, mn = inf;
        for (int base = threadIdx.x; base < nch; base += kSegThreads * kBatch) {
            float v[kBatch][8];
            int sl[kBatch][8];
#pragma unroll
            for (int i = 0; i < kBatch; i++) {
                const int c = base + kSegThreads * i;
                if (c < nch) {
                    Chunk<T>::load(xrow + (int64_t)c * 8, v[i]);
                    load_slot(c, sl[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < kBatch; i++) {
                if (base + kSegThreads * i < nch) {
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        mx = fmaxf(mx, sl[i][e] < 0 ? v[i][e] : -inf);
                        mn = fminf(mn, sl[i][e] < 0 ? v[i][e] : inf);
                    }
                }
            }
        }
        const float xmax = block_reduce<true>(mx, red);
        const float xmin = -block_reduce<true>(-mn, red);
        if (xmax > -inf) {  // some column outside O
            if constexpr (PRE == 0) {
                a = fmaxf(xmax, -xmin);
            } else {
                a = fabsf(gelu_erf(xmax));
                if (!(xmax >= kGeluPosBound)) {
                    float lo = -inf, hi = inf;
#pragma unroll 4
                    for (int c = threadIdx.x; c < nch; c += kSegThreads) {
                        float v[8];
                        int sl[8];
                        Chunk<T>::load(xrow + (int64_t)c * 8, v);
                        load_slot(c, sl);
#pragma unroll
                        for (int e = 0; e < 8; e++) {
                            lo = fmaxf(lo, sl[e] < 0 && v[e] <= kGeluArgMin ? v[e] : -inf);
                            hi = fminf(hi, sl[e] < 0 && v[e] > kGeluArgMin ? v[e] : inf);
                        }
                    }
                    const float L = block_reduce<true>(lo, red);
                    const float R = -block_reduce<true>(-hi, red);
                    if (L > -inf)
                        a = fmaxf(a, fabsf(gelu_erf(L)));
                    if (R < inf)
                        a = fmaxf(a, fabsf(gelu_erf(R)));
                }
            }
        }
    }

    const float scale = a / 127.0f;
    const bool fast = rcp_quant_ok(scale);
    const float rs = fast ? 1.0f / scale : 0.0f;
    if (own < nch) {
        float y[8];
        if constexpr (PRE == 2) {
#pragma unroll
            for (int e = 0; e < 8; e++)
                y[e] = gelu_erf(mine[e]);
        } else if constexpr (PRE == 1) {
            float g[8], b[8];
            load_affine(own, g, b);
#pragma unroll
            for (int e = 0; e < 8; e++)
                y[e] = fmaf(mine[e] - mean, rstd * g[e], b[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; e++)
                y[e] = mine[e];
        }
#pragma unroll
        for (int e = 0; e < 8; e++) {
            if (osl[e] >= 0) {
                XO[m * (int64_t)K + osl[e]] = (_Float16)y[e];
                y[e] = 0.0f;
            }
        }
        *reinterpret_cast<uint2 *>(Xq + m * K + (int64_t)own * 8) = quant8(y, scale, rs, fast);
    }
    if (seg == 0 && threadIdx.x == 0)
        sx[m] = scale;
}

// MAXN: the most 16-byte pieces per lane this shape is launched with (cases
// above it are not instantiated; a row needing more is an invalid launch).
template <typename T, int WPT, int TPB, bool OUT_F16 = false, bool FP8 = false, int DEC = 0,
          int MAXN = 16>
hipError_t launch_cfg(const T *X, int64_t M, int64_t K, int pre, const float *gamma,
                      const float *beta, float eps, int8_t *Xq, float *sx, hipStream_t stream,
                      _Float16 *Y16 = nullptr, float alpha = 0.0f,
                      int32_t *slot = nullptr, _Float16 *XO = nullptr)
{
    const int64_t nchunks = K / 8;
    const int64_t per = (nchunks + kWave * WPT - 1) / (kWave * WPT);
    const dim3 grid((unsigned)((M + TPB - 1) / TPB));
    const dim3 block(kWave * WPT * TPB);
#define ZQ_LNQ_CASE(n)                                                                          \
    if constexpr (n <= MAXN)                                                                    \
    if (per <= n) {                                                                             \
        hipLaunchKernelGGL((k_ln_quant<T, n, WPT, TPB, OUT_F16, FP8, DEC>), grid, block, 0,     \
                           stream, X, (int)M, (int)K, pre, gamma, beta, eps, Xq, sx, Y16,       \
                           alpha, slot, XO);                                                    \
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

// k_ln_quant_f16, one instantiation per op and per exact piece count NCH
// (so only a lane's last piece can lie past the row's end).
template <int WPT, int TPB, int PRE, bool FP8>
hipError_t launch_f16_op(const _Float16 *X, int64_t M, int64_t K, const float *gamma,
                         const float *beta, float eps, int8_t *Xq, float *sx, hipStream_t stream)
{
    const int64_t per = (K / 8 + kWave * WPT - 1) / (kWave * WPT);
    const dim3 grid((unsigned)((M + TPB - 1) / TPB));
    const dim3 block(kWave * WPT * TPB);
#define ZQ_F16_CASE(n)                                                                            \
    case n:                                                                                       \
        hipLaunchKernelGGL((k_ln_quant_f16<n, WPT, TPB, PRE, FP8>), grid, block, 0, stream, X,    \
                           (int)M, (int)K, gamma, beta, eps, Xq, sx);                             \
        return hipGetLastError();
    switch (per) {
    ZQ_F16_CASE(1)
    ZQ_F16_CASE(2)
    ZQ_F16_CASE(3)
    ZQ_F16_CASE(4)
    default: return hipErrorInvalidValue;
    }
#undef ZQ_F16_CASE
}

template <int WPT, int TPB, bool FP8>
hipError_t launch_f16(const _Float16 *X, int64_t M, int64_t K, int pre, const float *gamma,
                      const float *beta, float eps, int8_t *Xq, float *sx, hipStream_t stream)
{
    if (pre == 1)
        return launch_f16_op<WPT, TPB, 1, FP8>(X, M, K, gamma, beta, eps, Xq, sx, stream);
    if (pre == 2)
        return launch_f16_op<WPT, TPB, 2, FP8>(X, M, K, gamma, beta, eps, Xq, sx, stream);
    return launch_f16_op<WPT, TPB, 0, FP8>(X, M, K, gamma, beta, eps, Xq, sx, stream);
}

// Waves per token by row length.  Rows up to 2048 elements take one wave
// (four tokens per block).  Up to 8192 they take four waves (one token per
// block): each lane then holds at most four 16-byte pieces of the row, few
// enough registers for six to eight waves per SIMD, so the loads of some
// tokens overlap the arithmetic of others (one wave per token, holding up to
// 16 pieces, left room for two or three).  Longer rows take 16 waves.
template <typename T, bool OUT_F16, bool FP8, int DEC>
hipError_t launch_rows(const T *X, int64_t M, int64_t K, int pre, const float *gamma,
                       const float *beta, float eps, int8_t *Xq, float *sx, hipStream_t stream,
                       _Float16 *Y16, float alpha = 0.0f,
                       int32_t *slot = nullptr, _Float16 *XO = nullptr)
{
    if constexpr (std::is_same<T, _Float16>::value && !OUT_F16 && DEC == 0) {
        // fp16 rows up to 8192 elements to codes: k_ln_quant_f16
        if (K <= 2048)
            return launch_f16<1, 4, FP8>(X, M, K, pre, gamma, beta, eps, Xq, sx, stream);
        if (K <= 8192)
            return launch_f16<4, 1, FP8>(X, M, K, pre, gamma, beta, eps, Xq, sx, stream);
    } else {
        if (K <= 2048)
            return launch_cfg<T, 1, 4, OUT_F16, FP8, DEC, 4>(X, M, K, pre, gamma, beta, eps, Xq,
                                                             sx, stream, Y16, alpha, slot, XO);
        if (K <= 8192)
            return launch_cfg<T, 4, 1, OUT_F16, FP8, DEC, 4>(X, M, K, pre, gamma, beta, eps, Xq,
                                                             sx, stream, Y16, alpha, slot, XO);
    }
    return launch_cfg<T, 16, 1, OUT_F16, FP8, DEC, 16>(X, M, K, pre, gamma, beta, eps, Xq, sx,
                                                       stream, Y16, alpha, slot, XO);
}

template <typename T>
hipError_t launch_typed(const T *X, int64_t M, int64_t K, int pre, const float *gamma,
                        const float *beta, float eps, int8_t *Xq, float *sx, hipStream_t stream,
                        bool fp8)
{
    // Few tokens with long rows: spread each row over ceil(K / 2048) workgroups.
    if (M <= kRowSegMaxM && K >= kRowSegMinK) {
        const int nseg = (int)((K + kSegElems - 1) / kSegElems);
        const dim3 grid((unsigned)(8 * ((M + 7) / 8) * nseg));
#define ZQ_ROWSEG(P, F)                                                                           \
    hipLaunchKernelGGL((k_rowseg_quant<T, P, F>), grid, dim3(kSegThreads), 0, stream, X, (int)M,  \
                       (int)K, nseg, gamma, beta, eps, Xq, sx)
        if (fp8) {
            if (pre == 1)
                ZQ_ROWSEG(1, true);
            else if (pre == 2)
                ZQ_ROWSEG(2, true);
            else
                ZQ_ROWSEG(0, true);
        } else {
            if (pre == 1)
                ZQ_ROWSEG(1, false);
            else if (pre == 2)
                ZQ_ROWSEG(2, false);
            else
                ZQ_ROWSEG(0, false);
        }
#undef ZQ_ROWSEG
        return hipGetLastError();
    }
    if (fp8)
        return launch_rows<T, false, true, 0>(X, M, K, pre, gamma, beta, eps, Xq, sx, stream,
                                              nullptr);
    return launch_rows<T, false, false, 0>(X, M, K, pre, gamma, beta, eps, Xq, sx, stream,
                                           nullptr);
}

}  // namespace

hipError_t launch_ln_to_f16(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                            const float *gamma, const float *beta, float eps, _Float16 *Y16,
                            hipStream_t stream)
{
    if (x_f16)
        return launch_rows<_Float16, true, false, 0>(static_cast<const _Float16 *>(X), M, K, pre,
                                                     gamma, beta, eps, nullptr, nullptr, stream,
                                                     Y16);
    return launch_rows<float, true, false, 0>(static_cast<const float *>(X), M, K, pre, gamma, beta,
                                              eps, nullptr, nullptr, stream, Y16);
}

namespace {
template <typename T, int DEC>
hipError_t launch_decomp_typed(const T *X, int64_t M, int64_t K, int pre, const float *gamma,
                               const float *beta, float eps, float alpha, int32_t *slot,
                               int8_t *Xq, float *sx, _Float16 *XO, hipStream_t stream)
{
    return launch_rows<T, false, false, DEC>(X, M, K, pre, gamma, beta, eps, Xq, sx, stream,
                                             nullptr, alpha, slot, XO);
}
}  // namespace

bool outlier_detect_writes_all(int64_t M, int64_t K, int pre)
{
    return M >= 1 && M <= kRowSegMaxM && K >= kRowSegMinK && pre != 1;
}

hipError_t launch_outlier_detect(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                                 const float *gamma, const float *beta, float eps, float alpha,
                                 int32_t *slot, hipStream_t stream)
{
    if (outlier_detect_writes_all(M, K, pre)) {
        const dim3 grid((unsigned)((K / 8 + kMarkChunks - 1) / kMarkChunks));
#define ZQ_MARK(T, P)                                                                            \
    hipLaunchKernelGGL((k_mark_cols<T, P>), grid, dim3(kSegThreads), 0, stream,                   \
                       static_cast<const T *>(X), (int)M, (int)K, alpha, slot)
        if (x_f16) {
            if (pre == 2)
                ZQ_MARK(_Float16, 2);
            else
                ZQ_MARK(_Float16, 0);
        } else {
            if (pre == 2)
                ZQ_MARK(float, 2);
            else
                ZQ_MARK(float, 0);
        }
#undef ZQ_MARK
        return hipGetLastError();
    }
    if (x_f16)
        return launch_decomp_typed<_Float16, 1>(static_cast<const _Float16 *>(X), M, K, pre, gamma,
                                                beta, eps, alpha, slot, nullptr, nullptr, nullptr,
                                                stream);
    return launch_decomp_typed<float, 1>(static_cast<const float *>(X), M, K, pre, gamma, beta,
                                         eps, alpha, slot, nullptr, nullptr, nullptr, stream);
}

hipError_t launch_ln_quant_decomp(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                                  const float *gamma, const float *beta, float eps,
                                  const int32_t *slot, int8_t *Xq, float *x_scales, _Float16 *XO,
                                  hipStream_t stream)
{
    if (M <= kRowSegMaxM && K >= kRowSegMinK) {
        const int nseg = (int)((K + kSegElems - 1) / kSegElems);
        const dim3 grid((unsigned)(8 * ((M + 7) / 8) * nseg));
#define ZQ_RSD(T, P)                                                                             \
    hipLaunchKernelGGL((k_rowseg_decomp<T, P>), grid, dim3(kSegThreads), 0, stream,               \
                       static_cast<const T *>(X), (int)M, (int)K, nseg, gamma, beta, eps, slot,   \
                       Xq, x_scales, XO)
        if (x_f16) {
            if (pre == 1)
                ZQ_RSD(_Float16, 1);
            else if (pre == 2)
                ZQ_RSD(_Float16, 2);
            else
                ZQ_RSD(_Float16, 0);
        } else {
            if (pre == 1)
                ZQ_RSD(float, 1);
            else if (pre == 2)
                ZQ_RSD(float, 2);
            else
                ZQ_RSD(float, 0);
        }
#undef ZQ_RSD
        return hipGetLastError();
    }
    int32_t *sl = const_cast<int32_t *>(slot);  // read only in this pass
    if (x_f16)
        return launch_decomp_typed<_Float16, 2>(static_cast<const _Float16 *>(X), M, K, pre, gamma,
                                                beta, eps, 0.0f, sl, Xq, x_scales, XO, stream);
    return launch_decomp_typed<float, 2>(static_cast<const float *>(X), M, K, pre, gamma, beta,
                                         eps, 0.0f, sl, Xq, x_scales, XO, stream);
}

hipError_t launch_ln_quant(const void *X, bool x_f16, int64_t M, int64_t K, int pre,
                           const float *gamma, const float *beta, float eps, int8_t *Xq,
                           float *x_scales, hipStream_t stream, bool fp8)
{
    if (x_f16)
        return launch_typed(static_cast<const _Float16 *>(X), M, K, pre, gamma, beta, eps, Xq,
                            x_scales, stream, fp8);
    return launch_typed(static_cast<const float *>(X), M, K, pre, gamma, beta, eps, Xq, x_scales,
                        stream, fp8);
}

// Codes of fp16 rows whose absmax comes from partial maxima: part[m * groups + j]
// holds max |Y[m, n]| over column group j (written by the producing GEMM's
// epilogue), so max_j part[m * groups + j] is the row's absmax exactly.  One
// workgroup per row: the partials are combined first, then s = fl32(a / 127)
// as the prologue computes it and the same quantizer.
namespace {
constexpr int kQpThreads = 128;

__global__ __launch_bounds__(kQpThreads) void k_quant_rows_part(
    const _Float16 *__restrict__ Y, int K, const float *__restrict__ part, int groups,
    int8_t *__restrict__ Xq, float *__restrict__ sx)
{
    __shared__ float red[kQpThreads / kWave];
    const int64_t m = blockIdx.x;
    float a = 0.0f;
    for (int j = threadIdx.x; j < groups; j += kQpThreads)
        a = fmaxf(a, part[m * groups + j]);
    a = wave_max(a);
    if (threadIdx.x % kWave == 0)
        red[threadIdx.x / kWave] = a;
    __syncthreads();
    a = red[0];
#pragma unroll
    for (int w = 1; w < kQpThreads / kWave; w++)
        a = fmaxf(a, red[w]);
    const float scale = a / 127.0f;
    const bool fast = rcp_quant_ok(scale);
    const float rs = fast ? 1.0f / scale : 0.0f;
    const _Float16 *yrow = Y + m * (int64_t)K;
    int8_t *qrow = Xq + m * (int64_t)K;
    for (int c = threadIdx.x; c < K / 8; c += kQpThreads) {
        float y[8];
        Chunk<_Float16>::load(yrow + (int64_t)c * 8, y);
        *reinterpret_cast<uint2 *>(qrow + (int64_t)c * 8) = quant8(y, scale, rs, fast);
    }
    if (threadIdx.x == 0)
        sx[m] = scale;
}
}  // namespace

hipError_t launch_quant_rows_part(const _Float16 *Y, int64_t M, int64_t K, const float *part,
                                  int64_t groups, int8_t *Xq, float *x_scales, hipStream_t stream)
{
    if (M < 1)
        return hipSuccess;
    hipLaunchKernelGGL(k_quant_rows_part, dim3((unsigned)M), dim3(kQpThreads), 0, stream, Y,
                       (int)K, part, (int)groups, Xq, x_scales);
    return hipGetLastError();
}

}  // namespace zq
