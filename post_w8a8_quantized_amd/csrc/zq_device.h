// Device helpers shared by the gfx950 kernels of libzq (not by anything else).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Exact (erf) GeLU, gelu(x) = x * Phi(x), evaluated in fp32 without erff.
// Phi(x) = 1 - erfc(z)/2 for x >= 0 and erfc(z)/2 for x < 0, z = |x| / sqrt 2,
// with erfc from the Chebyshev-fitted form of Numerical Recipes ("erfcc":
// t = 1/(1 + z/2), erfc(z) = t exp(-z^2 + P(t)), P of degree 9, fractional
// error below 1.2e-7 for all z >= 0).  Taking erfc on the negative side
// keeps the relative accuracy in the tail.  Branch-free, about 20 VALU
// instructions versus about 50 for the device library's erff.  Measured in
// fp32 against exact GeLU: relative error <= 2.1e-5 (only far in the tail,
// from rounding -z^2), fp16 results never differ by more than 1 ulp.
__device__ __forceinline__ float gelu_erf(float x)
{
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
    float p = 0.17087277f;
    p = fmaf(p, t, -0.82215223f);
    p = fmaf(p, t, 1.48851587f);
    p = fmaf(p, t, -1.13520398f);
    p = fmaf(p, t, 0.27886807f);
    p = fmaf(p, t, -0.18628806f);
    p = fmaf(p, t, 0.09678418f);
    p = fmaf(p, t, 0.37409196f);
    p = fmaf(p, t, 1.00002368f);
    p = fmaf(p, t, -1.26551223f);
    const float e = __builtin_amdgcn_exp2f(fmaf(-z, z, p) * 1.4426950408889634f);
    const float h = 0.5f * t * e;
    return x * (x >= 0.0f ? 1.0f - h : h);
}

// GeLU for the fp16 epilogues: GeLU(x) = max(x, 0) - |x| Phi(-|x|) with
// Phi(-u) = exp2(P(u)), P a degree-7 polynomial approximating log2 Phi(-u)
// (fitted here by iteratively reweighted least squares on [0, 6.5]; max error
// 6.7e-6 in log2 units there).  P's leading coefficient is negative and its
// degree odd: evaluated in fp32 it stays below -34.5 for every u > 6.5 up to
// the fp32 range (u Phi(-u) < 3e-15 there, -inf once Horner overflows, whose
// exp2 is 0), so u needs no clamp.  Measured in fp32 against exact GeLU:
// relative error <= 5.7e-6 for |x| <= 4, absolute error <= 8.1e-7
// everywhere, fp16 results never more than 1 ulp from the exact ones.  Nine
// VALU instructions (seven FMAs, a max, an FMA) and one exp2.
__device__ __forceinline__ float gelu_fast(float x)
{
    const float u = fabsf(x);
    float e = -1.75778052e-06f;
    e = fmaf(e, u, 5.99366795e-05f);
    e = fmaf(e, u, -0.000916363904f);
    e = fmaf(e, u, 0.00844739005f);
    e = fmaf(e, u, -0.0538245142f);
    e = fmaf(e, u, -0.45861569f);
    e = fmaf(e, u, -1.15118015f);
    e = fmaf(e, u, -1.00000381f);
    return fmaf(-u, __builtin_amdgcn_exp2f(e), fmaxf(x, 0.0f));
}

// Symmetric absmax code: clamp(round_half_even(fl32(v / s)), -127, 127); s == 0 gives 0.
// The division is IEEE-correct (HIP's default for fp32 '/').
__device__ __forceinline__ int quant_code(float v, float s)
{
    if (s == 0.0f)
        return 0;
    float r = __builtin_rintf(v / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// The same code from t = v * rs with rs = fl32(1 / s), without a division in
// the common case.  t is within 3 ulp of v / s and fl32(v / s) within 1 ulp;
// below 2^8 an ulp is at most 2^-16, so when t is more than 2^-13 away from
// every half-integer both round to the same integer.  Otherwise (about one
// element in 10^4) the IEEE quotient decides.  Requires s normal and nonzero
// and rs = fl32(1/s) finite (the caller checks this once per vector).
//
// v is an element of the vector whose absmax defined s, so |v / s| <= 127
// up to rounding and no clamp is needed on the fast path (rint(t) <= 127 for
// t < 127.5); the exact path clamps as quant_code does.
__device__ __forceinline__ int quant_code_rcp(float v, float s, float rs)
{
    const float t = v * rs;
    const float r = __builtin_rintf(t);
    if (fabsf(t - r) <= 0.4998779296875f)  // more than 2^-13 away from a half-integer
        return (int)r;
    return quant_code(v, s);
}

// Whether quant_code_rcp may be used for scale s.
__device__ __forceinline__ bool rcp_quant_ok(float s)
{
    return s >= 1.0e-30f && s <= 1.0e30f;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d)
{
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// ---- FP8 codes (OCP E4M3: bias 7, no infinities, largest finite 448) with
// power-of-two scales ("探秘Transformer系列之（36）--- 大模型量化方案", the ZeroQuant-FP
// paragraph: FP8 activations, every scale a power of two). ----

// Exponent e of the smallest power of two with a <= 448 * 2^e, for a > 0;
// exact (fp64 comparisons of exact values).
__device__ __forceinline__ int fp8_scale_exp(float a)
{
    int e;
    frexp((double)a, &e);
    e -= 8;
    while (448.0 * ldexp(1.0, e) < (double)a)
        e++;
    while (448.0 * ldexp(1.0, e - 1) >= (double)a)
        e--;
    return e;
}

// Scale 2^e of a vector with absmax a (0 when a is 0 or 2^e is below the fp32 range).
__device__ __forceinline__ float fp8_scale(float a, int &e)
{
    if (!(a > 0.0f)) {
        e = 0;
        return 0.0f;
    }
    e = fp8_scale_exp(a);
    return (float)ldexp(1.0, e);
}

// Four E4M3 codes of y * 2^-e (|y * 2^-e| <= 448; exact scaling, then the
// hardware conversion: nearest, ties to even), little-endian in a word.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d, int e)
{
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(a, -e), ldexpf(b, -e), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(c, -e), ldexpf(d, -e), w, true);
    return (uint32_t)w;
}

// Wave-wide reductions without LDS: DPP within each 16-lane row (quad
// swaps, half-row and row mirrors), then the four row results are read into
// scalar registers and combined in a fixed order, so every lane gets the same
// bits.
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float rows_combine_sum(float v)
{
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float rows_combine_max(float v)
{
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<0xb1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4e>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    v += dpp<0x140>(v);  // row_mirror
    return rows_combine_sum(v);
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp<0xb1>(v));
    v = fmaxf(v, dpp<0x4e>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return rows_combine_max(v);
}

// Non-negative floats order like their bit patterns, so an unsigned atomic
// max on the bits is a float max that does not depend on arrival order.
__device__ __forceinline__ void atomic_max_nonneg(uint32_t *addr, float v)
{
    atomicMax(addr, __float_as_uint(v));
}


// ---- LDS DMA (global_load_lds_dwordx4) and its wait ----

// Each lane's 16 bytes at src go to LDS at lds_base + 16 * lane (lds_base is
// the same for the whole wave).  POLICY is the load's cache-policy operand
// (0: default, 2: non-temporal, for data read once).
template <int POLICY = 0>
__device__ __forceinline__ void dma16(const int8_t *src, int8_t *lds_base)
{
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)lds_base, 16, 0,
                                     POLICY);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their no-wait maxima).  The counter covers loads, LDS DMA and stores
// alike, in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS data written with ordinary ds_write: this wave's
// LDS operations complete (lgkmcnt(0)), then s_barrier.  Its global loads,
// stores and LDS DMA stay in flight (__syncthreads, and a release fence even
// when limited to LDS, wait for all of them, LDS DMA included).  The
// single-thread fences and the scheduling barrier keep the compiler from
// moving memory operations across it.
__device__ __forceinline__ void lds_barrier()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until this wave's LDS reads and writes have completed (lgkmcnt(0)).
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);
}

}  // namespace zq
