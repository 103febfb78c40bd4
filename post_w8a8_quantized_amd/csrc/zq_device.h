// Device helpers shared by the gfx950 kernels of libzq (not by anything else).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace zq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

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

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d)
{
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Non-negative floats order like their bit patterns, so an unsigned atomic
// max on the bits is a float max that does not depend on arrival order.
__device__ __forceinline__ void atomic_max_nonneg(uint32_t *addr, float v)
{
    atomicMax(addr, __float_as_uint(v));
}

}  // namespace zq
