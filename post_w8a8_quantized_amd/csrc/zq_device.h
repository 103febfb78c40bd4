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

// Exact (erf) GeLU in fp32: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)).
__device__ __forceinline__ float gelu_erf(float x)
{
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
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
