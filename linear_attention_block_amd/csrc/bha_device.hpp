// Device helpers shared by the libbha.so kernels.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace bha {

// Element loads as float: float32 as is, bfloat16 from its 16 bits (exact).
__device__ __forceinline__ float ld_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_elem(const uint16_t* p, int64_t i)
{
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// Element stores from float: bfloat16 rounds to nearest even in hardware.
__device__ __forceinline__ void st_elem(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st_elem(uint16_t* p, int64_t i, float x)
{
    p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ uint16_t bf16_bits(float x)
{
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Offset (in floats) of S[f][c] inside one state record whose S part is stored
// in 32 x 4 tiles: tile (c/32, f/4) holds 32 columns x 4 features, the four
// features of a column contiguous.
__device__ __forceinline__ int64_t s_offset(int f, int c, int F)
{
    return (static_cast<int64_t>(c >> 5) * (F >> 2) + (f >> 2)) * 128 + (c & 31) * 4 + (f & 3);
}

// Merge weights of the two branches. The value
//   (num_sm + g e^{-m} num_lin) / (l + g e^{-m} den_lin)
// is evaluated as (al num_sm + be num_lin) / (al l + be den_lin) with
// (al, be) = (1, g e^{-m}) when g e^{-m} <= 1 and (e^{m}/g, 1) otherwise, the
// same quotient with numerator and denominator scaled by one positive number,
// so that e^{-m} never overflows. g == 0 gives (1, 0); g < 0 or NaN gives NaN.
__device__ __forceinline__ void merge_weights(float gamma, float m, float& al, float& be)
{
    if (!(gamma >= 0.0f)) {
        al = __builtin_nanf("");
        be = al;
    } else if (gamma == 0.0f) {
        al = 1.0f;
        be = 0.0f;
    } else {
        const float e = logf(gamma) - m;
        if (e <= 0.0f) {
            al = 1.0f;
            be = expf(e);
        } else {
            al = expf(-e);
            be = 1.0f;
        }
    }
}

__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

}  // namespace bha
