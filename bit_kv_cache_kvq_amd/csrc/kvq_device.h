// kvq_device.h -- device-side helpers shared by the libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t x = __float_as_uint(f);
    x += 0x7FFFu + ((x >> 16) & 1u);
    return x >> 16;
}

// fp32 -> fp16 bits with the hardware conversion (round to nearest even, subnormals kept).
__device__ __forceinline__ uint32_t f32_to_f16(float f)
{
    _Float16 h = (_Float16)f;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ __forceinline__ float lo_f16(uint32_t w) { return f16_to_f32(w & 0xFFFFu); }
__device__ __forceinline__ float hi_f16(uint32_t w) { return f16_to_f32(w >> 16); }

// two fp32 -> packed fp16 pair (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b)
{
    h2 v;
    v.x = (_Float16)a;
    v.y = (_Float16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// packed fp16 product of two pairs (round to nearest even per half)
__device__ __forceinline__ uint32_t mul_f16x2(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) * __builtin_bit_cast(h2, b));
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Bucket-relative RoPE (Dual-QK sec. 3.4 / C.4): rotate a head vector back by its bucket's
// anchor.  Lane l holds channels CPL*l .. CPL*l+CPL-1; channel i < D/2 pairs with i + D/2,
// which sits in lane l ^ 32.  cs = the bucket's (cos, sin) pairs [D/2][2].  With (c, s) of
// pair i: y_i <- y_i c + y_{i+D/2} s, y_{i+D/2} <- y_{i+D/2} c - y_i s, each product rounded
// before the sum (no contraction), as the format fixes.
// anchor_cs: this lane's (c, s) pairs of a bucket; anchor_apply: the rotation with them.
template <int CPL>
__device__ __forceinline__ void anchor_cs(float2 (&e)[CPL], const float *__restrict__ cs, int lane)
{
#pragma unroll
    for (int s = 0; s < CPL; s++)
        e[s] = *reinterpret_cast<const float2 *>(cs + 2 * ((lane & 31) * CPL + s));
}

template <int CPL>
__device__ __forceinline__ void anchor_apply(float (&y)[CPL], const float2 (&e)[CPL], int lane)
{
#pragma clang fp contract(off)
    const bool upper = lane >= 32;
#pragma unroll
    for (int s = 0; s < CPL; s++) {
        const float other = __shfl_xor(y[s], 32);
        const float a = y[s] * e[s].x;
        const float b = other * e[s].y;
        y[s] = upper ? a - b : a + b;
    }
}

template <int CPL>
__device__ __forceinline__ void anchor_rotate(float (&y)[CPL], const float *__restrict__ cs, int lane)
{
    float2 e[CPL];
    anchor_cs<CPL>(e, cs, lane);
    anchor_apply<CPL>(y, e, lane);
}

__device__ __forceinline__ float uniformf(float v)
{
    return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v)));
}

} // namespace kvq
