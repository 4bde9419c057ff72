// The int4 group-affine quantiser of one packed word, for any kernel that
// writes cache rows (the append kernel and the fused decode step).
//
// "Background: Why TurboQuant Fails on Gemma 4" (Gemma page) fixes the
// format: int4 codes with an fp16 scale and bias per group; the exact rule
// (bias = min rounded down to fp16, scale = (max - bias)/15 rounded up to
// fp16, codes rint((x - bias)/scale) clamped to [0, 15], 0 when scale is 0,
// -0 stored as +0) is spelled out in include/kvq.h.
//
// Bit-exactness: no contraction (a*b+c stays two roundings), division is the
// correctly rounded IEEE one, rint is round-half-even, and the fp16
// conversions are the hardware round-to-nearest-even plus a one-ulp step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {
namespace quant {

__device__ __forceinline__ uint16_t h_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }
__device__ __forceinline__ float h_value(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// largest fp16 <= x (x finite, |x| <= 65504)
__device__ __forceinline__ uint16_t f16_round_down(float x)
{
    uint16_t b = h_bits((_Float16)x);
    if (h_value(b) > x) {
        if ((b & 0x7fff) == 0)
            b = 0x8001;
        else
            b = (b & 0x8000) ? (uint16_t)(b + 1) : (uint16_t)(b - 1);
    }
    return b;
}

// smallest fp16 >= x (x finite, 0 <= x <= 65504)
__device__ __forceinline__ uint16_t f16_round_up(float x)
{
    uint16_t b = h_bits((_Float16)x);
    if (h_value(b) < x) {
        if ((b & 0x7fff) == 0)
            b = 0x0001;
        else
            b = (b & 0x8000) ? (uint16_t)(b - 1) : (uint16_t)(b + 1);
    }
    return b;
}

// Eight consecutive values of a row (element j -> nibble j of the word).
template <typename T>
__device__ __forceinline__ void load8(const T *p, float (&x)[8]);

template <>
__device__ __forceinline__ void load8<_Float16>(const _Float16 *p, float (&x)[8])
{
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    h8 v = *reinterpret_cast<const h8 *>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        x[j] = (float)v[j];
}

template <>
__device__ __forceinline__ void load8<float>(const float *p, float (&x)[8])
{
    float4 a = reinterpret_cast<const float4 *>(p)[0];
    float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Quantise one word of a group whose G values are held by LPG = G/8
// consecutive lanes (every lane of the group must call this together: the
// group's min and max meet through lane swaps). Returns the packed codes and
// the group's fp16 scale and bias bit patterns (the same on every lane).
template <int LPG>
__device__ __forceinline__ uint32_t quantize_word(const float (&x)[8], uint16_t &scale_bits, uint16_t &bias_bits)
{
#pragma clang fp contract(off)
    float lo = x[0], hi = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        lo = fminf(lo, x[j]);
        hi = fmaxf(hi, x[j]);
    }
#pragma unroll
    for (int off = 1; off < LPG; off <<= 1) {
        lo = fminf(lo, __shfl_xor(lo, off));
        hi = fmaxf(hi, __shfl_xor(hi, off));
    }
    uint16_t bb = f16_round_down(lo);
    if (bb == 0x8000)
        bb = 0;
    const float bf = h_value(bb);
    const float range = hi - bf;
    const float s32 = range / 15.0f;
    uint16_t sb = f16_round_up(s32);
    if (sb == 0x8000)
        sb = 0;
    const float sf = h_value(sb);

    uint32_t word = 0;
    if (sf != 0.0f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float diff = x[j] - bf;
            const float u = diff / sf;
            float r = rintf(u);
            r = fminf(fmaxf(r, 0.0f), 15.0f);
            word |= (uint32_t)r << (4 * j);
        }
    }
    scale_bits = sb;
    bias_bits = bb;
    return word;
}

}  // namespace quant
}  // namespace kvq
