// The group-affine quantiser of eight values of a row, for any kernel that
// writes cache rows (the append kernel and the fused decode step).
//
// "Background: Why TurboQuant Fails on Gemma 4" (Gemma page) fixes the
// format: int4 codes with an fp16 scale and bias per group; the exact rule
// (bias = min rounded down to fp16, scale = (max - bias)/L rounded up to
// fp16, codes rint((x - bias)/scale) clamped to [0, L], 0 when scale is 0,
// -0 stored as +0; L = 15 for int4 codes, 255 for the 8-bit cache of the
// Gemma page's "What I Tried" table) is spelled out in include/kvq.h.
//
// Bit-exactness: no contraction (a*b+c stays two roundings), every quotient
// that can change a code is the correctly rounded IEEE one (see
// quantize_codes), rint is round-half-even, and the fp16 conversions are the
// hardware round-to-nearest-even plus a one-ulp step.
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

// Eight consecutive values of a row (element j -> code j of the lane's
// word, or of its two words for 8-bit codes).
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

// One DPP exchange inside rows of 16 lanes (a bound-checked source lane is
// always a lane of the same row for the controls used here).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Minimum and maximum over the LPG aligned lanes of a group (LPG in {4, 8,
// 16}): quad exchanges (lane ^ 1, lane ^ 2), then the mirror inside 8 lanes
// and inside 16 lanes, each pairing lanes of different halves. The
// NaN-propagating minimum/maximum need no canonical operands (inputs are
// finite; a zero's sign is dropped later with the bias and scale).
template <int LPG>
__device__ __forceinline__ void group_min_max(float &lo, float &hi)
{
    lo = __builtin_elementwise_minimum(lo, dpp_f<0xB1>(lo));  // quad_perm [1,0,3,2]
    hi = __builtin_elementwise_maximum(hi, dpp_f<0xB1>(hi));
    lo = __builtin_elementwise_minimum(lo, dpp_f<0x4E>(lo));  // quad_perm [2,3,0,1]
    hi = __builtin_elementwise_maximum(hi, dpp_f<0x4E>(hi));
    if constexpr (LPG >= 8) {
        lo = __builtin_elementwise_minimum(lo, dpp_f<0x141>(lo));  // row_half_mirror
        hi = __builtin_elementwise_maximum(hi, dpp_f<0x141>(hi));
    }
    if constexpr (LPG >= 16) {
        lo = __builtin_elementwise_minimum(lo, dpp_f<0x140>(lo));  // row_mirror
        hi = __builtin_elementwise_maximum(hi, dpp_f<0x140>(hi));
    }
}

// Quantise eight values of a group whose G values are held by LPG = G/8
// consecutive, aligned lanes (every lane of the group must call this
// together: the group's min and max meet through lane exchanges). Stores the
// packed codes, BITS/4 words (int4: one word of eight nibbles; int8: two
// words of four bytes, lowest first), and returns the group's fp16 scale and
// bias bit patterns (the same on every lane).
template <int LPG, int BITS>
__device__ __forceinline__ void quantize_codes(const float (&x)[8], uint32_t (&words)[BITS / 4], uint16_t &scale_bits,
                                               uint16_t &bias_bits)
{
#pragma clang fp contract(off)
    static_assert(LPG == 4 || LPG == 8 || LPG == 16, "groups of 32, 64 or 128 values");
    static_assert(BITS == 4 || BITS == 8, "int4 or int8 codes");
    constexpr float L = (float)((1 << BITS) - 1);
    float lo = x[0], hi = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
        lo = __builtin_elementwise_minimum(lo, x[j]);
        hi = __builtin_elementwise_maximum(hi, x[j]);
    }
    group_min_max<LPG>(lo, hi);
    uint16_t bb = f16_round_down(lo);
    if (bb == 0x8000)
        bb = 0;
    const float bf = h_value(bb);
    const float range = hi - bf;
    const float s32 = range / L;
    uint16_t sb = f16_round_up(s32);
    if (sb == 0x8000)
        sb = 0;
    const float sf = h_value(sb);

    // The code is rint of the correctly rounded quotient u = (x - bias) /
    // scale, which lies in [0, L + 1). The product (x - bias) * rcp(scale)
    // (v_rcp_f32, 1 ulp) is within (L + 1) * 1.5 * 2^-23 of the exact
    // quotient and u within (L + 1) * 2^-24 of it, so both round to the same
    // integer unless the product lies within (L + 1) * 2^-22 of a
    // half-integer (3.8e-6 for int4, 6.1e-5 for int8). When some lane of the
    // wavefront has a product closer than the margin (twice that or more:
    // 2^-16 for int4, 2^-13 for int8), the wavefront recomputes its codes
    // from correctly rounded quotients.
    constexpr float margin = BITS == 4 ? 0x1p-16f : 0x1p-13f;
    float r[8];
    const float rs = sf != 0.0f ? __builtin_amdgcn_rcpf(sf) : 0.0f;
    bool near = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float u = (x[j] - bf) * rs;
        r[j] = rintf(u);
        near |= fabsf(u - r[j]) > 0.5f - margin;
    }
    if (__builtin_amdgcn_ballot_w64(near) != 0) {
        asm volatile("" ::: "memory");  // a real branch: the divisions run only here
#pragma unroll
        for (int j = 0; j < 8; ++j)
            r[j] = sf != 0.0f ? rintf((x[j] - bf) / sf) : 0.0f;
    }
    constexpr int P = 32 / BITS;  // codes per word
#pragma unroll
    for (int i = 0; i < BITS / 4; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < P; ++j)
            word |= (uint32_t)__builtin_amdgcn_fmed3f(r[P * i + j], 0.0f, L) << (BITS * j);
        words[i] = word;
    }
    scale_bits = sb;
    bias_bits = bb;
}

// The int4 word of eight values (see quantize_codes).
template <int LPG>
__device__ __forceinline__ uint32_t quantize_word(const float (&x)[8], uint16_t &scale_bits, uint16_t &bias_bits)
{
    uint32_t w[1];
    quantize_codes<LPG, 4>(x, w, scale_bits, bias_bits);
    return w[0];
}

}  // namespace quant
}  // namespace kvq
