// Quantise new K/V rows into the int4 group-affine cache.
//
// The decode-step listing of the "turboquant-llama3.170B" README quantises K
// and V to int4 before the fused attention; "Background: Why TurboQuant Fails
// on Gemma 4" (Gemma page) fixes the format as int4 codes with a scale and a
// bias per group. The exact rule (directed fp16 rounding of bias and scale,
// fp32 round-to-nearest-even steps) is spelled out in include/kvq.h.
//
// Mapping: one lane per packed word. A group of G values is G/8 consecutive
// lanes of one wavefront; they reduce min/max with cross-lane swaps, every
// lane derives the same bias and scale, packs its eight codes into one word
// and stores it; the first lane of the group stores the fp16 scale and bias.
// Loads are 16-byte (fp16) or 2x16-byte (fp32) per lane and consecutive lanes
// touch consecutive addresses, so both loads and stores coalesce.
//
// Bit-exactness: no contraction (a*b+c stays two roundings), division is the
// correctly rounded IEEE one, rint is round-half-even, and the fp16
// conversions are the hardware round-to-nearest-even plus a one-ulp step.
#pragma clang fp contract(off)

#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __forceinline__ uint16_t h_bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }
__device__ __forceinline__ float h_val(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// largest fp16 <= x (x finite, |x| <= 65504)
__device__ __forceinline__ uint16_t f16_round_down(float x)
{
    uint16_t b = h_bits((_Float16)x);
    if (h_val(b) > x) {
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
    if (h_val(b) < x) {
        if ((b & 0x7fff) == 0)
            b = 0x0001;
        else
            b = (b & 0x8000) ? (uint16_t)(b - 1) : (uint16_t)(b + 1);
    }
    return b;
}

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

template <typename T, int LPG>  // LPG = lanes per group = G / 8
__global__ __launch_bounds__(256) void quantize_append_kernel(QuantizeArgs a)
{
    const int which = blockIdx.y;  // 0: K, 1: V
    const T *src = reinterpret_cast<const T *>(which ? a.v_new : a.k_new);
    uint32_t *dq = which ? a.v_q : a.k_q;
    uint16_t *dscale = which ? a.v_scale : a.k_scale;
    uint16_t *dbias = which ? a.v_bias : a.k_bias;

    const int W = a.D >> 3;  // words per row
    const int64_t lane_id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = a.rows * W;
    // Lanes past the end still take part in the swaps of their (partial)
    // group; groups never straddle the end because W is a multiple of LPG.
    const bool active = lane_id < total;
    const int64_t row = active ? lane_id / W : 0;
    const int w = active ? (int)(lane_id - row * W) : 0;

    float x[8];
    if (active) {
        load8<T>(src + row * a.D + 8 * w, x);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = 0.0f;
    }
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
    if (!active)
        return;

    uint16_t bb = f16_round_down(lo);
    if (bb == 0x8000)
        bb = 0;
    const float bf = h_val(bb);
    const float range = hi - bf;
    const float s32 = range / 15.0f;
    uint16_t sb = f16_round_up(s32);
    if (sb == 0x8000)
        sb = 0;
    const float sf = h_val(sb);

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
    const int64_t bh = row / a.n_new;
    const int64_t t = row - bh * a.n_new;
    const int64_t crow = bh * a.cap + a.len + t;
    dq[crow * W + w] = word;
    if ((w & (LPG - 1)) == 0) {
        const int NG = a.D / a.G;
        const int g = w / LPG;
        dscale[crow * NG + g] = sb;
        dbias[crow * NG + g] = bb;
    }
}

template <typename T>
hipError_t launch_t(const QuantizeArgs &a, hipStream_t s)
{
    const int64_t total = a.rows * (a.D / 8);
    const int64_t blocks = (total + 255) / 256;
    dim3 grid((unsigned)blocks, 2, 1);
    switch (a.G) {
    case 32:
        hipLaunchKernelGGL((quantize_append_kernel<T, 4>), grid, dim3(256), 0, s, a);
        break;
    case 64:
        hipLaunchKernelGGL((quantize_append_kernel<T, 8>), grid, dim3(256), 0, s, a);
        break;
    case 128:
        hipLaunchKernelGGL((quantize_append_kernel<T, 16>), grid, dim3(256), 0, s, a);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantizeArgs &a, int dtype, hipStream_t s)
{
    return dtype == KVQ_F16 ? launch_t<_Float16>(a, s) : launch_t<float>(a, s);
}

}  // namespace kvq
