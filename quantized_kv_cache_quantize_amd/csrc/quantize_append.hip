// Quantise new K/V rows into the group-affine cache (int4 codes, or int8).
//
// The decode-step listing of the "turboquant-llama3.170B" README quantises K
// and V to int4 before the fused attention; the rule itself is in
// quant_rule.h.
//
// Mapping: one lane per eight values of a row. A group of G values is G/8
// consecutive lanes of one wavefront; they reduce min/max with cross-lane
// swaps, every lane derives the same bias and scale, packs its eight codes
// (one word of nibbles, or two words of bytes) and stores them; the first
// lane of the group stores the fp16 scale and bias. Loads are 16-byte (fp16)
// or 2x16-byte (fp32) per lane and consecutive lanes touch consecutive
// addresses, so both loads and stores coalesce.
//
// The rotated variant (fp16 rows) first applies the normalised Hadamard
// rotation of hadamard_row.h to the row, whose D/8 lanes are consecutive in
// one wavefront, and quantises the fp32 rounding of the rotated values.
#include "hadamard_row.h"
#include "kvq_internal.h"
#include "quant_rule.h"

namespace kvq {
namespace {

template <typename T, int LPG, bool ROT, int BITS>  // LPG = lanes per group = G / 8
__global__ __launch_bounds__(256) void quantize_append_kernel(QuantizeArgs a)
{
    const int which = blockIdx.y;  // 0: K, 1: V
    const T *src = reinterpret_cast<const T *>(which ? a.v_new : a.k_new);
    uint32_t *dq = which ? a.v_q : a.k_q;
    uint16_t *dscale = which ? a.v_scale : a.k_scale;
    uint16_t *dbias = which ? a.v_bias : a.k_bias;

    const int W = a.D >> 3;            // lanes per row, a power of two
    const int lw = __builtin_ctz(W);   // (shifts, not 64-bit divisions)
    const int64_t lane_id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = a.rows * W;
    // Lanes past the end still take part in the swaps of their (partial)
    // group; groups never straddle the end because W is a multiple of LPG.
    const bool active = lane_id < total;
    const int64_t row = active ? lane_id >> lw : 0;
    const int w = (int)(lane_id & (W - 1));

    float x[8];
    if (active) {
        quant::load8<T>(src + row * a.D + 8 * w, x);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = 0.0f;
    }
    if constexpr (ROT) {
        // every lane of the row, past-the-end ones included, joins the shuffles
        double xd[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            xd[j] = (double)x[j];
        hadamard_row(xd, w, W, a.rot_scale);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = (float)xd[j];
    }
    // lanes past the end still take part in their group's swaps
    uint16_t sb, bb;
    uint32_t words[BITS / 4];
    quant::quantize_codes<LPG, BITS>(x, words, sb, bb);
    if (!active)
        return;
    // (batch * KV head, new row) of this row: a 32-bit division whenever the
    // row count fits (a 64-bit one costs several times as many instructions)
    int64_t bh, t;
    if (a.rows <= (int64_t)0xffffffff) {
        const uint32_t r = (uint32_t)row, n = (uint32_t)a.n_new, qt = r / n;
        bh = qt;
        t = r - qt * n;
    } else {
        bh = row / a.n_new;
        t = row - bh * a.n_new;
    }
    const int64_t crow = bh * a.cap + a.len + t;
    if constexpr (BITS == 4)
        dq[(crow << lw) + w] = words[0];
    else
        *reinterpret_cast<uint2 *>(dq + (crow << (lw + 1)) + 2 * w) = make_uint2(words[0], words[1]);
    if ((w & (LPG - 1)) == 0) {
        const int NG = W / LPG;
        const int g = w / LPG;
        dscale[crow * NG + g] = sb;
        dbias[crow * NG + g] = bb;
    }
}

template <typename T, bool ROT, int BITS>
hipError_t launch_tb(const QuantizeArgs &a, hipStream_t s)
{
    const int64_t total = a.rows * (a.D / 8);
    const int64_t blocks = (total + 255) / 256;
    dim3 grid((unsigned)blocks, 2, 1);
    switch (a.G) {
    case 32:
        hipLaunchKernelGGL((quantize_append_kernel<T, 4, ROT, BITS>), grid, dim3(256), 0, s, a);
        break;
    case 64:
        hipLaunchKernelGGL((quantize_append_kernel<T, 8, ROT, BITS>), grid, dim3(256), 0, s, a);
        break;
    case 128:
        hipLaunchKernelGGL((quantize_append_kernel<T, 16, ROT, BITS>), grid, dim3(256), 0, s, a);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, bool ROT>
hipError_t launch_t(const QuantizeArgs &a, hipStream_t s)
{
    if (a.bits == 8)
        return launch_tb<T, ROT, 8>(a, s);
    return a.bits == 4 ? launch_tb<T, ROT, 4>(a, s) : hipErrorInvalidValue;
}

// One lane per 8 values of a row: the rotation of hadamard_row.h in float64,
// rounded once to fp32. A row's lanes read all their values before any lane
// stores, so out may be x itself when x is fp32.
template <typename T>
__global__ __launch_bounds__(256) void hadamard_rotate_kernel(RotateArgs a)
{
    const int W = a.D >> 3;
    const int lw = __builtin_ctz(W);
    const int64_t lane_id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const bool active = lane_id < a.rows * W;
    const int64_t row = active ? lane_id >> lw : 0;
    const int w = (int)(lane_id & (W - 1));
    float x[8];
    if (active) {
        quant::load8<T>(reinterpret_cast<const T *>(a.x) + row * a.D + 8 * w, x);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = 0.0f;
    }
    double xd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        xd[j] = (double)x[j];
    hadamard_row(xd, w, W, a.scale);
    if (!active)
        return;
    float *o = a.out + row * a.D + 8 * w;
    *reinterpret_cast<float4 *>(o) = make_float4((float)xd[0], (float)xd[1], (float)xd[2], (float)xd[3]);
    *reinterpret_cast<float4 *>(o + 4) = make_float4((float)xd[4], (float)xd[5], (float)xd[6], (float)xd[7]);
}

}  // namespace

hipError_t launch_quantize(const QuantizeArgs &a, int dtype, hipStream_t s)
{
    if (a.rot_scale != 0.0)
        return dtype == KVQ_F16 ? launch_t<_Float16, true>(a, s) : hipErrorInvalidValue;
    return dtype == KVQ_F16 ? launch_t<_Float16, false>(a, s) : launch_t<float, false>(a, s);
}

hipError_t launch_rotate(const RotateArgs &a, int dtype, hipStream_t s)
{
    const int64_t blocks = (a.rows * (a.D / 8) + 255) / 256;
    if (dtype == KVQ_F16)
        hipLaunchKernelGGL((hadamard_rotate_kernel<_Float16>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((hadamard_rotate_kernel<float>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
