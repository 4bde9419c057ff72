// Normalised Hadamard rotation of cache-shaped rows on the GPU: the rotation
// of the blog on running Gemma 4 with TurboQuant (its "TurboQuant" section,
// the worked example and step "1. Vector Rotation"), y = H_D x / sqrt(D) with
// H_D in Sylvester order (entry (i, j) = (-1)^popcount(i & j)).
//
// Layout: a row of D = 8 W values is held by W consecutive lanes of one
// wavefront (W <= 32, rows aligned to W lanes), lane w holding
// dimensions 8w .. 8w + 7, the same one-lane-per-packed-word mapping as the
// append kernel. The transform is the butterfly (a, b) -> (a + b, a - b) on
// every bit of the dimension index: the three low bits inside a lane, the
// others between lanes w and w ^ m.
//
// Arithmetic is float64. For fp16 rows every partial sum is a multiple of
// 2^-24 below 2^23 in magnitude, so the sums are exact in any order, and each
// result is one rounding of the exact product by c = 1 / sqrt(D) (computed on
// the host with correctly rounded sqrt and division) before the caller's
// conversion to fp32.
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

// The value of lane l ^ M (M a power of two up to 16) without the LDS
// crossbar: inside a row of 16 lanes by DPP moves (M = 1, 2: quad
// permutations; 4: reverse the quad, then mirror the half-row, l -> l ^ 3 ->
// l ^ 7; 8: rotate the row by 8), between rows by the gfx950 swap of odd and
// even rows, whose two results with both operands equal hold a lane's own
// value and its partner's (the partner's in the second result for an even
// row).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

template <int M>
__device__ __forceinline__ uint32_t lane_xor_u(uint32_t v, int lane)
{
    if constexpr (M == 1) {
        return dpp_u<0xB1>(v);  // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        return dpp_u<0x4E>(v);  // quad_perm [2,3,0,1]
    } else if constexpr (M == 4) {
        return dpp_u<0x141>(dpp_u<0x1B>(v));  // quad_perm [3,2,1,0], then row_half_mirror
    } else if constexpr (M == 8) {
        return dpp_u<0x128>(v);  // row_ror:8
    } else {
        static_assert(M == 16, "lane distances 1 ... 16: rows of at most 32 lanes (D <= 256)");
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        // (elements go through scalars: a bit cast of a vector element in
        // place reads element 0)
        const uint32_t r0 = r[0], r1 = r[1];
        return (lane & 16) ? r0 : r1;
    }
}

template <int M>
__device__ __forceinline__ double lane_xor(double v, int lane)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = lane_xor_u<M>((uint32_t)u, lane), hi = lane_xor_u<M>((uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// One butterfly stage between lanes w and w ^ M of a row: the lower lane
// keeps x + y, the upper one y - x, computed as (-x) + y (the same IEEE
// result) with the sign flipped by an XOR
template <int M>
__device__ __forceinline__ void hadamard_stage(double (&x)[8], int w, int lane)
{
#pragma clang fp contract(off)
    const uint64_t sign = (w & M) ? 0x8000000000000000ull : 0ull;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const double y = lane_xor<M>(x[j], lane);
        x[j] = __builtin_bit_cast(double, __builtin_bit_cast(uint64_t, x[j]) ^ sign) + y;
    }
}

__device__ __forceinline__ void hadamard_row(double (&x)[8], int w, int W, double c)
{
#pragma clang fp contract(off)
#pragma unroll
    for (int s = 1; s < 8; s <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (!(j & s)) {
                const double a = x[j], b = x[j | s];
                x[j] = a + b;
                x[j | s] = a - b;
            }
    // W is uniform: every lane of the wavefront runs every stage
    const int lane = (int)(threadIdx.x & 63);
    if (W > 1)
        hadamard_stage<1>(x, w, lane);
    if (W > 2)
        hadamard_stage<2>(x, w, lane);
    if (W > 4)
        hadamard_stage<4>(x, w, lane);
    if (W > 8)
        hadamard_stage<8>(x, w, lane);
    if (W > 16)
        hadamard_stage<16>(x, w, lane);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        x[j] = x[j] * c;
}

}  // namespace kvq
