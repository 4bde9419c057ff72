// Normalised Hadamard rotation of cache-shaped rows on the GPU: the rotation
// of the blog on running Gemma 4 with TurboQuant (its "TurboQuant" section,
// the worked example and step "1. Vector Rotation"), y = H_D x / sqrt(D) with
// H_D in Sylvester order (entry (i, j) = (-1)^popcount(i & j)).
//
// Layout: a row of D = 8 W values is held by W consecutive lanes of one
// wavefront (W divides 64), lane w holding dimensions 8w .. 8w + 7, the same
// one-lane-per-packed-word mapping as the append kernel. The transform is the
// butterfly (a, b) -> (a + b, a - b) on every bit of the dimension index: the
// three low bits inside a lane, the others between lanes w and w ^ m.
//
// Arithmetic is float64. For fp16 rows every partial sum is a multiple of
// 2^-24 below 2^23 in magnitude, so the sums are exact in any order, and each
// result is one rounding of the exact product by c = 1 / sqrt(D) (computed on
// the host with correctly rounded sqrt and division) before the caller's
// conversion to fp32.
#pragma once

#include <hip/hip_runtime.h>

namespace kvq {

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
    for (int m = 1; m < W; m <<= 1) {  // W is uniform: every lane runs every shuffle
        const bool upper = (w & m) != 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const double y = __shfl_xor(x[j], m);
            x[j] = upper ? y - x[j] : x[j] + y;
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
        x[j] = x[j] * c;
}

}  // namespace kvq
