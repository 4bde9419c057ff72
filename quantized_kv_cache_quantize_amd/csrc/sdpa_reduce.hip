// Phase 2 of split-K decode attention: combine per-chunk partial softmax
// states into the output (split-K paragraph of the "turboquant-llama3.170B"
// README: a second phase reduces the partial softmax results and must run
// after the first; here both are launched on one stream, which orders them).
//
// With M = max_c m_c:  out[d] = sum_c e^{m_c-M} acc_c[d] / sum_c e^{m_c-M} l_c.
//
// One workgroup of 256 threads per (batch, query head). The threads split
// into 256/D lanes-groups that take every (256/D)-th chunk; each thread owns
// one dimension, so every chunk's accumulator row is read with coalesced
// 4-byte loads. The per-group sums meet in LDS.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int RT = 256;

__global__ __launch_bounds__(RT) void sdpa_reduce_kernel(ReduceArgs a)
{
    const int64_t head = blockIdx.x;
    const int tid = threadIdx.x;
    const int D = a.D;
    const int ngrp = RT / D;
    const int grp = tid / D;
    const int d = tid % D;
    const float *m = a.part_m + head * a.C;
    const float *l = a.part_l + head * a.C;
    const float *acc = a.part_acc + head * a.C * D;

    __shared__ float red[RT / 64];
    __shared__ float num_s[RT];
    __shared__ float den_s[RT];

    // M = max over chunks
    float mx = -INFINITY;
    for (int64_t c = tid; c < a.C; c += RT)
        mx = fmaxf(mx, m[c]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((tid & 63) == 0)
        red[tid >> 6] = mx;
    __syncthreads();
    float M = red[0];
    for (int i = 1; i < RT / 64; ++i)
        M = fmaxf(M, red[i]);

    float num = 0.0f, den = 0.0f;
    for (int64_t c = grp; c < a.C; c += ngrp) {
        const float f = exp2f((m[c] - M) * kLog2e);
        den = fmaf(f, l[c], den);
        num = fmaf(f, acc[c * D + d], num);
    }
    num_s[tid] = num;
    den_s[tid] = den;
    __syncthreads();
    if (grp == 0) {
        for (int g = 1; g < ngrp; ++g) {
            num += num_s[g * D + d];
            den += den_s[g * D + d];
        }
        a.out[head * D + d] = num / den;
    }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(sdpa_reduce_kernel, dim3((unsigned)a.heads), dim3(RT), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
