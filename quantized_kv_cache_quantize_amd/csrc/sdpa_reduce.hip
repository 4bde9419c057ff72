// Phase 2 of split-K decode attention: combine per-chunk partial softmax
// states into the output (split-K paragraph of the "turboquant-llama3.170B"
// README: a second phase reduces the partial softmax results and must run
// after the first; here both are launched on one stream, which orders them).
//
// With M = max_c m_c:  out[d] = sum_c e^{m_c-M} acc_c[d] / sum_c e^{m_c-M} l_c.
//
// Grid: (batch x query head, D / 32). A workgroup owns 32 output dimensions
// of one head; its 256 threads are 8 chunk lanes x 32 dimensions, so every
// chunk's 128-byte slice of the accumulator is one coalesced read and each
// thread keeps 8 independent loads in flight. The chunk lanes meet in LDS.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int RT = 256;
constexpr int DS = 32;         // dimensions per workgroup
constexpr int CL = RT / DS;    // chunk lanes
constexpr int UNROLL = 8;

__global__ __launch_bounds__(RT) void sdpa_reduce_kernel(ReduceArgs a)
{
    const int64_t head = blockIdx.x;
    const int d0 = blockIdx.y * DS;
    const int tid = threadIdx.x;
    const int cl = tid / DS;
    const int d = tid % DS;
    const int D = a.D;
    const int64_t C = a.C;
    const float *m = a.part_m + head * C;
    const float *l = a.part_l + head * C;
    const float *acc = a.part_acc + head * C * D + d0 + d;

    __shared__ float red[RT / 64];
    __shared__ float num_s[CL][DS];
    __shared__ float den_s[CL][DS];

    // M = max over chunks
    float mx = -INFINITY;
    for (int64_t c = tid; c < C; c += RT)
        mx = fmaxf(mx, m[c]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((tid & 63) == 0)
        red[tid >> 6] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int i = 1; i < RT / 64; ++i)
        M = fmaxf(M, red[i]);

    float num = 0.0f, den = 0.0f;
    int64_t c = cl;
    for (; c + (UNROLL - 1) * CL < C; c += UNROLL * CL) {
        float mv[UNROLL], lv[UNROLL], av[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            mv[u] = m[c + u * CL];
            lv[u] = l[c + u * CL];
            av[u] = acc[(c + u * CL) * D];
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const float f = exp2f((mv[u] - M) * kLog2e);
            den = fmaf(f, lv[u], den);
            num = fmaf(f, av[u], num);
        }
    }
    for (; c < C; c += CL) {
        const float f = exp2f((m[c] - M) * kLog2e);
        den = fmaf(f, l[c], den);
        num = fmaf(f, acc[c * D], num);
    }
    num_s[cl][d] = num;
    den_s[cl][d] = den;
    __syncthreads();
    if (cl == 0) {
#pragma unroll
        for (int g = 1; g < CL; ++g) {
            num += num_s[g][d];
            den += den_s[g][d];
        }
        a.out[head * D + d0 + d] = num / den;
    }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(sdpa_reduce_kernel, dim3((unsigned)a.heads, (unsigned)(a.D / DS)), dim3(RT), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
