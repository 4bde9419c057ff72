// Phase 2 of split-K decode attention: combine per-chunk partial softmax
// states into the output (split-K paragraph of the "turboquant-llama3.170B"
// README: a second phase merges the per-chunk softmax states and has to run
// after the first; here both are launched on one stream, which orders them).
//
// With M = max_c m_c:  out[d] = sum_c e^{m_c-M} acc_c[d] / sum_c e^{m_c-M} l_c.
//
// Grid: (batch x query head, D / 32). A workgroup owns 32 output dimensions of
// one head; its 256 threads are 32 chunk lanes x 8 groups of 4 dimensions.
// A thread takes every 32nd chunk, reading its (m, l) and a 16-byte slice of
// its accumulator; all of a thread's loads are issued before the first use
// (one memory round trip up to 256 chunks) and combined with a running
// maximum; the 32 chunk lanes then meet in a butterfly and one LDS step.
//
// Rotated variant (the output of a Hadamard-rotated cache): a workgroup owns
// a whole head, so that after the merge the D outputs can be rotated back,
// y = H_D o / sqrt(D) (fp32 butterflies: two index bits inside a lane, the
// others between lanes), before they are stored.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int RT = 256;
constexpr int DS = 32;          // dimensions per workgroup
constexpr int DQ = DS / 4;      // float4 groups per workgroup
constexpr int CL = RT / DQ;     // chunk lanes (32)
constexpr int UNROLL = 8;       // chunks per thread per round

__global__ __launch_bounds__(RT) void sdpa_reduce_kernel(ReduceArgs a)
{
    const int64_t head = blockIdx.x;
    const int d0 = blockIdx.y * DS;
    const int tid = threadIdx.x;
    const int cl = tid / DQ;
    const int dq = tid % DQ;
    const int D = a.D;
    const int64_t C = a.C;
    const float *m = a.part_m + head * C;
    const float *l = a.part_l + head * C;
    const float *acc = a.part_acc + head * C * D + d0 + 4 * dq;

    // running state of this thread's chunks (natural-log maxima)
    float M = -INFINITY, den = 0.0f;
    float4 num = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t c0 = cl; c0 < C; c0 += UNROLL * CL) {
        float mv[UNROLL], lv[UNROLL];
        float4 av[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t c = c0 + u * CL;
            const bool in = c < C;
            mv[u] = in ? m[c] : -INFINITY;
            lv[u] = in ? l[c] : 0.0f;
            av[u] = in ? *reinterpret_cast<const float4 *>(acc + c * D) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            Mn = fmaxf(Mn, mv[u]);
        if (Mn != -INFINITY) {
            const float r = exp2f((M - Mn) * kLog2e);  // 0 while M is -inf
            den *= r;
            num.x *= r; num.y *= r; num.z *= r; num.w *= r;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const float f = exp2f((mv[u] - Mn) * kLog2e);
                den = fmaf(f, lv[u], den);
                num.x = fmaf(f, av[u].x, num.x);
                num.y = fmaf(f, av[u].y, num.y);
                num.z = fmaf(f, av[u].z, num.z);
                num.w = fmaf(f, av[u].w, num.w);
            }
            M = Mn;
        }
    }

    // combine the chunk lanes: a butterfly over the 8 lanes of a wavefront
    // that share dq (lane offsets 8, 16, 32), then the 4 wavefronts in LDS
    auto merge = [](float &Ma, float &da, float4 &na, float Mb, float db, float4 nb) {
        const float Mn = fmaxf(Ma, Mb);
        if (Mn == -INFINITY)
            return;  // neither side has chunks
        const float fa = exp2f((Ma - Mn) * kLog2e), fb = exp2f((Mb - Mn) * kLog2e);
        da = fmaf(da, fa, db * fb);
        na.x = fmaf(na.x, fa, nb.x * fb);
        na.y = fmaf(na.y, fa, nb.y * fb);
        na.z = fmaf(na.z, fa, nb.z * fb);
        na.w = fmaf(na.w, fa, nb.w * fb);
        Ma = Mn;
    };
#pragma unroll
    for (int off = DQ; off < 64; off <<= 1) {
        const float Mb = __shfl_xor(M, off), db = __shfl_xor(den, off);
        const float4 nb = make_float4(__shfl_xor(num.x, off), __shfl_xor(num.y, off), __shfl_xor(num.z, off),
                                      __shfl_xor(num.w, off));
        merge(M, den, num, Mb, db, nb);
    }
    constexpr int NW = RT / 64;
    __shared__ float m_s[NW][DQ];
    __shared__ float den_s[NW][DQ];
    __shared__ float4 num_s[NW][DQ];
    const int w = tid >> 6;
    if ((tid & 63) < DQ) {
        m_s[w][dq] = M;
        den_s[w][dq] = den;
        num_s[w][dq] = num;
    }
    __syncthreads();
    if (tid < DQ) {
#pragma unroll
        for (int g = 1; g < NW; ++g)
            merge(M, den, num, m_s[g][dq], den_s[g][dq], num_s[g][dq]);
        *reinterpret_cast<float4 *>(a.out + head * D + d0 + 4 * dq) =
            make_float4(num.x / den, num.y / den, num.z / den, num.w / den);
    }
}

// One head per workgroup: 256 threads = (256 / (D/4)) chunk lanes x D/4
// groups of 4 dimensions (D in {64, 128, 256}). (1024 threads measured
// slower: the last wavefront then merges 16 states in series.)
constexpr int RTH = 256;

template <int D>
__global__ __launch_bounds__(RTH) void sdpa_reduce_rot_kernel(ReduceArgs a)
{
#pragma clang fp contract(off)
    constexpr int DQH = D / 4;      // float4 groups of the head (<= 64: one wavefront holds them)
    constexpr int CLH = RTH / DQH;  // chunk lanes
    const int64_t head = blockIdx.x;
    const int tid = threadIdx.x;
    const int cl = tid / DQH;
    const int dq = tid % DQH;
    const int64_t C = a.C;
    const float *m = a.part_m + head * C;
    const float *l = a.part_l + head * C;
    const float *acc = a.part_acc + head * C * D + 4 * dq;

    float M = -INFINITY, den = 0.0f;
    float4 num = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t c0 = cl; c0 < C; c0 += UNROLL * CLH) {
        float mv[UNROLL], lv[UNROLL];
        float4 av[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t c = c0 + u * CLH;
            const bool in = c < C;
            mv[u] = in ? m[c] : -INFINITY;
            lv[u] = in ? l[c] : 0.0f;
            av[u] = in ? *reinterpret_cast<const float4 *>(acc + c * D) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        float Mn = M;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            Mn = fmaxf(Mn, mv[u]);
        if (Mn != -INFINITY) {
            const float r = exp2f((M - Mn) * kLog2e);
            den *= r;
            num.x *= r; num.y *= r; num.z *= r; num.w *= r;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const float f = exp2f((mv[u] - Mn) * kLog2e);
                den = fmaf(f, lv[u], den);
                num.x = fmaf(f, av[u].x, num.x);
                num.y = fmaf(f, av[u].y, num.y);
                num.z = fmaf(f, av[u].z, num.z);
                num.w = fmaf(f, av[u].w, num.w);
            }
            M = Mn;
        }
    }
    auto merge = [](float &Ma, float &da, float4 &na, float Mb, float db, float4 nb) {
        const float Mn = fmaxf(Ma, Mb);
        if (Mn == -INFINITY)
            return;
        const float fa = exp2f((Ma - Mn) * kLog2e), fb = exp2f((Mb - Mn) * kLog2e);
        da = fmaf(da, fa, db * fb);
        na.x = fmaf(na.x, fa, nb.x * fb);
        na.y = fmaf(na.y, fa, nb.y * fb);
        na.z = fmaf(na.z, fa, nb.z * fb);
        na.w = fmaf(na.w, fa, nb.w * fb);
        Ma = Mn;
    };
#pragma unroll
    for (int off = DQH; off < 64; off <<= 1) {
        const float Mb = __shfl_xor(M, off), db = __shfl_xor(den, off);
        const float4 nb = make_float4(__shfl_xor(num.x, off), __shfl_xor(num.y, off), __shfl_xor(num.z, off),
                                      __shfl_xor(num.w, off));
        merge(M, den, num, Mb, db, nb);
    }
    constexpr int NWH = RTH / 64;
    __shared__ float m_s[NWH][DQH];
    __shared__ float den_s[NWH][DQH];
    __shared__ float4 num_s[NWH][DQH];
    const int w = tid >> 6;
    if ((tid & 63) < DQH) {
        m_s[w][dq] = M;
        den_s[w][dq] = den;
        num_s[w][dq] = num;
    }
    __syncthreads();
    if (tid < 64) {  // the first wavefront: lanes dq < DQH hold the head
#pragma unroll
        for (int g = 1; g < NWH; ++g)
            if (tid < DQH)
                merge(M, den, num, m_s[g][dq], den_s[g][dq], num_s[g][dq]);
        // o in fp32 as the plain reduce stores it, then rotated in fp32
        // (log2 D butterfly stages: a relative error of a few 2^-24)
        float x[4] = {num.x / den, num.y / den, num.z / den, num.w / den};
        {
            const float p0 = x[0] + x[1], p1 = x[0] - x[1], p2 = x[2] + x[3], p3 = x[2] - x[3];
            x[0] = p0 + p2; x[2] = p0 - p2; x[1] = p1 + p3; x[3] = p1 - p3;
        }
#pragma unroll
        for (int mb = 1; mb < DQH; mb <<= 1) {  // dimension bits 2 and up: lanes dq ^ mb
            const float sign = (dq & mb) ? -1.0f : 1.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                x[j] = fmaf(sign, x[j], __shfl_xor(x[j], mb));
        }
        const float rs = (float)a.rot_scale;
        if (tid < DQH)
            *reinterpret_cast<float4 *>(a.out + head * D + 4 * dq) = make_float4(x[0] * rs, x[1] * rs, x[2] * rs,
                                                                                x[3] * rs);
    }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s)
{
    if (a.rot_scale != 0.0) {
        switch (a.D) {
        case 64:
            hipLaunchKernelGGL((sdpa_reduce_rot_kernel<64>), dim3((unsigned)a.heads), dim3(RTH), 0, s, a);
            break;
        case 128:
            hipLaunchKernelGGL((sdpa_reduce_rot_kernel<128>), dim3((unsigned)a.heads), dim3(RTH), 0, s, a);
            break;
        case 256:
            hipLaunchKernelGGL((sdpa_reduce_rot_kernel<256>), dim3((unsigned)a.heads), dim3(RTH), 0, s, a);
            break;
        default:
            return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    hipLaunchKernelGGL(sdpa_reduce_kernel, dim3((unsigned)a.heads, (unsigned)(a.D / DS)), dim3(RT), 0, s, a);
    return hipGetLastError();
}

}  // namespace kvq
