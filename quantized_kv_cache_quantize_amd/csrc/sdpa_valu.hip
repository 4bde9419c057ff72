// Split-K decode attention on the quantised cache (int4 codes, or the 8-bit
// variant), vector-ALU kernel.
//
// Phase 1 of the split-K scheme of the "turboquant-llama3.170B" README: each
// workgroup owns one (batch, KV head, head tile, chunk) and emits the partial
// softmax state (m, l, acc) of every query head of its tile for that chunk.
// K and V codes are dequantised in registers (code * scale + bias, the
// per-group affine format of the Gemma page's "Background" section); scores,
// weights and the running softmax live in registers and LDS only.
//
// This variant handles every supported shape (any GQA ratio, D in
// {64,128,256}, G in {32,64,128}, any chunk length, 4- or 8-bit codes) and
// is the fallback for what the matrix-core kernels do not cover. Within a
// chunk the rows are walked in tiles of 256 with an online softmax across
// tiles.
//
// Layout per tile (256 threads, 4 wavefronts):
//   K pass: thread i scores row tile+i for all NREP heads (q broadcast from LDS).
//   V pass: thread (word w, slot r) accumulates words w of rows r, r+NT/W, ...
//           so each wavefront load instruction reads whole 32..256-byte rows.
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ float h_val(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

template <typename QT>
__device__ __forceinline__ float q_load(const QT *p, int i);
template <>
__device__ __forceinline__ float q_load<_Float16>(const _Float16 *p, int i) { return (float)p[i]; }
template <>
__device__ __forceinline__ float q_load<float>(const float *p, int i) { return p[i]; }

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off);
    return v;
}

template <int D, int NREP, typename QT, int BITS>
__global__ __launch_bounds__(NT) void sdpa_partial_valu_kernel(PartialArgs a)
{
    constexpr int P = 32 / BITS;  // codes per word
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    constexpr int W = D / P;      // words per row
    constexpr int NS = NT / W;    // V-pass row slots
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int c = blockIdx.x;
    const int tiles_per_kv = a.n_rep / NREP;
    const int kvh = blockIdx.y / tiles_per_kv;
    const int h0 = kvh * a.n_rep + (blockIdx.y % tiles_per_kv) * NREP;  // first query head
    const int b = blockIdx.z;
    const int G = a.G;
    const int NG = D / G;

    const int64_t t0 = (int64_t)c * a.chunk;
    const int64_t t1 = min(t0 + (int64_t)a.chunk, a.skv);
    const int64_t kvrow0 = ((int64_t)b * a.Hkv + kvh) * a.cap;

    __shared__ __align__(16) float q_s[NREP][D];
    __shared__ float p_s[NREP][NT];
    __shared__ float red_s[NREP][4];
    __shared__ __align__(16) float acc_s[4][NREP][D];

    const QT *qp = reinterpret_cast<const QT *>(a.q) + ((int64_t)b * a.Hq + h0) * D;
    for (int i = tid; i < NREP * D; i += NT)
        q_s[i / D][i % D] = q_load<QT>(qp, i);
    __syncthreads();

    const int w = tid % W;
    const int slot = tid / W;
    const int gw = (P * w) / G;  // group of this thread's V word

    float acc[NREP][P];
    float m_run[NREP], l_part[NREP];
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
        m_run[h] = -INFINITY;
        l_part[h] = 0.0f;
#pragma unroll
        for (int j = 0; j < P; ++j)
            acc[h][j] = 0.0f;
    }

    for (int64_t tb = t0; tb < t1; tb += NT) {
        // ---- K pass: one row per thread, scores for all heads of the tile
        const int64_t t = tb + tid;
        float s[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h)
            s[h] = 0.0f;
        if (t < t1) {
            const uint32_t *kr = a.k_q + (kvrow0 + t) * W;
            const uint16_t *ksr = a.k_scale + (kvrow0 + t) * NG;
            const uint16_t *kbr = a.k_bias + (kvrow0 + t) * NG;
#pragma unroll 4
            for (int w4 = 0; w4 < W; w4 += 4) {
                const uint4 words = *reinterpret_cast<const uint4 *>(kr + w4);
                const uint32_t wv[4] = {words.x, words.y, words.z, words.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int g = (P * (w4 + u)) / G;
                    const float sc = h_val(ksr[g]);
                    const float bi = h_val(kbr[g]);
                    float kv[P];
#pragma unroll
                    for (int j = 0; j < P; ++j)
                        kv[j] = fmaf((float)((wv[u] >> (BITS * j)) & MASK), sc, bi);
#pragma unroll
                    for (int h = 0; h < NREP; ++h) {
                        float acc_s0 = s[h];
#pragma unroll
                        for (int j4 = 0; j4 < P; j4 += 4) {
                            const float4 qa = *reinterpret_cast<const float4 *>(&q_s[h][P * (w4 + u) + j4]);
                            acc_s0 = fmaf(qa.x, kv[j4 + 0], acc_s0);
                            acc_s0 = fmaf(qa.y, kv[j4 + 1], acc_s0);
                            acc_s0 = fmaf(qa.z, kv[j4 + 2], acc_s0);
                            acc_s0 = fmaf(qa.w, kv[j4 + 3], acc_s0);
                        }
                        s[h] = acc_s0;
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < NREP; ++h)
                s[h] *= a.score_scale;
        } else {
#pragma unroll
            for (int h = 0; h < NREP; ++h)
                s[h] = -INFINITY;
        }

        // ---- tile max per head
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
            const float mx = wave_max(s[h]);
            if (lane == 0)
                red_s[h][wave] = mx;
        }
        __syncthreads();
        float corr[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
            const float tmax = fmaxf(fmaxf(red_s[h][0], red_s[h][1]), fmaxf(red_s[h][2], red_s[h][3]));
            const float m_new = fmaxf(m_run[h], tmax);  // finite: the tile holds >= 1 row
            corr[h] = exp2f(m_run[h] - m_new);          // 0 on the first tile
            m_run[h] = m_new;
            const float p = (t < t1) ? exp2f(s[h] - m_new) : 0.0f;
            p_s[h][tid] = p;
            l_part[h] = l_part[h] * corr[h] + p;
        }
        __syncthreads();

        // ---- V pass
#pragma unroll
        for (int h = 0; h < NREP; ++h)
#pragma unroll
            for (int j = 0; j < P; ++j)
                acc[h][j] *= corr[h];
        const int nrows = (int)min((int64_t)NT, t1 - tb);
        for (int r = slot; r < nrows; r += NS) {
            const int64_t vrow = kvrow0 + tb + r;
            const uint32_t word = a.v_q[vrow * W + w];
            const float sc = h_val(a.v_scale[vrow * NG + gw]);
            const float bi = h_val(a.v_bias[vrow * NG + gw]);
            float vv[P];
#pragma unroll
            for (int j = 0; j < P; ++j)
                vv[j] = fmaf((float)((word >> (BITS * j)) & MASK), sc, bi);
#pragma unroll
            for (int h = 0; h < NREP; ++h) {
                const float p = p_s[h][r];
#pragma unroll
                for (int j = 0; j < P; ++j)
                    acc[h][j] = fmaf(p, vv[j], acc[h][j]);
            }
        }
        __syncthreads();  // p_s and red_s are rewritten by the next tile
    }

    // ---- combine the V-pass slots: first inside the wavefront ...
#pragma unroll
    for (int off = W; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < NREP; ++h)
#pragma unroll
            for (int j = 0; j < P; ++j)
                acc[h][j] += __shfl_xor(acc[h][j], off);
    // ... then across the four wavefronts through LDS
    if (lane < W) {
#pragma unroll
        for (int h = 0; h < NREP; ++h)
#pragma unroll
            for (int j = 0; j < P; ++j)
                acc_s[wave][h][P * w + j] = acc[h][j];
    }
    // l: sum of every thread's running partial (all scaled to the same m)
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
        const float ls = wave_sum(l_part[h]);
        if (lane == 0)
            red_s[h][wave] = ls;
    }
    __syncthreads();

    const int64_t C = a.num_chunks;
    for (int i = tid; i < NREP * D; i += NT) {
        const int h = i / D, d = i % D;
        const float v = acc_s[0][h][d] + acc_s[1][h][d] + acc_s[2][h][d] + acc_s[3][h][d];
        a.part_acc[(((int64_t)b * a.Hq + h0 + h) * C + c) * D + d] = v;
    }
    if (tid < NREP) {
        const int h = tid;
        const int64_t o = ((int64_t)b * a.Hq + h0 + h) * C + c;
        a.part_m[o] = m_run[h] * kLn2;
        a.part_l[o] = red_s[h][0] + red_s[h][1] + red_s[h][2] + red_s[h][3];
    }
}

template <int D, typename QT, int BITS>
hipError_t launch_d(const PartialArgs &a, int batch, const Launch &l)
{
    int tile = 1;
    for (int t = 8; t >= 1; t >>= 1)
        if (a.n_rep % t == 0) {
            tile = t;
            break;
        }
    dim3 grid((unsigned)a.num_chunks, (unsigned)(a.Hkv * (a.n_rep / tile)), (unsigned)batch);
    switch (tile) {
    case 8:
        hipExtLaunchKernelGGL((sdpa_partial_valu_kernel<D, 8, QT, BITS>), grid, dim3(NT), 0, l.s, l.start, l.stop, 0, a);
        break;
    case 4:
        hipExtLaunchKernelGGL((sdpa_partial_valu_kernel<D, 4, QT, BITS>), grid, dim3(NT), 0, l.s, l.start, l.stop, 0, a);
        break;
    case 2:
        hipExtLaunchKernelGGL((sdpa_partial_valu_kernel<D, 2, QT, BITS>), grid, dim3(NT), 0, l.s, l.start, l.stop, 0, a);
        break;
    default:
        hipExtLaunchKernelGGL((sdpa_partial_valu_kernel<D, 1, QT, BITS>), grid, dim3(NT), 0, l.s, l.start, l.stop, 0, a);
        break;
    }
    return hipGetLastError();
}

template <typename QT, int BITS>
hipError_t launch_q(const PartialArgs &a, int D, int batch, const Launch &l)
{
    switch (D) {
    case 64:
        return launch_d<64, QT, BITS>(a, batch, l);
    case 128:
        return launch_d<128, QT, BITS>(a, batch, l);
    case 256:
        return launch_d<256, QT, BITS>(a, batch, l);
    default:
        return hipErrorInvalidValue;
    }
}

template <int BITS>
hipError_t launch_b(const PartialArgs &a, int D, int q_dtype, int batch, const Launch &l)
{
    return q_dtype == KVQ_F16 ? launch_q<_Float16, BITS>(a, D, batch, l) : launch_q<float, BITS>(a, D, batch, l);
}

}  // namespace

hipError_t launch_partial_valu(const PartialArgs &a, int D, int q_dtype, int batch, const Launch &l)
{
    if (a.bits == 8)
        return launch_b<8>(a, D, q_dtype, batch, l);
    return a.bits == 4 ? launch_b<4>(a, D, q_dtype, batch, l) : hipErrorInvalidValue;
}

}  // namespace kvq
