// Split-K decode attention on the int4 cache, matrix-core variant for gfx950.
//
// Same contract as the vector-ALU kernel (phase 1 of the split-K scheme in
// the "turboquant-llama3.170B" README: per (KV head, 512-row chunk) partial
// softmax state), but the two contractions run on v_mfma_f32_16x16x32_f16.
// With GQA the n_rep query heads of a KV head share every K and V row, so the
// decode step is a skinny dense product, (n_rep x D) . (D x T) for scores and
// (n_rep x T) . (T x D) for values; at 8 query heads per KV head it needs
// 14.2 multiply-adds per cache byte, more than the fp32 vector ALU delivers
// at HBM speed.
//
// Exactness of the fp16 operands:
//  - codes enter as the exact fp16 integers code - 8 (magic-number unpack and
//    an exact fp16 subtraction; see Unpacker for why they are centred);
//  - fp16 Q is exact; fp32 Q is split into hi + lo fp16 halves (two MFMAs);
//  - the value weights p * scale_v are split into hi + lo fp16 halves, so
//    about 22 bits of each weight survive (the four-wavefront kernel takes
//    them in two MFMAs; the one-wavefront kernel keeps the lo halves times
//    2^11 in operand rows of their own, above the fp16 subnormals);
//  - products of these operands are exact before the matrix core sums them.
// Scale and bias are applied outside the matrix core, per group, as in
// "What I Built Instead" (Gemma page): q . k^ = sum_g s_g (q . code)_g +
// b_g (sum q)_g, and sum_t p v^ = sum_t (p s_v) code + sum_t p b_v.
//
// Score GEMM: S[t][(h,g)] = Kcodes[t][:] . Qg[(h,g)][:], where column (h,g)
// of Qg holds query head h restricted to scale group g (zeros elsewhere), so
// each group's partial dot product comes out separately. A grid row takes a
// block of the KV head's query heads whose (head, group) columns fit the 16
// columns (8 in the one-wavefront kernel's layouts other than D = 128 with
// two groups, whose value products use rows 8-15 for the lo halves). K rows
// are the A operand: a lane loads 16 bytes (32 nibbles) of one row (8 at
// D = 64); the contraction order of dimensions is permuted identically in
// Qg.
//
// Value GEMM: O[(h,g)][d] += P'_g[(h,g)][t] . Vcodes[t][d]; rows whose group g
// differs from the group of column d are discarded. A lane holds 8 rows of
// one output column, so the V words of its 8 rows are transposed nibble-pair
// by nibble-pair with v_perm while unpacking (at D = 64 a column is half a
// word, four dimensions).
//
// Softmax: each wavefront takes every fourth 32-row tile of the chunk and
// keeps an online softmax across its tiles (the accumulator is rescaled only
// when some head's running max rises); the four wavefronts are merged at the
// end. Scale and bias of K and V are staged in LDS per 512-row round, and a
// wavefront requests the K and V words of all its tiles of the round at once.
//
// Memory access: buffer loads against per-head resources whose size is the
// valid rows (Skv), so rows past the end read as zero without per-row
// clamping, and the eight value rows of a lane share one address register
// (their distances are instruction offsets).
#include "hadamard_row.h"
#include "kvq_internal.h"
#include "mfma_common.h"
#include "quant_rule.h"

namespace kvq {
namespace {


constexpr int NT = 256;                 // threads per workgroup
constexpr int TILE = 32;                // rows per tile
constexpr int MAXT = 4;                 // tiles per wavefront per round
constexpr int ROUND = 4 * MAXT * TILE;  // 512 rows
// Occupancy target (wavefronts per SIMD) for D = 128; D = 256 needs the
// whole register file of one wavefront.
#ifndef WAVES_D128
#define WAVES_D128 2
#endif

__device__ __forceinline__ float quarter_max(float v)
{
    v = fmaxf(v, __shfl_xor(v, 16));
    return fmaxf(v, __shfl_xor(v, 32));
}

__device__ __forceinline__ float quarter_sum(float v)
{
    v += __shfl_xor(v, 16);
    return v + __shfl_xor(v, 32);
}

__device__ __forceinline__ void h4_to_f32(uint2 v, float *out)
{
    out[0] = h_val(v.x & 0xFFFF);
    out[1] = h_val(v.x >> 16);
    out[2] = h_val(v.y & 0xFFFF);
    out[3] = h_val(v.y >> 16);
}

template <int D, int NG, bool Q32>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(D == 128 ? WAVES_D128 : 1)))
void sdpa_partial_mfma_kernel(PartialArgs a)
{
    constexpr int W = D / 8;        // words per row
    constexpr int WPL = W / 4;      // K words per lane per 16-row block
    constexpr int KM = W / 4;       // score MFMAs per 16-row block (32 dims each)
    constexpr int VS = W / 16;      // value column sets of 16 words
    constexpr int WPG = W / NG;     // words per scale group
    constexpr int MAXH = 16 / NG;   // most query heads per KV head
    constexpr int META_HALVES = 4 * NG * ROUND;  // K scale, K bias, V scale, V bias
    constexpr int OUT_FLOATS = 4 * MAXH * D;     // per-wavefront outputs for the merge
    constexpr int SMEM_BYTES = (META_HALVES * 2 > OUT_FLOATS * 4) ? META_HALVES * 2 : OUT_FLOATS * 4;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q4 = lane >> 4;
    const int col = lane & 15;
    const int c = blockIdx.x;
    // grid row y = (KV head, block of its query heads): the n_rep query heads
    // of a KV head come in head_split blocks of nrep columns each
    const int kvh = blockIdx.y / a.head_split;
    const int b = blockIdx.z;
    const int nrep = a.n_rep / a.head_split;
    const int R = nrep * NG;
    const int hl = col / NG, gl = col % NG;
    const bool col_on = col < R;
    const float col_mask = col_on ? 0.0f : -INFINITY;
    const int h0 = kvh * a.n_rep + (blockIdx.y - kvh * a.head_split) * nrep;  // first query head of the block

    // Rows are counted inside one (batch, KV head); the host checks that a
    // head's code array stays below 2 GiB, so 32-bit offsets suffice.
    const int t0 = (int)((int64_t)c * a.chunk);
    const int t1 = (int)min((int64_t)t0 + a.chunk, a.skv);
    const int last = t1 - 1;
    const int64_t kvrow0 = ((int64_t)b * a.Hkv + kvh) * a.cap;
    const uint32_t rows_ok = (uint32_t)a.skv;
    const __amdgpu_buffer_rsrc_t kq = make_rsrc(a.k_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t vq = make_rsrc(a.v_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t mres[4] = {
        make_rsrc(a.k_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.k_bias + kvrow0 * NG, rows_ok * NG * 2u),
        make_rsrc(a.v_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.v_bias + kvrow0 * NG, rows_ok * NG * 2u)};

    __shared__ __align__(16) unsigned char smem[SMEM_BYTES];
    __shared__ float m_s[4][16];
    __shared__ float l_s[4][16];
    uint16_t *meta = reinterpret_cast<uint16_t *>(smem);  // [4][NG][ROUND]

    const Unpacker unpack = Unpacker::make();

    // ---- startup: issue the Q loads, the first round's scale/bias loads and
    //      the first tile's K/V loads back to back, then wait for each group
    //      only where it is first used.
    // Q operand (B of the score GEMM): every lane loads the 8 dimensions of
    // each of its words unconditionally (lanes of unused columns read head
    // 0); entries outside the lane's (head, group) are zeroed afterwards.
    float qv[KM][8];
    {
        const int64_t qrow = ((int64_t)b * a.Hq + h0 + (col_on ? hl : 0)) * D;
#pragma unroll
        for (int u = 0; u < KM; ++u) {
            const int word = WPL * q4 + u;
            if constexpr (Q32) {
                const float *qp = reinterpret_cast<const float *>(a.q) + qrow + 8 * word;
                const float4 x0 = *reinterpret_cast<const float4 *>(qp);
                const float4 x1 = *reinterpret_cast<const float4 *>(qp + 4);
                qv[u][0] = x0.x; qv[u][1] = x0.y; qv[u][2] = x0.z; qv[u][3] = x0.w;
                qv[u][4] = x1.x; qv[u][5] = x1.y; qv[u][6] = x1.z; qv[u][7] = x1.w;
            } else {
                const half8 x = *reinterpret_cast<const half8 *>(reinterpret_cast<const _Float16 *>(a.q) + qrow + 8 * word);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    qv[u][j] = (float)x[j];
            }
        }
    }

    // scale and bias of K and V for one 512-row round, staged in LDS as
    // [array][group][row] (rows past Skv read as zero)
    constexpr int PER = META_HALVES / NT;  // halves per thread
    constexpr int ARR = NG * ROUND;        // halves per array
    static_assert(ARR % NT == 0, "each array is a whole number of thread sweeps");
    uint16_t mtmp[PER];
    auto stage_issue = [&](int rb) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int arr = (i * NT) / ARR;  // compile-time after unrolling
            const int rem = (int)threadIdx.x + (i * NT) % ARR;
            mtmp[i] = __builtin_amdgcn_raw_buffer_load_b16(mres[arr], (rb * NG + rem) * 2, 0, 0);
        }
    };
    auto stage_write = [&]() {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int arr = (i * NT) / ARR;
            const int rem = (int)threadIdx.x + (i * NT) % ARR;
            const int r = rem / NG, g = rem - r * NG;
            meta[(arr * NG + g) * ROUND + r] = mtmp[i];
        }
    };

    // K words (A operand rows) and V words (this lane's 8 rows) of each of
    // this wavefront's tiles in the current round, all requested at once
    uint4 kbuf[MAXT][2][WPL / 4];
    uint32_t vbuf[MAXT][VS][8];
    auto load_tile = [&](int trow, uint4 (&kt)[2][WPL / 4], uint32_t (&vt)[VS][8]) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int off = ((trow + 16 * blk + col) * W + WPL * q4) * 4;
#pragma unroll
            for (int v4 = 0; v4 < WPL / 4; ++v4)
                kt[blk][v4] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kq, off + 16 * v4, 0, 0));
        }
        const int voff = ((trow + 4 * q4) * W + col) * 4;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int s2 = 0; s2 < VS; ++s2)
                vt[s2][j] = __builtin_amdgcn_raw_buffer_load_b32(
                    vq, voff + ((16 * (j >> 2) + (j & 3)) * W + 16 * s2) * 4, 0, 0);
    };

    // every tile of this wavefront in the round starting at rb
    auto load_round = [&](int rb) {
        const int ntile = (min(rb + ROUND, t1) - rb + TILE - 1) / TILE;
#pragma unroll
        for (int k = 0; k < MAXT; ++k)
            if (wave + 4 * k < ntile)
                load_tile(rb + TILE * (wave + 4 * k), kbuf[k], vbuf[k]);
    };

    stage_issue(t0);
    load_round(t0);

    half8 qhi[KM], qlo[KM];
    float qsum = 0.0f;
#pragma unroll
    for (int u = 0; u < KM; ++u) {
        const int word = WPL * q4 + u;
        const bool mine = col_on && (word / WPG) == gl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = mine ? qv[u][kPerm[j]] : 0.0f;
            qsum += x;
            const _Float16 hi = (_Float16)x;
            qhi[u][j] = hi;
            if constexpr (Q32)
                qlo[u][j] = (_Float16)(x - (float)hi);
        }
    }
    qsum = quarter_sum(qsum);

    const float cs = a.score_scale;
    float m_run = -INFINITY, l_run = 0.0f, b_run = 0.0f;
    float4v acc[VS][8];
#pragma unroll
    for (int s = 0; s < VS; ++s)
#pragma unroll
        for (int m = 0; m < 8; ++m)
            acc[s][m] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

    for (int rb = t0; rb < t1; rb += ROUND) {
        const int ntile = (min(rb + ROUND, t1) - rb + TILE - 1) / TILE;
        if (rb != t0) {
            __syncthreads();  // the previous round's readers are done
            stage_issue(rb);
            load_round(rb);
        }
        stage_write();
        __syncthreads();  // metadata staged

        // ---- this wavefront's tiles of the round: ti = wave + 4k, k < kn
        const int kn = (ntile - wave + 3) / 4;  // uniform; <= MAXT

#pragma unroll
        for (int k = 0; k < MAXT; ++k) {
            if (k >= kn)
                break;
            const int ti = wave + 4 * k;
            const bool tail = rb + TILE * ti + TILE > t1;  // uniform
            const uint4 (&kcur)[2][WPL / 4] = kbuf[k];
            const uint32_t (&vcur)[VS][8] = vbuf[k];

            // ---- scores of the tile's 8 rows held by this lane
            float sc[8];
            float mx = -INFINITY;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                float4v sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int u = 0; u < KM; ++u) {
                    const uint4 x = kcur[blk][u / 4];
                    const uint32_t w = (u % 4 == 0) ? x.x : (u % 4 == 1) ? x.y : (u % 4 == 2) ? x.z : x.w;
                    half2v hk[4];
                    unpack(w, hk);
                    const half8 ka = cat8(hk[0], hk[1], hk[2], hk[3]);
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qhi[u], sacc, 0, 0, 0);
                    if constexpr (Q32)
                        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qlo[u], sacc, 0, 0, 0);
                }
                // rows TILE*ti + 16*blk + 4*q4 + i (round-relative) of column (hl, gl)
                const int lr0 = TILE * ti + 16 * blk + 4 * q4;
                float ks[4], kb[4];
                h4_to_f32(*reinterpret_cast<const uint2 *>(&meta[(0 * NG + gl) * ROUND + lr0]), ks);
                h4_to_f32(*reinterpret_cast<const uint2 *>(&meta[(1 * NG + gl) * ROUND + lr0]), kb);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float kb8 = fmaf(8.0f, ks[i], kb[i]);  // bias of the centred codes
                    const float part = fmaf(ks[i], sacc[i], kb8 * qsum);
                    float v = fmaf(group_sum<NG>(part), cs, col_mask);
                    if (tail)
                        v = (rb + lr0 + i <= last) ? v : -INFINITY;
                    sc[4 * blk + i] = v;
                    mx = fmaxf(mx, v);
                }
            }

            // ---- online softmax across tiles: rescale only when a head's max rises
            mx = quarter_max(mx);
            const float m_new = fmaxf(m_run, mx);
            const bool first = (rb == t0) && (k == 0);
            if (!first && __builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
                const float corr = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.0f : m_new));
                l_run *= corr;
                b_run *= corr;
                // accumulator element i of this lane belongs to row 4*q4 + i,
                // whose factor lives in the lane of that column
                float4v corr_row;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    corr_row[i] = __shfl(corr, 4 * q4 + i);
#pragma unroll
                for (int s2 = 0; s2 < VS; ++s2)
#pragma unroll
                    for (int m = 0; m < 8; ++m)
                        acc[s2][m] *= corr_row;
            }
            m_run = m_new;
            const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;

            // ---- weights and values
            float vs[8], vb[8];
            {
                const int lr0 = TILE * ti + 4 * q4;
                h4_to_f32(*reinterpret_cast<const uint2 *>(&meta[(2 * NG + gl) * ROUND + lr0]), &vs[0]);
                h4_to_f32(*reinterpret_cast<const uint2 *>(&meta[(2 * NG + gl) * ROUND + lr0 + 16]), &vs[4]);
                h4_to_f32(*reinterpret_cast<const uint2 *>(&meta[(3 * NG + gl) * ROUND + lr0]), &vb[0]);
                h4_to_f32(*reinterpret_cast<const uint2 *>(&meta[(3 * NG + gl) * ROUND + lr0 + 16]), &vb[4]);
            }
            half8 phi, plo;
            float lsum = 0.0f, bsum = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p = __builtin_amdgcn_exp2f(sc[j] - m_use);
                lsum += p;
                bsum = fmaf(p, fmaf(8.0f, vs[j], vb[j]), bsum);  // bias of the centred codes
                const float pw = p * vs[j];
                const _Float16 hi = (_Float16)pw;
                phi[j] = hi;
                plo[j] = (_Float16)(pw - (float)hi);
            }
            l_run += lsum;
            b_run += bsum;
#pragma unroll
            for (int s2 = 0; s2 < VS; ++s2) {
                half2v lo4[4][4], hi4[4][4];  // [pair][m]
#pragma unroll
                for (int jp = 0; jp < 4; ++jp) {
                    const uint32_t x = __builtin_amdgcn_perm(vcur[s2][2 * jp + 1], vcur[s2][2 * jp], 0x05040100u);
                    const uint32_t y = __builtin_amdgcn_perm(vcur[s2][2 * jp + 1], vcur[s2][2 * jp], 0x07060302u);
                    unpack(x, lo4[jp]);
                    unpack(y, hi4[jp]);
                }
#pragma unroll
                for (int m = 0; m < 8; ++m) {
                    const half8 bv = m < 4 ? cat8(lo4[0][m], lo4[1][m], lo4[2][m], lo4[3][m])
                                           : cat8(hi4[0][m - 4], hi4[1][m - 4], hi4[2][m - 4], hi4[3][m - 4]);
                    acc[s2][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi, bv, acc[s2][m], 0, 0, 0);
                    acc[s2][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(plo, bv, acc[s2][m], 0, 0, 0);
                }
            }

        }
    }

    // ---- wavefront totals: l and the value-bias term per column (h, g)
    const float l_tot = quarter_sum(l_run);
    const float b_tot = quarter_sum(b_run);
    __syncthreads();  // metadata no longer read: the buffer now holds outputs
    float *out_s = reinterpret_cast<float *>(smem);  // [4][MAXH][D]
    if (q4 == 0) {
        m_s[wave][col] = m_run;
        l_s[wave][col] = l_tot;
    }
    // accumulator lane layout: rows r' = 4*q4 + i, column n = col
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = 4 * q4 + i;
        const float bias_r = __shfl(b_tot, rr);
        if (rr < R) {
            const int h = rr / NG, g = rr % NG;
#pragma unroll
            for (int s = 0; s < VS; ++s) {
                const int word = 16 * s + col;
                if (word / WPG == g) {
#pragma unroll
                    for (int m = 0; m < 8; ++m)
                        out_s[(wave * MAXH + h) * D + 8 * word + m] = acc[s][m][i] + bias_r;
                }
            }
        }
    }
    __syncthreads();

    // ---- merge the four wavefronts and write the partial state
    const int64_t C = a.num_chunks;
    for (int e = threadIdx.x; e < nrep * D; e += NT) {
        const int h = e / D, d = e % D;
        const int r0 = h * NG;  // any group column of head h carries its m and l
        const float M = fmaxf(fmaxf(m_s[0][r0], m_s[1][r0]), fmaxf(m_s[2][r0], m_s[3][r0]));
        float accv = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
            accv = fmaf(__builtin_amdgcn_exp2f(m_s[w][r0] - M), out_s[(w * MAXH + h) * D + d], accv);
        const int64_t o = ((int64_t)b * a.Hq + h0 + h) * C + c;
        a.part_acc[o * D + d] = accv;
        if (d == 0) {
            float L = 0.0f;
#pragma unroll
            for (int w = 0; w < 4; ++w)
                L = fmaf(__builtin_amdgcn_exp2f(m_s[w][r0] - M), l_s[w][r0], L);
            a.part_m[o] = M * kLn2;
            a.part_l[o] = L;
        }
    }
}

// ---------------------------------------------------------------------------
// One-wavefront variant: a 64-thread workgroup owns one (chunk <= 512 rows,
// KV head, batch). The same tile computation as above, but with no barriers
// and no cross-wavefront merge: the chunk's scale and bias are staged once in
// a wavefront-private LDS area, K/V tiles stream through a static ring of PF
// tiles in flight (slot u is refilled with tile u + PF right after tile u is
// consumed), and the partial state is written straight from registers. With
// 512-row chunks every wavefront streams 16 tiles, so its start-up latency is
// paid once per 73 KB instead of once per 18 KB.
// ---------------------------------------------------------------------------
constexpr int CH1 = 512;  // most rows of a chunk in the one-wavefront kernel

// Fused decode step: quantise this (batch, KV head)'s new K and V rows into
// cache row a.append_row (the rule of quant_rule.h; lanes 0..D/8-1 take the
// K words, the next D/8 lanes the V words, idle lanes only join the swaps of
// their group), then wait until the stores are done, so that the wavefront's
// later loads of that row, all issued after this, see the new values.
template <int D, int NG, int BITS>
__device__ void append_new_row(const PartialArgs &a, int b, int kvh, int64_t kvrow0)
{
    constexpr int W = D / 8;     // lanes per row (eight values each)
    constexpr int LPG = W / NG;  // lanes per scale group
    const int lane = threadIdx.x & 63;
    const bool active = lane < 2 * W;
    const int which = lane / W;  // 0: K, 1: V
    const int w = lane % W;
    const int64_t src = ((int64_t)b * a.Hkv + kvh) * D + 8 * w;
    float x[8];
    if (!active) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = 0.0f;
    } else if (a.append_dtype == KVQ_F32) {
        quant::load8<float>(reinterpret_cast<const float *>(which ? a.v_new : a.k_new) + src, x);
    } else {
        quant::load8<_Float16>(reinterpret_cast<const _Float16 *>(which ? a.v_new : a.k_new) + src, x);
    }
    if (a.rotate & kRotateRows) {  // uniform: the rows of a Hadamard-rotated cache (fp16 rows, W lanes each)
        double xd[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            xd[j] = (double)x[j];
        hadamard_row(xd, w, W, a.rot_scale);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = (float)xd[j];
    }
    uint16_t sb, bb;
    uint32_t words[BITS / 4];
    quant::quantize_codes<LPG, BITS>(x, words, sb, bb);
    if (active) {
        const int64_t row = kvrow0 + a.append_row;
        uint32_t *dq = const_cast<uint32_t *>(which ? a.v_q : a.k_q);
        if constexpr (BITS == 4)
            dq[row * W + w] = words[0];
        else
            *reinterpret_cast<uint2 *>(dq + row * (2 * W) + 2 * w) = make_uint2(words[0], words[1]);
        if (w % LPG == 0) {
            uint16_t *ds = const_cast<uint16_t *>(which ? a.v_scale : a.k_scale);
            uint16_t *db = const_cast<uint16_t *>(which ? a.v_bias : a.k_bias);
            ds[row * NG + w / LPG] = sb;
            db[row * NG + w / LPG] = bb;
        }
    }
    // every store of this wavefront has completed before any later load issues
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

// Merges of the decode step's multi-wavefront workgroups, run by all
// 64 * WG threads of a workgroup after each wavefront has put its state (m
// in log2 units, l, and the D value sums of each of its nrep query heads)
// into LDS, heads MAXH apart. 1) The workgroup merges its wavefronts' states
// into one partial state. Then either
//  - (a.part_acc set) it stores that state as split-K partial blockIdx.x
//    of a.nwg, for the reduce kernel launched after it; or
//  - the split-K merge of the README's split-K paragraph happens inside the
//    same launch: 2) the workgroup stores its partial in a.merge_ws, waits
//    until the stores are complete and takes a ticket from its (batch, KV
//    head) arrival counter; all but the last of the a.nwg workgroups are
//    then done; 3) the last one reads the other partials, merges them with
//    its own (kept in registers) into the normalised output and sets the
//    counter back to zero. The partials cross workgroups, and the chip's
//    separate L2 caches, as device-scope atomic stores and loads (coherent
//    at the device's memory side); a store is complete before its
//    workgroup's ticket is taken, and every load of the last workgroup is
//    issued after its own ticket came back, after every other ticket.
// Elements are handled in pairs of adjacent dimensions (one 64-bit access).
// bh: the (batch, grid row) index of this workgroup's counter and partials;
// hq0: the index b * Hq + h of its first query head.
template <int D, int NG, int WG>
__device__ __forceinline__ void merge_epilogue(const PartialArgs &a, int64_t bh, int64_t hq0, int nrep,
                                               const float *ml_s, const float *acc_s)
{
    constexpr int NT1 = 64 * WG;
    constexpr int MAXH = 16 / NG;
    constexpr int EP = (MAXH * D / 2 + NT1 - 1) / NT1;  // dimension pairs per thread, at most
    constexpr int PB = 32 / EP;                         // partials per batch of loads (128 registers)
    const int tid = threadIdx.x;
    const int nwg = a.nwg;
    const int npair = nrep * D / 2;
    __syncthreads();  // every wavefront's state is in LDS

    // 1) this workgroup's partial: per head the largest m, then every
    //    wavefront's state weighted by exp2(m_w - M) (0 for one without rows)
    float2 own[EP];
    float own_m[EP], own_l[EP];  // of each pair's head
#pragma unroll
    for (int k = 0; k < EP; ++k) {
        const int pr = tid + k * NT1;
        own[k] = make_float2(0.0f, 0.0f);
        own_m[k] = -INFINITY;
        own_l[k] = 0.0f;
        if (pr < npair) {
            const int h = 2 * pr / D, d = 2 * pr % D;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < WG; ++w)
                M = fmaxf(M, ml_s[(w * MAXH + h) * 2]);
            float2 sum = make_float2(0.0f, 0.0f);
            float L = 0.0f;
#pragma unroll
            for (int w = 0; w < WG; ++w) {
                const float f = __builtin_amdgcn_exp2f(ml_s[(w * MAXH + h) * 2] - M);
                const float2 v = *reinterpret_cast<const float2 *>(acc_s + (w * MAXH + h) * D + d);
                sum.x = fmaf(f, v.x, sum.x);
                sum.y = fmaf(f, v.y, sum.y);
                L = fmaf(f, ml_s[(w * MAXH + h) * 2 + 1], L);
            }
            own[k] = sum;
            own_m[k] = M;
            own_l[k] = L;
        }
    }

    if (a.part_acc) {  // split-K partial blockIdx.x of nwg, m in natural-log units
        const int64_t C = nwg;
        const int64_t o = hq0 * C + blockIdx.x;
#pragma unroll
        for (int k = 0; k < EP; ++k) {
            const int pr = tid + k * NT1;
            if (pr < npair) {
                const int h = 2 * pr / D, d = 2 * pr % D;
                *reinterpret_cast<float2 *>(a.part_acc + (o + h * C) * D + d) = own[k];
                if (d == 0) {
                    a.part_m[o + h * C] = own_m[k] * kLn2;
                    a.part_l[o + h * C] = own_l[k];
                }
            }
        }
        return;
    }

    // 2) the partial into the workspace: [nwg][kMergeHeader + nrep D] words,
    //    (m, l) pairs of the heads first, then the value sums
    const int stride = kMergeHeader + nrep * D;
    uint64_t *ws = reinterpret_cast<uint64_t *>(a.merge_ws + bh * nwg * (int64_t)stride);  // 8-byte words
    uint64_t *mine = ws + (int64_t)blockIdx.x * (stride / 2);
#pragma unroll
    for (int k = 0; k < EP; ++k) {
        const int pr = tid + k * NT1;
        if (pr < npair) {
            __hip_atomic_store(mine + kMergeHeader / 2 + pr, __builtin_bit_cast(uint64_t, own[k]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            if (2 * pr % D == 0)
                __hip_atomic_store(mine + 2 * pr / D, __builtin_bit_cast(uint64_t, make_float2(own_m[k], own_l[k])),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);  // the stores are complete
    __shared__ uint32_t ticket;
    __syncthreads();
    if (tid == 0)
        ticket = __hip_atomic_fetch_add(a.counters + bh, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (ticket != (uint32_t)nwg - 1)
        return;

    // 3) the last workgroup: out = sum_p exp2(m_p - M) acc_p / sum_p exp2(m_p - M) l_p,
    //    the partials taken in index order (so the result does not depend on
    //    which workgroup came last), PB at a time with every load of a batch
    //    issued before the first is used
    float M[EP], L[EP];
    float2 acc[EP];
#pragma unroll
    for (int k = 0; k < EP; ++k) {
        M[k] = -INFINITY;
        L[k] = 0.0f;
        acc[k] = make_float2(0.0f, 0.0f);
    }
    const int me = blockIdx.x;
    for (int p0 = 0; p0 < nwg; p0 += PB) {
        float2 ml[PB][EP], av[PB][EP];
#pragma unroll
        for (int u = 0; u < PB; ++u) {
            const uint64_t *src = ws + (int64_t)min(p0 + u, nwg - 1) * (stride / 2);
#pragma unroll
            for (int k = 0; k < EP; ++k) {
                const int pr = min(tid + k * NT1, npair - 1);
                ml[u][k] = __builtin_bit_cast(
                    float2, __hip_atomic_load(src + 2 * pr / D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                av[u][k] = __builtin_bit_cast(
                    float2, __hip_atomic_load(src + kMergeHeader / 2 + pr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            }
        }
#pragma unroll
        for (int k = 0; k < EP; ++k) {
            float Mn = M[k];
#pragma unroll
            for (int u = 0; u < PB; ++u)
                if (p0 + u < nwg)
                    Mn = fmaxf(Mn, p0 + u == me ? own_m[k] : ml[u][k].x);
            const float r = __builtin_amdgcn_exp2f(M[k] - Mn);  // 0 while M is -inf (Mn is finite)
            L[k] *= r;
            acc[k].x *= r;
            acc[k].y *= r;
#pragma unroll
            for (int u = 0; u < PB; ++u)
                if (p0 + u < nwg) {
                    const bool self = p0 + u == me;
                    const float f = __builtin_amdgcn_exp2f((self ? own_m[k] : ml[u][k].x) - Mn);
                    const float2 v = self ? own[k] : av[u][k];
                    L[k] = fmaf(f, self ? own_l[k] : ml[u][k].y, L[k]);
                    acc[k].x = fmaf(f, v.x, acc[k].x);
                    acc[k].y = fmaf(f, v.y, acc[k].y);
                }
            M[k] = Mn;
        }
    }
#pragma unroll
    for (int k = 0; k < EP; ++k) {
        const int pr = tid + k * NT1;
        if (pr < npair) {
            const int h = 2 * pr / D, d = 2 * pr % D;
            *reinterpret_cast<float2 *>(a.out + (hq0 + h) * D + d) =
                make_float2(acc[k].x / L[k], acc[k].y / L[k]);
        }
    }
    if (tid == 0)
        __hip_atomic_store(a.counters + bh, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// WG wavefronts per workgroup. WG = 1: the split-K partial kernel, one
// (chunk, KV head, batch) per workgroup, its state written as that chunk's
// partial. WG > 1: the single-launch decode step, WG consecutive chunks of
// one (KV head, batch) per workgroup, merged in LDS, then across workgroups
// by the last one to arrive (merge_epilogue).
template <int D, int NG, bool Q32, int PF, int BITS, int WG = 1>
__global__ __launch_bounds__(64 * WG) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void sdpa_partial_mfma1_kernel(PartialArgs a)
{
    // BITS = 8: byte codes, two words per eight dimensions, both K and V
    // codes entering as the exact centred integers n - 128. The value
    // weights p * s_v are carried times WS = 2^6: byte scales are 17 times
    // finer than int4 ones, and the factor keeps the weights' fp16 halves as
    // far above the subnormal range as with int4 codes, while
    // p * s_v * 2^6 <= 514 * 64 stays below the fp16 maximum for any fp16
    // input range. The value products are multiplied by VU = 1 / WS when the
    // partial state is written.
    static_assert(PF % 2 == 0, "the scale/bias ring alternates two slots");
    constexpr bool B8 = BITS == 8;
    // D = 64: eight dimension octets per row, so each of the 16 value
    // columns is half an octet (octet col & 7, dimensions 4 (col >> 3) + m,
    // m < 4); otherwise a column is a whole octet
    constexpr bool HV = D == 64;
    constexpr int W = D * BITS / 32;  // words per row
    constexpr int WPL = W / 4;        // K words per lane: a quarter row
    constexpr int KV4 = (WPL + 3) / 4;  // 16-byte K loads per lane and block (int4 at D = 64: one 8-byte load)
    constexpr int KM = D / 32;        // score products per 16-row block
    constexpr int VS = HV ? 1 : D / 128;  // sets of 16 value columns
    constexpr int VM = HV ? 4 : 8;        // dimensions per value column
    constexpr int VW = BITS / 4;      // value words per row and octet
    constexpr int NV = HV ? 1 : VW;   // value words per row and column
    constexpr int WPG = D / 8 / NG;   // eight-dimension columns per scale group
    constexpr float VC = B8 ? 128.0f : 8.0f;     // centre of the value codes
    constexpr float WS = B8 ? 64.0f : 1.0f;      // scale of the value weights
    constexpr float VU = B8 ? 1.0f / 64.0f : 1.0f;  // unit of the value products: 1 / WS
    constexpr int PAIRS = TILE * NG;        // (row, group) pairs of scale/bias per tile
    constexpr int MP = (PAIRS + 63) / 64;   // pairs per lane (NG = 1: lanes 32-63 repeat 0-31)
    // D = 128 with two scale groups: value products group by group, with the
    // hi and lo weight halves as operand rows (half the matrix instructions).
    // Every other layout has at most 8 score columns (the host's head
    // blocks): the hi halves of columns 0-7 are operand rows 0-7 and their lo
    // halves rows 8-15, so that one matrix instruction takes both. Either way
    // the lo halves are stored times kLoScale, above the fp16 subnormals.
    constexpr bool GV = D == 128 && NG == 2;
    constexpr float LS = kLoScale;  // scale of the lo weight halves

    const int lane = threadIdx.x & 63;
    const int wave = WG > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
    const int q4 = lane >> 4;
    const int col = lane & 15;
    const int c = blockIdx.x * WG + wave;  // this wavefront's chunk of rows
    // grid row y = (KV head, block of its query heads), as in the split kernel
    const int kvh = blockIdx.y / a.head_split;
    const int b = blockIdx.z;
    const int nrep = a.n_rep / a.head_split;
    const int R = nrep * NG;
    // score column col = (head hl, scale group gl): hl * NG + gl, or with GV
    // hl + 8 gl, so that a lane and its partner of the other group are
    // lanes l and l ^ 8, which a bank-masked DPP move can pair
    const int hl = GV ? (col & 7) : col / NG, gl = GV ? (col >> 3) : col % NG;
    // columns without a query head compute on zero Q and are never written;
    // every column keeps its own softmax state, so they need no masking
    const bool col_on = hl < nrep;
    const int h0 = kvh * a.n_rep + (blockIdx.y - kvh * a.head_split) * nrep;  // first query head of the block
    const bool low8 = (lane & 8) == 0;  // GV: this lane's V word is in group 0

    // Rows of this wavefront: tiles of TILE rows from t0, TS * TILE apart,
    // below t1. WG = 1: the chunk [c * chunk, (c + 1) * chunk). WG > 1: the
    // workgroup's WG * chunk rows, its wavefronts taking every WG-th tile
    // (at any time the workgroup streams one region of each array instead of
    // WG of them).
    constexpr int TS = WG;
    const int t0 = WG == 1 ? (int)((int64_t)c * a.chunk)
                           : (int)((int64_t)blockIdx.x * WG * a.chunk) + TILE * wave;
    const int t1 = WG == 1 ? (int)min((int64_t)t0 + a.chunk, a.skv)
                           : (int)min((int64_t)(blockIdx.x + 1) * WG * a.chunk, a.skv);
    const int last = t1 - 1;
    const int ntile = t1 > t0 ? (t1 - t0 + TS * TILE - 1) / (TS * TILE) : 0;
    const int64_t kvrow0 = ((int64_t)b * a.Hkv + kvh) * a.cap;
    // uniform: the fused decode step's new row is in one of this wavefront's
    // tiles. Every query-head block of the KV head quantises and stores it:
    // the stores are the same bytes, and each block reads the row only after
    // its own stores are complete, so no block can see the old row.
    if (a.append_row >= t0 && a.append_row < t1 && ((a.append_row - t0) / TILE) % TS == 0)
        append_new_row<D, NG, BITS>(a, b, kvh, kvrow0);
    const uint32_t rows_ok = (uint32_t)a.skv;
    const __amdgpu_buffer_rsrc_t kq = make_rsrc(a.k_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t vq = make_rsrc(a.v_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t mres[4] = {
        make_rsrc(a.k_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.k_bias + kvrow0 * NG, rows_ok * NG * 2u),
        make_rsrc(a.v_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.v_bias + kvrow0 * NG, rows_ok * NG * 2u)};

    // Scale and bias travel with the tiles: a lane loads the four fp16 values
    // of MP (row, group) pairs of a tile; one tile ahead of use they become
    // the fp32 factors of the tile code, one 16-byte record per pair in a
    // two-slot LDS buffer [slot][row * NG + group]:
    //   x: s_k * c * 2^20     (c = softmax scale * log2 e; 2^20 undoes the
    //                          subnormal scale of the int4 K operands), or
    //      s_k * c            (8-bit codes)
    //   y: b_k * c, or (b_k + 128 s_k) * c (the bias of centred 8-bit codes)
    //   z: s_v * WS
    //   w: b_v + VC s_v       (bias of the value codes centred by VC)
    __shared__ __align__(16) float4 mring_all[WG][2][PAIRS];
    float4 (&mring)[2][PAIRS] = mring_all[wave];
    const Unpacker unpack = Unpacker::make();
    const uint32_t m_fine = opaque_s_if<!B8>(0x00F000F0u);  // int4 K operands
    // 8-bit K operands: the magic exponent bytes (src0 bytes 4-7 of a permute)
    // and the selectors of bytes (0, 2) and (1, 3) under them
    const uint32_t magic8 = opaque_s_if<B8>(kMagic1024x4), magic16 = opaque_s_if<B8>(0x64006400u);
    const uint32_t sel_even = opaque_s_if<B8>(0x04020400u), sel_odd = opaque_s_if<B8>(0x04030401u);
    // 8-bit value pairs: byte m of the low source word into bits 0-7, byte m
    // of the high one into bits 16-23, zeros elsewhere
    const uint32_t sel_b[4] = {opaque_s_if<B8>(0x0C040C00u), opaque_s_if<B8>(0x0C050C01u),
                               opaque_s_if<B8>(0x0C060C02u), opaque_s_if<B8>(0x0C070C03u)};
    const float cs = a.score_scale;
    const float csk = B8 ? cs : cs * 1048576.0f;  // c, times 2^20 for the int4 K operands

    // ---- start-up: Q and the first PF tiles, all requested before the first wait
    float qv[KM][8];
    bool q_done = false;
    if constexpr (Q32 && D == 128) {
        if (a.rotate & kRotateQuery) {  // uniform: the query of a Hadamard-rotated cache
            // this lane's 32 dimensions 32 q4 + 8 u + j (exact in fp32), to be
            // rotated once the first tiles are requested
            const int64_t qrow = ((int64_t)b * a.Hq + h0 + (col_on ? hl : 0)) * D + 32 * q4;
#pragma unroll
            for (int u = 0; u < KM; ++u)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    qv[u][j] = a.q_f16 ? (float)reinterpret_cast<const _Float16 *>(a.q)[qrow + 8 * u + j]
                                       : reinterpret_cast<const float *>(a.q)[qrow + 8 * u + j];
            q_done = true;
        }
    }
    if (!q_done) {
        const int64_t qrow = ((int64_t)b * a.Hq + h0 + (col_on ? hl : 0)) * D;
#pragma unroll
        for (int u = 0; u < KM; ++u) {
            const int word = KM * q4 + u;  // dimensions 8 word .. 8 word + 7
            if constexpr (Q32) {
                const float *qp = reinterpret_cast<const float *>(a.q) + qrow + 8 * word;
                const float4 x0 = *reinterpret_cast<const float4 *>(qp);
                const float4 x1 = *reinterpret_cast<const float4 *>(qp + 4);
                qv[u][0] = x0.x; qv[u][1] = x0.y; qv[u][2] = x0.z; qv[u][3] = x0.w;
                qv[u][4] = x1.x; qv[u][5] = x1.y; qv[u][6] = x1.z; qv[u][7] = x1.w;
            } else {
                const half8 x = *reinterpret_cast<const half8 *>(reinterpret_cast<const _Float16 *>(a.q) + qrow + 8 * word);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    qv[u][j] = (float)x[j];
            }
        }
    }

    // Every ring refill is issued, also past the chunk's last tile: such a
    // request gets a byte base beyond the buffer's records, so it returns
    // zeros without touching memory. Unconditional requests keep the number
    // of loads in flight the same on every path, so each wait only covers the
    // data about to be used instead of draining the whole ring.
    constexpr uint32_t kNoRows = 0x80000000u;  // > any records size (capacity * D * BITS / 8 < 2^31)
    uint4 kbuf[PF][2][KV4];
    uint32_t vbuf[PF][VS][8 * NV];
    uint32_t mbuf[PF][MP][4];
    // scale/bias of a tile first, then its K and V words (a wait for the
    // scale/bias of the next tile then leaves that tile's words in flight)
    auto load_tile = [&](int ti, uint4 (&kt)[2][KV4], uint32_t (&vt)[VS][8 * NV], uint32_t (&mt)[MP][4]) {
        const bool in = ti < ntile;
#pragma unroll
        for (int p = 0; p < MP; ++p) {
            const int pr = (lane + 64 * p) % PAIRS;
            const uint32_t off = in ? (uint32_t)((t0 + TS * TILE * ti) * NG + pr) * 2u : kNoRows;
#pragma unroll
            for (int arr = 0; arr < 4; ++arr)
                mt[p][arr] = __builtin_amdgcn_raw_buffer_load_b16(mres[arr], off, 0, 0);
        }
        const uint32_t base = in ? (uint32_t)(t0 + TS * TILE * ti) * (uint32_t)(W * 4) : kNoRows;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const uint32_t off = base + (uint32_t)(((16 * blk + col) * W + WPL * q4) * 4);
            if constexpr (WPL == 2) {
                const auto x = __builtin_amdgcn_raw_buffer_load_b64(kq, off, 0, 0);
                kt[blk][0] = make_uint4(x[0], x[1], 0u, 0u);
            } else {
#pragma unroll
                for (int v4 = 0; v4 < KV4; ++v4)
                    kt[blk][v4] =
                        __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kq, off + 16 * v4, 0, 0));
            }
        }
        // first value word of this lane's column in a row; with HV the word
        // that holds dimensions 8 (col & 7) + 4 (col >> 3) .. + 3 (int4: the
        // word of the whole octet)
        const int vcol = HV ? (B8 ? 2 * (col & 7) + (col >> 3) : (col & 7)) : VW * col;
        const uint32_t voff = base + (uint32_t)((4 * q4 * W + vcol) * 4);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int s2 = 0; s2 < VS; ++s2) {
                const uint32_t o = voff + ((16 * (j >> 2) + (j & 3)) * W + 16 * VW * s2) * 4;
                if constexpr (HV) {
                    vt[s2][j] = __builtin_amdgcn_raw_buffer_load_b32(vq, o, 0, 0);
                } else if constexpr (B8) {
                    const auto x = __builtin_amdgcn_raw_buffer_load_b64(vq, o, 0, 0);
                    vt[s2][2 * j] = x[0];
                    vt[s2][2 * j + 1] = x[1];
                } else {
                    vt[s2][j] = __builtin_amdgcn_raw_buffer_load_b32(vq, o, 0, 0);
                }
            }
    };
    auto stage_meta = [&](int slot, const uint32_t (&mt)[MP][4]) {
#pragma unroll
        for (int p = 0; p < MP; ++p) {
            const int pr = (lane + 64 * p) % PAIRS;
            const float ks = h_val((uint16_t)mt[p][0]);
            const float kb = h_val((uint16_t)mt[p][1]);
            const float vs = h_val((uint16_t)mt[p][2]);
            const float vb = h_val((uint16_t)mt[p][3]);
            mring[slot][pr] = make_float4(ks * csk, (B8 ? fmaf(128.0f, ks, kb) : kb) * cs, vs * WS, fmaf(VC, vs, vb));
        }
        // LDS instructions of a wavefront execute in order, so the tile code
        // sees these records; only the compiler must not move reads above
        asm volatile("" ::: "memory");
    };
    // Issue the first PF tiles slot by slot, in the order the ring refills
    // them. The wait counts at the loop head are the smaller of the start-up
    // and the steady-state ones; a start-up order with all K loads last would
    // make every pass over the ring wait for nearly all loads in flight.
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        load_tile(u, kbuf[u], vbuf[u], mbuf[u]);
    }
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (Q32 && D == 128) {
        if (a.rotate & kRotateQuery) {
            // the query rotated in fp32 (its exact fp16 or fp32 values, seven
            // butterfly stages: a relative error of a few 2^-24, far below
            // the scores' own): dimension bits 0-4 inside the lane, bits 5
            // and 6 between the lanes l ^ 16 and l ^ 32 that hold the rest of
            // the head, each stage x' = partner + sign * x
#pragma unroll
            for (int sb = 1; sb < KM * 8; sb <<= 1)
#pragma unroll
                for (int j = 0; j < KM * 8; ++j)
                    if (!(j & sb)) {
                        float &x0 = qv[j / 8][j % 8], &x1 = qv[(j | sb) / 8][(j | sb) % 8];
                        const float p = x0, r = x1;
                        x0 = p + r;
                        x1 = p - r;
                    }
#pragma unroll
            for (int mb = 16; mb < 64; mb <<= 1) {
                const float sign = (lane & mb) ? -1.0f : 1.0f;
#pragma unroll
                for (int u = 0; u < KM; ++u)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        qv[u][j] = fmaf(sign, qv[u][j], __shfl_xor(qv[u][j], mb));
            }
            const float rs = (float)a.rot_scale;
#pragma unroll
            for (int u = 0; u < KM; ++u)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    qv[u][j] *= rs;
        }
    }

    // Q restricted to the column's group, in the dimension order of the K
    // operands; qsum is the group sum of exactly what the matrix core sees
    half8 qhi[KM], qlo[KM];
    float qsum = 0.0f;
#pragma unroll
    for (int u = 0; u < KM; ++u) {
        const int word = KM * q4 + u;
        const bool mine = col_on && (word / WPG) == gl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = mine ? qv[u][B8 ? kPerm8[j] : kPerm[j]] : 0.0f;
            const _Float16 hi = (_Float16)x;
            qhi[u][j] = hi;
            if constexpr (Q32) {
                const _Float16 lo = (_Float16)(x - (float)hi);
                qlo[u][j] = lo;
                qsum += (float)hi + (float)lo;
            } else {
                qsum += (float)hi;
            }
        }
    }
    qsum = xrow_sum(qsum);
    stage_meta(0, mbuf[0]);

    // m_run: the softmax reference of this lane's head (log2 units); scores
    // are computed relative to it, each of the NG group columns of a head
    // subtracting m_part = m_run / NG before their sum. m_top: this lane's
    // largest score so far, relative to m_run (the partial state is written
    // against the true maximum, which lies in [m_run - kHeadroom, m_run]).
    float m_run = 0.0f, m_part = 0.0f, l_run = 0.0f, b_run = 0.0f, m_top = -INFINITY;
    float4v acc[VS][VM];
#pragma unroll
    for (int s = 0; s < VS; ++s)
#pragma unroll
        for (int m = 0; m < VM; ++m)
            acc[s][m] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll 1
    for (int kk = 0; kk < ntile; kk += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            // tiles past the chunk (ntile not a multiple of PF) are run too:
            // their rows are all masked and their codes read as zeros, so
            // they add nothing, and the loop has no exit but its own test
            const int ti = kk + u;
            const int slot = u & 1;  // PF is even, so this is ti & 1
            const uint4 (&kcur)[2][KV4] = kbuf[u];
            const uint32_t (&vcur)[VS][8 * NV] = vbuf[u];

            // factors of the tile's 8 rows held by this lane: rows 4*q4 + i
            // (i < 4) and 16 + 4*q4 + i - 4 (i >= 4), column group gl
            float4 fac[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                fac[i] = mring[slot][(16 * (i >> 2) + 4 * q4 + (i & 3)) * NG + gl];

            // ---- scores of the tile's 8 rows held by this lane (log2 units)
            float sc[8];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                float4v sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int uu = 0; uu < KM; ++uu) {
                    half8 ka;
                    if constexpr (B8) {
                        const uint4 x = kcur[blk][uu / 2];
                        ka = (uu % 2 == 0) ? k_operand8(x.x, x.y, magic8, sel_even, sel_odd)
                                           : k_operand8(x.z, x.w, magic8, sel_even, sel_odd);
                    } else {
                        const uint4 x = kcur[blk][uu / 4];
                        const uint32_t w = (uu % 4 == 0) ? x.x : (uu % 4 == 1) ? x.y : (uu % 4 == 2) ? x.z : x.w;
                        ka = k_operand_sub(w, m_fine);
                    }
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qhi[uu], sacc, 0, 0, 0);
                    if constexpr (Q32)
                        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qlo[uu], sacc, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 f = fac[4 * blk + i];
                    const float sg = fmaf(f.x, sacc[i], fmaf(f.y, qsum, -m_part));
                    sc[4 * blk + i] = GV ? sg + dpp_f<0x128>(sg) : group_sum<NG>(sg);  // row_ror:8
                }
            }
            if (t0 + TS * TILE * ti + TILE > t1) {  // uniform: the chunk's last tiles
                asm volatile("" ::: "memory");  // keep this a branch
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = t0 + TS * TILE * ti + 16 * (i >> 2) + 4 * q4 + (i & 3);
                    sc[i] = r <= last ? sc[i] : -INFINITY;
                }
            }
            const float mx = max3_raw(max3_raw(sc[0], sc[1], sc[2]), max3_raw(sc[3], sc[4], sc[5]),
                                      max_raw(sc[6], sc[7]));
            m_top = max_raw(m_top, mx);

            // ---- online softmax across tiles. The scores are relative to the
            // head's reference m_run, which is raised only when a score
            // exceeds it, and then to that maximum plus kHeadroom: every
            // weight exp2(s - m_run) stays <= 1, the small rises of the
            // running maximum over most later tiles cost nothing, and only
            // the first tile and the rare raise take this branch (the first
            // sets the reference from its own maximum).
            if (ti == 0 || __builtin_amdgcn_ballot_w64(mx > 0.0f) != 0) {
                const float full = xrow_max(mx, -INFINITY);  // the head's tile maximum
                const bool raise = full > 0.0f || (ti == 0 && full > -INFINITY);
                const float delta = raise ? full + kHeadroom : 0.0f;
                m_run += delta;
                m_part = m_run * (1.0f / NG);
                m_top -= delta;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    sc[i] -= delta;
                if (ti != 0) {
                    const float corr = __builtin_amdgcn_exp2f(-delta);
                    l_run *= corr;
                    b_run *= corr;
                    float4v corr_row;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        corr_row[i] = __shfl(corr, GV ? 4 * q4 + i : (4 * q4 + i) & 7);  // lo row r: column r - 8
                    mfma_result_wait();
#pragma unroll
                    for (int s2 = 0; s2 < VS; ++s2)
#pragma unroll
                        for (int m = 0; m < VM; ++m)
                            scale_in_place(acc[s2][m], corr_row);
                }
            }

            // ---- weights p * s_v as hi + lo fp16 halves, and the bias term
            half8 phi, plo;
            float lsum = 0.0f, bsum = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                const float p0 = __builtin_amdgcn_exp2f(sc[j]);
                const float p1 = __builtin_amdgcn_exp2f(sc[j + 1]);
                lsum += p0 + p1;
                bsum = fmaf(p0, fac[j].w, fmaf(p1, fac[j + 1].w, bsum));
                const float w0 = p0 * fac[j].z, w1 = p1 * fac[j + 1].z;
                // any rounding of hi works: lo = w - hi is exact in fp32; the
                // lo halves have operand rows of their own and are kept as
                // lo * kLoScale, above the fp16 subnormal range
                const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(w0, w1));
                const half2v l = __builtin_bit_cast(
                    half2v, __builtin_amdgcn_cvt_pkrtz((w0 - (float)h[0]) * LS, (w1 - (float)h[1]) * LS));
                phi[j] = h[0]; phi[j + 1] = h[1];
                plo[j] = l[0]; plo[j + 1] = l[1];
            }
            l_run += lsum;
            b_run += bsum;
            // the operand rows of the other layouts: lanes 8-15 of each row
            // of 16 (columns without a query head) take the lo halves of
            // lanes 0-7
            half8 alr;
            if constexpr (!GV) {
                const u32x4 H = __builtin_bit_cast(u32x4, phi), L = __builtin_bit_cast(u32x4, plo);
                u32x4 A;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    A[r] = take_half_row<0xC>(H[r], L[r]);
                alr = __builtin_bit_cast(half8, A);
            }
            if constexpr (GV) {
                // Group-aligned value products: row h + 8 e of group g's
                // value operand is the hi (e = 0) or lo (e = 1) half of head
                // h's weights for group g. The lane of column h + 8 g holds
                // both halves for group g, so group 0's operand takes the lo
                // half into lanes 8-15 of each row and group 1's the hi half
                // into lanes 0-7, each with one DPP move per register.
                const u32x4 H = __builtin_bit_cast(u32x4, phi), L = __builtin_bit_cast(u32x4, plo);
                u32x4 A0, A1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t h = H[r], lo = L[r];
                    A0[r] = take_half_row<0xC>(h, lo);
                    A1[r] = take_half_row<0x3>(lo, h);
                }
                const half8 a0 = __builtin_bit_cast(half8, A0), a1 = __builtin_bit_cast(half8, A1);
                // A lane of column col < 8 holds a group-0 V word, col >= 8 a
                // group-1 word; in group g's products a lane whose word is in
                // g gives its dimensions 0..3, the others dimensions 4..7 of
                // the word of lane l ^ 8 (see the store)
                if constexpr (B8) {
                    // the same exchange on whole words: row r's words hold
                    // dimensions 0..3 and 4..7 of the lane's eight; rows
                    // (2jp, 2jp + 1) meet byte by byte in each operand pair
                    uint32_t bx[2][8];
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        bx[0][r] = take_half_row<0xC>(vcur[0][2 * r], vcur[0][2 * r + 1]);
                        bx[1][r] = take_half_row<0x3>(vcur[0][2 * r], vcur[0][2 * r + 1]);
                    }
#pragma unroll
                    for (int g = 0; g < 2; ++g)
#pragma unroll
                        for (int mm = 0; mm < 4; ++mm) {
                            half2v e[4];
#pragma unroll
                            for (int jp = 0; jp < 4; ++jp)
                                e[jp] = v_pair8(bx[g][2 * jp], bx[g][2 * jp + 1], sel_b[mm], magic16);
                            const half8 bv = cat8(e[0], e[1], e[2], e[3]);
                            acc[0][4 * g + mm] =
                                __builtin_amdgcn_mfma_f32_16x16x32_f16(g ? a1 : a0, bv, acc[0][4 * g + mm], 0, 0, 0);
                        }
                } else {
                    uint32_t bx[2][4];
#pragma unroll
                    for (int jp = 0; jp < 4; ++jp) {
                        const uint32_t xw = __builtin_amdgcn_perm(vcur[0][2 * jp + 1], vcur[0][2 * jp], 0x05040100u);
                        const uint32_t yw = __builtin_amdgcn_perm(vcur[0][2 * jp + 1], vcur[0][2 * jp], 0x07060302u);
                        bx[0][jp] = take_half_row<0xC>(xw, yw);
                        bx[1][jp] = take_half_row<0x3>(xw, yw);
                    }
#pragma unroll
                    for (int g = 0; g < 2; ++g)
#pragma unroll
                        for (int mm = 0; mm < 4; ++mm) {
                            half2v e[4];
#pragma unroll
                            for (int jp = 0; jp < 4; ++jp)
                                e[jp] = unpack.one(bx[g][jp], mm);
                            const half8 bv = cat8(e[0], e[1], e[2], e[3]);
                            acc[0][4 * g + mm] =
                                __builtin_amdgcn_mfma_f32_16x16x32_f16(g ? a1 : a0, bv, acc[0][4 * g + mm], 0, 0, 0);
                        }
                }
            } else {
#pragma unroll
                for (int s2 = 0; s2 < VS; ++s2) {
                    if constexpr (HV) {
                        // dimension m of the column's half octet in rows (2jp,
                        // 2jp + 1): byte m of their words (8-bit codes), or
                        // nibble m of the two bytes the lane's half selects
                        uint32_t xw[4];
                        const uint32_t hsel = (col >> 3) ? 0x07060302u : 0x05040100u;
#pragma unroll
                        for (int jp = 0; jp < 4; ++jp)
                            xw[jp] = B8 ? 0u : __builtin_amdgcn_perm(vcur[s2][2 * jp + 1], vcur[s2][2 * jp], hsel);
#pragma unroll
                        for (int m = 0; m < VM; ++m) {
                            half2v e[4];
#pragma unroll
                            for (int jp = 0; jp < 4; ++jp) {
                                if constexpr (B8)
                                    e[jp] = v_pair8(vcur[s2][2 * jp], vcur[s2][2 * jp + 1], sel_b[m], magic16);
                                else
                                    e[jp] = unpack.one(xw[jp], m);
                            }
                            const half8 bv = cat8(e[0], e[1], e[2], e[3]);
                            acc[s2][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alr, bv, acc[s2][m], 0, 0, 0);
                        }
                    } else if constexpr (B8) {
                        // column dimension m of rows (2jp, 2jp + 1): byte m & 3
                        // of their first (m < 4) or second word
#pragma unroll
                        for (int m = 0; m < 8; ++m) {
                            half2v e[4];
#pragma unroll
                            for (int jp = 0; jp < 4; ++jp)
                                e[jp] = v_pair8(vcur[s2][4 * jp + (m >> 2)], vcur[s2][4 * jp + 2 + (m >> 2)],
                                                sel_b[m & 3], magic16);
                            const half8 bv = cat8(e[0], e[1], e[2], e[3]);
                            acc[s2][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alr, bv, acc[s2][m], 0, 0, 0);
                        }
                    } else {
                        // rows (2jp, 2jp + 1) interleaved nibble-pair by nibble-pair:
                        // xw holds dimensions 8col + 0..3, yw dimensions 8col + 4..7
                        uint32_t xw[4], yw[4];
#pragma unroll
                        for (int jp = 0; jp < 4; ++jp) {
                            xw[jp] = __builtin_amdgcn_perm(vcur[s2][2 * jp + 1], vcur[s2][2 * jp], 0x05040100u);
                            yw[jp] = __builtin_amdgcn_perm(vcur[s2][2 * jp + 1], vcur[s2][2 * jp], 0x07060302u);
                        }
#pragma unroll
                        for (int m = 0; m < 8; ++m) {
                            half2v e[4];
#pragma unroll
                            for (int jp = 0; jp < 4; ++jp)
                                e[jp] = unpack.one(m < 4 ? xw[jp] : yw[jp], m & 3);
                            const half8 bv = cat8(e[0], e[1], e[2], e[3]);
                            acc[s2][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alr, bv, acc[s2][m], 0, 0, 0);
                        }
                    }
                }
            }

            // ---- refill this ring slot, then the next tile's factors
            load_tile(ti + PF, kbuf[u], vbuf[u], mbuf[u]);
            stage_meta(slot ^ 1, mbuf[(u + 1) % PF]);
        }
    }

    // ---- this wavefront's state against the head's true maximum: the
    // weights so far are relative to m_run, and the largest of them is
    // exp2(top) with top in [-kHeadroom, 0], so l and the products are
    // multiplied by exp2(-top) (a factor in [1, 2^kHeadroom]) and the state's
    // maximum is m = m_run + top. emit() stores it through m_at(h) (m in
    // units of m_unit per log2 unit, then l) and acc_at(h) (the D value sums)
    // for the query heads h of this KV head.
    const float top = xrow_max(m_top, -INFINITY);
    const float renorm = __builtin_amdgcn_exp2f(-top);
    const float l_tot = xrow_sum(l_run) * renorm;
    const float b_tot = xrow_sum(b_run) * renorm;
    auto emit = [&](auto m_at, auto l_at, auto acc_at, float m_unit) {
        if (q4 == 0 && col_on && gl == 0) {
            *m_at(hl) = (m_run + top) * m_unit;
            *l_at(hl) = l_tot;
        }
        if constexpr (GV) {
            // Row i = h + 8 e of the value products sits in lanes of q4 =
            // i / 4: lanes l < 32 hold the hi rows, lanes l ^ 32 the lo rows
            // (scaled by kLoScale) of the same heads 4 (q4 & 1) + r. One swap
            // of lanes 32-63 of group 0's value with lanes 0-31 of group 1's
            // leaves (hi, lo) of group 0 in lanes 0-31 and of group 1 in
            // lanes 32-63, so that hi + lo / kLoScale is group g = q4 / 2.
            // Group g's products of this lane are dimensions 8 col + 0..3
            // when its own V word is in group g, else 8 (col ^ 8) + 4..7.
            const int g = q4 >> 1;
            const int d0 = (g == (low8 ? 0 : 1)) ? 8 * col : 8 * (col ^ 8) + 4;
            float o[4][4];  // [r][mm]
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // (elements go through scalars: a bit cast of a vector
                    // element in place reads element 0)
                    const float e0 = acc[0][mm][r], e1 = acc[0][4 + mm][r];
                    const uint32_t a0 = __builtin_bit_cast(uint32_t, e0);
                    const uint32_t a1 = __builtin_bit_cast(uint32_t, e1);
                    // the swap leaves lanes 0-31 of both operands (the hi
                    // rows) in the first result and lanes 32-63 (the lo rows)
                    // in the second
                    const auto sw = __builtin_amdgcn_permlane32_swap(a0, a1, false, false);
                    const uint32_t x = sw[0], y = sw[1];
                    o[r][mm] = fmaf(__builtin_bit_cast(float, y), VU / kLoScale, __builtin_bit_cast(float, x) * VU);
                }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int h = 4 * (q4 & 1) + r;
                const float bias = __shfl(b_tot, h + 8 * g);
                const float f = __shfl(renorm, h + 8 * g);
                if (h < nrep)
                    *reinterpret_cast<float4 *>(acc_at(h) + d0) =
                        make_float4(fmaf(o[r][0], f, bias), fmaf(o[r][1], f, bias), fmaf(o[r][2], f, bias),
                                    fmaf(o[r][3], f, bias));
            }
        } else {
            // Rows 0-7 of the value products (the hi weight halves of columns
            // 0-7) sit in lanes q4 < 2, rows 8-15 (their lo halves times
            // kLoScale) in lanes l + 32: a swap of the upper and lower 32
            // lanes of a register with itself gives lanes l < 32 both, and
            // there column rr = 4 q4 + i holds hi + lo / kLoScale.
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 4 * q4 + i;
                const float bias_r = __shfl(b_tot, rr);
                const float f = __shfl(renorm, rr);
                float o[VS][VM];
#pragma unroll
                for (int s = 0; s < VS; ++s)
#pragma unroll
                    for (int m = 0; m < VM; ++m) {
                        const float e = acc[s][m][i];
                        const uint32_t x = __builtin_bit_cast(uint32_t, e);
                        const auto sw = __builtin_amdgcn_permlane32_swap(x, x, false, false);
                        // (through scalars: a bit cast of a vector element in place reads element 0)
                        const uint32_t own = sw[0], lo = sw[1];
                        o[s][m] = fmaf(__builtin_bit_cast(float, lo), 1.0f / kLoScale, __builtin_bit_cast(float, own));
                    }
                if (rr < R) {  // R <= 8: lanes q4 < 2
                    const int h = rr / NG, g = rr % NG;
                    float *dst = acc_at(h);
                    const float fu = f * VU;
                    if constexpr (HV) {
                        const int oct = col & 7;  // the column's octet, dimensions 4 (col >> 3) .. + 3 of it
                        if (oct / WPG == g)
                            *reinterpret_cast<float4 *>(dst + 8 * oct + 4 * (col >> 3)) =
                                make_float4(fmaf(o[0][0], fu, bias_r), fmaf(o[0][1], fu, bias_r),
                                            fmaf(o[0][2], fu, bias_r), fmaf(o[0][3], fu, bias_r));
                    } else {
#pragma unroll
                        for (int s = 0; s < VS; ++s) {
                            const int word = 16 * s + col;
                            if (word / WPG == g) {
                                float4 lo = {fmaf(o[s][0], fu, bias_r), fmaf(o[s][1], fu, bias_r),
                                             fmaf(o[s][2], fu, bias_r), fmaf(o[s][3], fu, bias_r)};
                                float4 hi = {fmaf(o[s][4], fu, bias_r), fmaf(o[s][5], fu, bias_r),
                                             fmaf(o[s][6], fu, bias_r), fmaf(o[s][7], fu, bias_r)};
                                *reinterpret_cast<float4 *>(dst + 8 * word) = lo;
                                *reinterpret_cast<float4 *>(dst + 8 * word + 4) = hi;
                            }
                        }
                    }
                }
            }
        }
    };

    if constexpr (WG == 1) {
        // the split-K partial state of chunk c (m in natural-log units)
        const int64_t C = a.num_chunks;
        const int64_t o = ((int64_t)b * a.Hq + h0) * C + c;
        emit([&](int h) { return a.part_m + o + h * C; }, [&](int h) { return a.part_l + o + h * C; },
             [&](int h) { return a.part_acc + (o + h * C) * D; }, kLn2);
    } else {
        // the wavefront's state into LDS (m in log2 units), then the merges
        constexpr int MAXH = 16 / NG;
        __shared__ __align__(16) float mg_ml[WG][MAXH][2];
        __shared__ __align__(16) float mg_acc[WG][MAXH][D];
        if (ntile <= 0) {  // uniform: a wavefront past the last row holds no state
            for (int e = lane; e < nrep * D; e += 64)
                mg_acc[wave][e / D][e % D] = 0.0f;
            if (lane < nrep) {
                mg_ml[wave][lane][0] = -INFINITY;
                mg_ml[wave][lane][1] = 0.0f;
            }
        } else {
            emit([&](int h) { return &mg_ml[wave][h][0]; }, [&](int h) { return &mg_ml[wave][h][1]; },
                 [&](int h) { return &mg_acc[wave][h][0]; }, 1.0f);
        }
        merge_epilogue<D, NG, WG>(a, (int64_t)b * gridDim.y + blockIdx.y, (int64_t)b * a.Hq + h0, nrep,
                                  &mg_ml[0][0][0], &mg_acc[0][0][0]);
    }
}

// Score columns of one grid row: at most 16, and at most 8 for the
// one-wavefront kernel's layouts other than D = 128 with two scale groups.
template <int D, int NG>
bool block_fits(const PartialArgs &a, bool one_wave)
{
    const int R = a.n_rep / a.head_split * NG;
    return a.head_split >= 1 && a.n_rep % a.head_split == 0 &&
           R <= ((one_wave && !(D == 128 && NG == 2)) ? 8 : 16);
}

// Tiles in flight per wavefront (even: the scale/bias ring has two slots):
// two. With 2048 wavefronts at 128K that is 19 MB of int4 tiles requested at
// the start; four (38 MB) measured 6% slower at 128K and 10% at 64K
// (presumably because each wavefront's first tile then queues behind more of
// the others' requests). At D = 64, whose tiles are half as many bytes, four
// and six measured 7% and 19% slower at 128K.
template <int D>
constexpr int ring_depth() { return 2; }

template <int D, int NG, bool Q32, int BITS>
void launch_one_wave(const PartialArgs &a, dim3 grid, const Launch &l)
{
    constexpr int PF = ring_depth<D>();
    hipExtLaunchKernelGGL((sdpa_partial_mfma1_kernel<D, NG, Q32, PF, BITS>), grid, dim3(64), 0, l.s, l.start, l.stop,
                          0, a);
}

// The one-wavefront kernel needs chunks of at most 512 rows (its scale and
// bias arrive as one 2-byte load per (row, group) and array, so any capacity
// and chunk length will do); it pays off once there are enough (chunk, head)
// items to give every SIMD two wavefronts.
bool one_wave_fits(const PartialArgs &a, int D, int batch)
{
    (void)D;
    (void)batch;
    return a.chunk <= CH1;
}

// 8-bit caches and D = 64: the one-wavefront kernel only
template <int D, int NG>
hipError_t launch_dg_wave(const PartialArgs &a, int q_dtype, int batch, int variant, const Launch &l)
{
    dim3 grid((unsigned)a.num_chunks, (unsigned)(a.Hkv * a.head_split), (unsigned)batch);
    if ((variant != KVQ_KERNEL_AUTO && variant != KVQ_KERNEL_MFMA && variant != KVQ_KERNEL_MFMA_WAVE) ||
        !one_wave_fits(a, D, batch) || !block_fits<D, NG>(a, true))
        return hipErrorInvalidValue;
    if (a.bits == 8) {
        if (q_dtype == KVQ_F32)
            launch_one_wave<D, NG, true, 8>(a, grid, l);
        else
            launch_one_wave<D, NG, false, 8>(a, grid, l);
    } else {
        if (q_dtype == KVQ_F32)
            launch_one_wave<D, NG, true, 4>(a, grid, l);
        else
            launch_one_wave<D, NG, false, 4>(a, grid, l);
    }
    return hipGetLastError();
}

template <int D, int NG>
hipError_t launch_dg(const PartialArgs &a, int q_dtype, int batch, int variant, const Launch &l)
{
    if constexpr (D == 64) {
        return launch_dg_wave<D, NG>(a, q_dtype, batch, variant, l);
    } else {
        if (a.bits == 8)
            return launch_dg_wave<D, NG>(a, q_dtype, batch, variant, l);
        dim3 grid((unsigned)a.num_chunks, (unsigned)(a.Hkv * a.head_split), (unsigned)batch);
        const int64_t items = (int64_t)a.num_chunks * a.Hkv * a.head_split * batch;
        bool one = variant == KVQ_KERNEL_MFMA_WAVE;
        if (variant == KVQ_KERNEL_MFMA || variant == KVQ_KERNEL_AUTO)
            one = one_wave_fits(a, D, batch) && items >= kOneWaveItems;
        if ((one && !one_wave_fits(a, D, batch)) || !block_fits<D, NG>(a, one))
            return hipErrorInvalidValue;
        if (one) {
            if (q_dtype == KVQ_F32)
                launch_one_wave<D, NG, true, 4>(a, grid, l);
            else
                launch_one_wave<D, NG, false, 4>(a, grid, l);
        } else if (q_dtype == KVQ_F32) {
            hipExtLaunchKernelGGL((sdpa_partial_mfma_kernel<D, NG, true>), grid, dim3(NT), 0, l.s, l.start, l.stop, 0,
                                  a);
        } else {
            hipExtLaunchKernelGGL((sdpa_partial_mfma_kernel<D, NG, false>), grid, dim3(NT), 0, l.s, l.start, l.stop, 0,
                                  a);
        }
        return hipGetLastError();
    }
}

}  // namespace

// Query-head blocks per KV head for the matrix-core kernels: a block is the
// largest divisor of n_rep whose (head, group) columns fit the score columns
// of one block: the 16 of one score instruction at D = 128 with two scale
// groups, 8 elsewhere (the one-wavefront kernel's value products there take
// the lo weight halves as operand rows 8-15); 0 when no matrix-core kernel
// takes the shape.
int mfma_head_split(int D, int G, int n_rep)
{
    if (D != 64 && D != 128 && D != 256)
        return 0;
    if ((G != 32 && G != 64 && G != 128) || G > D)
        return 0;
    const int NG = D / G;
    if (NG > 4 || n_rep < 1)
        return 0;
    const int cols = (D == 128 && NG == 2) ? 16 : 8;
    for (int nsub = cols / NG; nsub >= 1; --nsub)
        if (n_rep % nsub == 0)
            return n_rep / nsub;
    return 0;
}

bool mfma_supports(int D, int G, int n_rep, int chunk)
{
    (void)chunk;
    return mfma_head_split(D, G, n_rep) > 0;
}

hipError_t launch_partial_mfma(const PartialArgs &a, int D, int q_dtype, int batch, int variant, const Launch &l)
{
    if (a.bits != 4 && a.bits != 8)
        return hipErrorInvalidValue;
    const int NG = D / a.G;
    if (D == 64) {
        if (NG == 1) return launch_dg<64, 1>(a, q_dtype, batch, variant, l);
        if (NG == 2) return launch_dg<64, 2>(a, q_dtype, batch, variant, l);
    } else if (D == 128) {
        if (NG == 1) return launch_dg<128, 1>(a, q_dtype, batch, variant, l);
        if (NG == 2) return launch_dg<128, 2>(a, q_dtype, batch, variant, l);
        if (NG == 4) return launch_dg<128, 4>(a, q_dtype, batch, variant, l);
    } else if (D == 256) {
        if (NG == 2) return launch_dg<256, 2>(a, q_dtype, batch, variant, l);
        if (NG == 4) return launch_dg<256, 4>(a, q_dtype, batch, variant, l);
    }
    return hipErrorInvalidValue;
}

bool mfma_one_wave_ok(const PartialArgs &a, int D, int batch) { return one_wave_fits(a, D, batch); }


hipError_t launch_decode_fused(const PartialArgs &a, int D, int q_dtype, int batch, const Launch &l)
{
    if (!one_wave_fits(a, D, batch) || a.append_row < 0)
        return hipErrorInvalidValue;
    return launch_partial_mfma(a, D, q_dtype, batch, KVQ_KERNEL_MFMA_WAVE, l);
}

// Single-launch decode step. Workgroups of WG wavefronts (two per SIMD of
// one CU at D = 128, one at D = 256), each wavefront streaming `rows` rows;
// rows is the largest power of two from 512 down to 512 / WG that still
// gives as many wavefronts as the 256-CU chip holds at once (two per SIMD at
// D = 128: at 64K rows of the Llama layer 256 rows; one per SIMD at D = 256,
// whose kernel takes more than half a SIMD's registers), so short contexts
// trade longer streams for more of them, and no context runs in two rounds
// where one would do.
constexpr int64_t kSingleWaves = 2048;

template <int D>
constexpr int single_wg() { return D <= 128 ? 8 : 4; }

bool decode_single_plan(int D, int G, int n_rep, int bits, int64_t skv, int64_t heads, int32_t &rows, int32_t &nwg)
{
    if (!mfma_supports(D, G, n_rep, 512) || (bits != 4 && bits != 8) || skv < 1 || heads < 1)
        return false;
    heads *= mfma_head_split(D, G, n_rep);  // workgroup rows: (batch, KV head, query-head block)
    // rows per wavefront: halved from 512 while the grid has fewer than
    // kSingleWaves wavefronts, down to 512 / WG (a workgroup then still
    // covers 512 rows: at most one partial per 512 rows, the workspace's
    // count)
    const int wg = D <= 128 ? single_wg<128>() : single_wg<256>();
    int r = 512;
    const int64_t waves = D <= 128 ? kSingleWaves : kSingleWaves / 2;
    while (r > 512 / wg && heads * ((skv + r - 1) / r) < waves)
        r /= 2;
    const int64_t n = (skv + (int64_t)wg * r - 1) / ((int64_t)wg * r);
    if (n > kMaxMergeGroups)
        return false;
    rows = r;
    nwg = (int32_t)n;
    return true;
}

template <int D, int NG, bool Q32, int BITS>
void launch_single(const PartialArgs &a, dim3 grid, const Launch &l)
{
    constexpr int WG = single_wg<D>();
    hipExtLaunchKernelGGL((sdpa_partial_mfma1_kernel<D, NG, Q32, ring_depth<D>(), BITS, WG>), grid, dim3(64 * WG), 0,
                          l.s, l.start, l.stop, 0, a);
}

template <int D, int NG>
hipError_t launch_single_dg(const PartialArgs &a, int q_dtype, int batch, const Launch &l)
{
    const dim3 grid((unsigned)a.nwg, (unsigned)(a.Hkv * a.head_split), (unsigned)batch);
    if (!block_fits<D, NG>(a, true))
        return hipErrorInvalidValue;
    if (a.bits == 8) {
        if (q_dtype == KVQ_F32)
            launch_single<D, NG, true, 8>(a, grid, l);
        else
            launch_single<D, NG, false, 8>(a, grid, l);
    } else {
        if (q_dtype == KVQ_F32)
            launch_single<D, NG, true, 4>(a, grid, l);
        else
            launch_single<D, NG, false, 4>(a, grid, l);
    }
    return hipGetLastError();
}

hipError_t launch_decode_single(const PartialArgs &a, int D, int q_dtype, int batch, const Launch &l)
{
    // the merge inside the launch needs its workspace and the output; split-K
    // partials (part_acc set) go to the reduce launched after this kernel
    if (a.nwg < 1 || a.chunk > CH1 || (!a.part_acc && (!a.merge_ws || !a.counters || !a.out)))
        return hipErrorInvalidValue;
    const int NG = D / a.G;
    if (D == 64) {
        if (NG == 1) return launch_single_dg<64, 1>(a, q_dtype, batch, l);
        if (NG == 2) return launch_single_dg<64, 2>(a, q_dtype, batch, l);
    } else if (D == 128) {
        if (NG == 1) return launch_single_dg<128, 1>(a, q_dtype, batch, l);
        if (NG == 2) return launch_single_dg<128, 2>(a, q_dtype, batch, l);
        if (NG == 4) return launch_single_dg<128, 4>(a, q_dtype, batch, l);
    } else if (D == 256) {
        if (NG == 2) return launch_single_dg<256, 2>(a, q_dtype, batch, l);
        if (NG == 4) return launch_single_dg<256, 4>(a, q_dtype, batch, l);
    }
    return hipErrorInvalidValue;
}

}  // namespace kvq
