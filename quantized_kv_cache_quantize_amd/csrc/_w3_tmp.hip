// Prefill-side attention over the int4 cache, matrix-core kernel for gfx950.
//
// The README's hybrid paragraph routes Sq > 1 (prefill) to a separate
// attention on fp16 K/V and only then quantises the rows into the cache; here
// the prefill block's queries read the quantised cache directly, the same
// packed rows the decode kernel reads. Query i of the block is position
// q_start + i; its K/V row is cache row q_start + i (appended before the
// call), and it attends to rows [0, q_start + i] (causal).
//
// Work split: a wavefront takes 32 / n_rep query positions x the n_rep heads
// of a KV head (32 query columns: two blocks of 16, each the N side of its
// own matrix instructions) and streams the rows its positions can see in
// 32-row tiles. With GQA the n_rep heads of a KV head and the block's
// positions all read the same rows, so every K/V tile is fetched and
// unpacked once for all the columns of a wavefront (and, in the int4 D = 128
// kernel, once for the four wavefronts of a workgroup).
//
// Scores (per tile): S^T[t][c] = Kcodes[t][:] . Q[c][:] on
// v_mfma_f32_16x16x32_f16, A = K codes (16 rows, 32 dimensions), B = the
// queries of a 16-column block. A lane loads the K words of its row strided
// by 4 words, so each instruction's 32 dimensions lie in one scale group and
// the group's scale applies in fp32 afterwards (the factored form of the
// Gemma page's "What I Built Instead"): s = sum_g s_g (q . code)_g +
// b_g (sum q)_g.
//
// Softmax: per query column, relative to a reference raised (with headroom)
// only when a score exceeds it, as in the decode kernel; the output is
// normalised in the kernel (no split over rows, so no partial state).
//
// Four kernels: 8-bit codes (sdpa_prefill_b8_kernel: per-group value
// weights, the layout the int4 kernels started from; sdpa_prefill_b8_wg_kernel
// at D = 128 with n_rep <= 16, the same arithmetic with one block of query
// columns per wavefront and the tile's operands shared by a workgroup), int4
// at D = 256 (sdpa_prefill_i4_kernel) and int4 at D = 64 and 128
// (sdpa_prefill_i4_wg_kernel, the tile's operands shared by a workgroup).

#include "kvq_internal.h"
#include "mfma_common.h"

namespace kvq {
namespace {

constexpr int PT = 32;  // rows per tile

// Workgroup order. A launch is one row of (position blocks x Hkv) workgroups
// per batch entry, dispatched in index order, consecutive workgroups going to
// the chip's eight XCDs in turn. The KV head varies fastest, so that with
// Hkv a multiple of 8 all workgroups of a head run on one XCD and share its
// L2 for the head's K/V rows; the position blocks come last first, so that
// under the causal mask the workgroups with the most rows start first and the
// short ones fill the end.
__device__ __forceinline__ int prefill_head(const PrefillArgs &a) { return (int)(blockIdx.x % (unsigned)a.Hkv); }
__device__ __forceinline__ int prefill_block(const PrefillArgs &a)
{
    return (int)(gridDim.x / (unsigned)a.Hkv) - 1 - (int)(blockIdx.x / (unsigned)a.Hkv);
}

// 8-bit codes (four per word). NB blocks of 16 query columns per wavefront
// (every unpacked K and V operand feeds NB matrix instructions), PF tiles in
// flight; operands are unpacked right before the instruction that reads them
// and the scale/bias factors read from LDS where they are used. NB = 2 runs
// one wavefront per SIMD with its query operands in LDS (read back every
// tile) to ease the register pressure (one block: 35.8 ms against 28.8 ms on
// the Llama layer's 4096-position chunk at row 61440).
//
// The K and V codes enter as the exact centred integers n - 128 through the
// byte permutes of the decode kernel (k_operand8, v_pair8); the value
// weights p * s_v of each scale group are hi and lo fp16 halves (lo scaled
// by 2^11) in separate accumulators, carried times WS = 2^6 (as in the
// decode kernel, to keep their fp16 halves clear of the subnormal range),
// and the value products are multiplied by VU = 1 / WS at the end.
//
// Q32 (fp32 queries, e.g. a query rotated for a Hadamard-rotated cache): the
// query is split into fp16 hi and lo halves, hi + lo exact to 22 bits, each
// the B operand of its own score product (as in the decode kernel).
//
// D = 256 (four scale groups): the value words of a row come in VS = D / 128
// sets of 32 words, each set two scale groups handled as the D = 128 layout
// handles its two; NB = 1 there (the accumulators of one block already take
// what two blocks take at D = 128).
template <int PF, int NB, bool Q32, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1)))
void sdpa_prefill_b8_kernel(PrefillArgs a)
{
    constexpr int NG = D / 64;   // scale groups of 64
    // D = 64: one group of 16 words per row; each of the 16 value columns is
    // one word (octet col & 7, dimensions 4 (col >> 3) + mm, mm < 4);
    // otherwise a column is an octet (two words), two groups per set
    constexpr bool HV = D == 64;
    constexpr int VS = HV ? 1 : D / 128;  // sets of 16 value columns
    constexpr int VM = HV ? 4 : 8;        // value accumulators per set
    constexpr int W = D / 4;    // words per row
    constexpr int KW = 2;       // words per eight dimensions
    constexpr int KM = D / 32;        // score products per 16-row block
    constexpr int KPG = KM / NG;      // of them per scale group
    constexpr float VC = 128.0f;       // centre of the value codes
    constexpr float WS = 64.0f;        // scale of the value weights
    constexpr float VU = 1.0f / 64.0f;  // unit of the value products
    constexpr int PAIRS = PT * NG;
    constexpr int MP = (PAIRS + 63) / 64;  // (row, group) pairs per lane (D = 64: lanes 0-31)
    static_assert(PAIRS % 64 == 0 || PAIRS == 32, "whole pairs per lane, or one for half the lanes");
    constexpr bool QLDS = NB > 1 || D > 128;  // query operands in LDS

    const int lane = threadIdx.x;
    const int q4 = lane >> 4;
    const int col = lane & 15;
    const int kvh = prefill_head(a);
    const int b = blockIdx.z;
    const int nrep = a.n_rep;
    const int p0 = prefill_block(a) * a.pb;        // first position of the block
    const int npos = min(a.pb, a.sq - p0);         // positions in this block
    const int t_end = (int)a.q_start + p0 + npos;  // rows [0, t_end) are read
    const int t_all = (int)a.q_start + p0;         // rows <= t_all are seen by every column
    const int ntile = (t_end + PT - 1) / PT;
    const int64_t kvrow0 = ((int64_t)b * a.Hkv + kvh) * a.cap;
    const bool low8 = (lane & 8) == 0;             // this lane's V word is in group 0

    // column 16 nb + col of the wavefront: position (16 nb + col) / nrep,
    // head (16 nb + col) % nrep (inactive columns compute on zero queries and
    // are never stored)
    int cpos[NB], chead[NB];
    bool con[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int cc = 16 * nb + col;
        cpos[nb] = cc / nrep;
        chead[nb] = cc % nrep;
        con[nb] = cc < a.pb * nrep && cpos[nb] < npos;
    }

    const uint32_t rows_ok = (uint32_t)t_end;
    const __amdgpu_buffer_rsrc_t kq = make_rsrc(a.k_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t vq = make_rsrc(a.v_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t mres[4] = {
        make_rsrc(a.k_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.k_bias + kvrow0 * NG, rows_ok * NG * 2u),
        make_rsrc(a.v_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.v_bias + kvrow0 * NG, rows_ok * NG * 2u)};

    // fp32 factors per (row, group) of a tile, two-slot LDS ring
    // (c = softmax scale * log2 e):
    //   x = s_k c 2^20 (int4: the subnormal scale of the K operands) or s_k c
    //   y = b_k c, or (b_k + 128 s_k) c (the bias of centred 8-bit codes)
    //   z = s_v WS, w = b_v + VC s_v
    __shared__ __align__(16) float4 mring[2][PAIRS];
    const float cs = a.score_scale;
    const float csk = cs;
    // the magic exponent bytes and the byte selectors of k_operand8 and v_pair8
    const uint32_t magic8 = opaque_s(kMagic1024x4), magic16 = opaque_s(0x64006400u);
    const uint32_t sel_even = opaque_s(0x04020400u), sel_odd = opaque_s(0x04030401u);
    const uint32_t sel_b[4] = {opaque_s(0x0C040C00u), opaque_s(0x0C050C01u), opaque_s(0x0C060C02u),
                               opaque_s(0x0C070C03u)};

    constexpr uint32_t kNoRows = 0x80000000u;  // > any records size (capacity * D < 2^31 bytes)
    uint32_t kbuf[PF][2][KM][KW];
    uint32_t vbuf[PF][VS][8 * KW];
    uint32_t mbuf[PF][MP][4];
    auto load_tile = [&](int ti, uint32_t (&kt)[2][KM][KW], uint32_t (&vt)[VS][8 * KW], uint32_t (&mt)[MP][4]) {
        const bool in = ti < ntile;
#pragma unroll
        for (int pp = 0; pp < MP; ++pp) {
            const uint32_t moff = in ? (uint32_t)((PT * ti) * NG + lane + 64 * pp) * 2u : kNoRows;
#pragma unroll
            for (int arr = 0; arr < 4; ++arr)
                mt[pp][arr] = __builtin_amdgcn_raw_buffer_load_b16(mres[arr], moff, 0, 0);
        }
        const uint32_t base = in ? (uint32_t)(PT * ti) * (uint32_t)(W * 4) : kNoRows;
        // K: row 16 blk + col, dimensions 32 uu + 8 q4 .. + 7 (the KW words
        // from word KW (4 uu + q4))
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const uint32_t off = base + (uint32_t)(((16 * blk + col) * W + KW * q4) * 4);
#pragma unroll
            for (int uu = 0; uu < KM; ++uu) {
                const auto x = __builtin_amdgcn_raw_buffer_load_b64(kq, off + 16 * KW * uu, 0, 0);
                kt[blk][uu][0] = x[0];
                kt[blk][uu][1] = x[1];
            }
        }
        // V: dimensions 128 s2 + 8 col .. + 7 (KW words) of rows 16 (j >> 2) + 4 q4 + (j & 3)
#pragma unroll
        for (int s2 = 0; s2 < VS; ++s2) {
            // HV: the one word of dimensions 8 (col & 7) + 4 (col >> 3) .. + 3
            const uint32_t voff =
                base + (uint32_t)((4 * q4 * W + (HV ? KW * (col & 7) + (col >> 3) : KW * (16 * s2 + col))) * 4);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t o = voff + ((16 * (j >> 2) + (j & 3)) * W) * 4;
                if constexpr (HV) {
                    vt[s2][j] = __builtin_amdgcn_raw_buffer_load_b32(vq, o, 0, 0);
                } else {
                    const auto x = __builtin_amdgcn_raw_buffer_load_b64(vq, o, 0, 0);
                    vt[s2][2 * j] = x[0];
                    vt[s2][2 * j + 1] = x[1];
                }
            }
        }
    };
    auto stage_meta = [&](int slot, const uint32_t (&mt)[MP][4]) {
#pragma unroll
        for (int pp = 0; pp < MP; ++pp) {
            if (PAIRS < 64 && lane + 64 * pp >= PAIRS)  // D = 64: lanes 32-63 loaded the next tile's words
                break;
            const float ks = h_val((uint16_t)mt[pp][0]);
            const float kb = h_val((uint16_t)mt[pp][1]);
            const float vs = h_val((uint16_t)mt[pp][2]);
            const float vb = h_val((uint16_t)mt[pp][3]);
            mring[slot][lane + 64 * pp] =
                make_float4(ks * csk, fmaf(128.0f, ks, kb) * cs, vs * WS, fmaf(VC, vs, vb));
        }
        asm volatile("" ::: "memory");
    };
    // factors (x, y) or (z, w) of row r, group g
    auto fac_xy = [&](int slot, int r, int g) {
        return *reinterpret_cast<const float2 *>(&mring[slot][r * NG + g]);
    };
    auto fac_zw = [&](int slot, int r, int g) {
        return *(reinterpret_cast<const float2 *>(&mring[slot][r * NG + g]) + 1);
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        load_tile(u, kbuf[u], vbuf[u], mbuf[u]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // each block's column query as B operands: score product uu holds
    // dimensions 32 uu + 8 q4 + kPerm[j] (kPerm8 for 8-bit codes); qsum:
    // group sums of exactly what the matrix core sees
    constexpr int QH = Q32 ? 2 : 1;  // query halves: hi (and lo)
    half8 qop[NB][QH][KM];
    float qsum[NB][NG];
    // NB > 1: the operands wait in LDS and are read back tile by tile, which
    // keeps the wavefront within 256 registers (see the kernel comment)
    __shared__ __align__(16) half8 q_lds[QLDS ? NB : 1][QH][KM][64];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t qrow = (((int64_t)b * a.Hq + kvh * nrep + (con[nb] ? chead[nb] : 0)) * a.sq + p0 +
                              (con[nb] ? cpos[nb] : 0)) * D;
        float gs[NG] = {};
#pragma unroll
        for (int uu = 0; uu < KM; ++uu) {
            float x[8];
            if constexpr (Q32) {
                const float *qp = reinterpret_cast<const float *>(a.q) + qrow + 32 * uu + 8 * q4;
                const float4 x0 = *reinterpret_cast<const float4 *>(qp);
                const float4 x1 = *reinterpret_cast<const float4 *>(qp + 4);
                x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
                x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
            } else {
                const half8 h8 = *reinterpret_cast<const half8 *>(reinterpret_cast<const _Float16 *>(a.q) + qrow +
                                                                  32 * uu + 8 * q4);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    x[j] = (float)h8[j];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xv = con[nb] ? x[kPerm8[j]] : 0.0f;
                const _Float16 hi = (_Float16)xv;
                qop[nb][0][uu][j] = hi;
                if constexpr (Q32) {
                    const _Float16 lo = (_Float16)(xv - (float)hi);
                    qop[nb][QH - 1][uu][j] = lo;
                    gs[uu / KPG] += (float)hi + (float)lo;
                } else {
                    gs[uu / KPG] += (float)hi;
                }
            }
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
            qsum[nb][g] = xrow_sum(gs[g]);
        if constexpr (QLDS) {
#pragma unroll
            for (int hl = 0; hl < QH; ++hl)
#pragma unroll
                for (int uu = 0; uu < KM; ++uu)
                    q_lds[nb][hl][uu][lane] = qop[nb][hl][uu];
        }
    }
    stage_meta(0, mbuf[0]);

    float m_run[NB], l_run[NB], b_run[NB][NG];
    float4v acc[NB][VM * VS], accl[NB][VM * VS];  // [nb][8 s2 + 4 g + mm]: hi and lo (x kLoScale) weight halves
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        m_run[nb] = 0.0f;
        l_run[nb] = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g)
            b_run[nb][g] = 0.0f;
#pragma unroll
        for (int m = 0; m < VM * VS; ++m) {
            acc[nb][m] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
            accl[nb][m] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
        }
    }

#pragma unroll 1
    for (int kk = 0; kk < ntile; kk += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int ti = kk + u;
            const int slot = u & 1;

            // ---- scores of the lane's 8 rows (4 q4 + i, 16 + 4 q4 + i - 4), log2 units,
            // for each block's column; every K operand serves all NB blocks
            float sc[NB][8];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                float s[NB][4];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        s[nb][i] = -m_run[nb];
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    float4v sacc[NB];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        sacc[nb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int k = 0; k < KPG; ++k) {
                        const uint32_t(&kw)[KW] = kbuf[u][blk][g * KPG + k];
                        const half8 ka = k_operand8(kw[0], kw[KW - 1], magic8, sel_even, sel_odd);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int hl = 0; hl < QH; ++hl) {
                                const half8 qb = QLDS ? q_lds[nb][hl][g * KPG + k][lane] : qop[nb][hl][g * KPG + k];
                                sacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb, sacc[nb], 0, 0, 0);
                            }
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float2 f = fac_xy(slot, 16 * blk + 4 * q4 + i, g);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            s[nb][i] = fmaf(f.x, sacc[nb][i], fmaf(f.y, qsum[nb][g], s[nb][i]));
                    }
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sc[nb][4 * blk + i] = s[nb][i];
            }
            if (PT * ti + PT - 1 > t_all) {  // uniform: some row is past some column's position
                asm volatile("" ::: "memory");  // keep this a branch
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int lim = t_all + cpos[nb];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int r = PT * ti + 16 * (i >> 2) + 4 * q4 + (i & 3);
                        sc[nb][i] = r <= lim ? sc[nb][i] : -INFINITY;
                    }
                }
            }
            float p[NB][8];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float mx = max3_raw(max3_raw(sc[nb][0], sc[nb][1], sc[nb][2]),
                                          max3_raw(sc[nb][3], sc[nb][4], sc[nb][5]), max_raw(sc[nb][6], sc[nb][7]));
                // ---- reference raised only when a score exceeds it (the first tile sets it)
                if (ti == 0 || __builtin_amdgcn_ballot_w64(mx > 0.0f) != 0) {
                    const float full = xrow_max(mx, -INFINITY);
                    const bool raise = full > 0.0f || (ti == 0 && full > -INFINITY);
                    const float delta = raise ? full + kHeadroom : 0.0f;
                    m_run[nb] += delta;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        sc[nb][i] -= delta;
                    if (ti != 0) {
                        const float corr = __builtin_amdgcn_exp2f(-delta);
                        l_run[nb] *= corr;
#pragma unroll
                        for (int g = 0; g < NG; ++g)
                            b_run[nb][g] *= corr;
                        float4v corr_row;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            corr_row[i] = __shfl(corr, 4 * q4 + i);
#pragma unroll
                        for (int m = 0; m < VM * VS; ++m) {
                            acc[nb][m] *= corr_row;
                            accl[nb][m] *= corr_row;
                        }
                    }
                }
                // ---- weights
                float lsum = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    p[nb][i] = __builtin_amdgcn_exp2f(sc[nb][i]);
                    lsum += p[nb][i];
                }
                l_run[nb] += lsum;
            }

            // ---- value products, group by group; the lane's eight dimensions
            // give 0..3 in its own group's products and lend 4..7 to lane
            // l ^ 8 (row r's two words hold dimensions 0..3 and 4..7), and
            // every unpacked operand serves all NB blocks
            if constexpr (HV) {
                // one scale group; rows (2 jp, 2 jp + 1) of the lane's word
                const uint32_t(&vw)[8 * KW] = vbuf[u][0];
                half8 phi[NB], plo[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    float bsum = 0.0f;
#pragma unroll
                    for (int j = 0; j < 8; j += 2) {
                        const float2 f0 = fac_zw(slot, 16 * (j >> 2) + 4 * q4 + (j & 3), 0);
                        const float2 f1 = fac_zw(slot, 16 * ((j + 1) >> 2) + 4 * q4 + ((j + 1) & 3), 0);
                        bsum = fmaf(p[nb][j], f0.y, fmaf(p[nb][j + 1], f1.y, bsum));
                        const float w0 = p[nb][j] * f0.x, w1 = p[nb][j + 1] * f1.x;
                        const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(w0, w1));
                        const half2v l = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(
                                                                        (w0 - (float)h[0]) * kLoScale,
                                                                        (w1 - (float)h[1]) * kLoScale));
                        phi[nb][j] = h[0]; phi[nb][j + 1] = h[1];
                        plo[nb][j] = l[0]; plo[nb][j + 1] = l[1];
                    }
                    b_run[nb][0] += bsum;
                }
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    half2v e[4];
#pragma unroll
                    for (int jp = 0; jp < 4; ++jp)
                        e[jp] = v_pair8(vw[2 * jp], vw[2 * jp + 1], sel_b[mm], magic16);
                    const half8 bv = cat8(e[0], e[1], e[2], e[3]);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        acc[nb][mm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi[nb], bv, acc[nb][mm], 0, 0, 0);
                        accl[nb][mm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(plo[nb], bv, accl[nb][mm], 0, 0, 0);
                    }
                }
            } else
#pragma unroll
            for (int s2 = 0; s2 < VS; ++s2) {
                const uint32_t(&vw)[8 * KW] = vbuf[u][s2];
                uint32_t bx[2][4 * KW];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    bx[0][r] = take_half_row<0xC>(vw[2 * r], vw[2 * r + 1]);
                    bx[1][r] = take_half_row<0x3>(vw[2 * r], vw[2 * r + 1]);
                }
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const int gg = 2 * s2 + g;  // scale group of the head
                    half8 phi[NB], plo[NB];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        float bsum = 0.0f;
#pragma unroll
                        for (int j = 0; j < 8; j += 2) {
                            const float2 f0 = fac_zw(slot, 16 * (j >> 2) + 4 * q4 + (j & 3), gg);
                            const float2 f1 = fac_zw(slot, 16 * ((j + 1) >> 2) + 4 * q4 + ((j + 1) & 3), gg);
                            bsum = fmaf(p[nb][j], f0.y, fmaf(p[nb][j + 1], f1.y, bsum));
                            const float w0 = p[nb][j] * f0.x, w1 = p[nb][j + 1] * f1.x;
                            const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(w0, w1));
                            const half2v l = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(
                                                                            (w0 - (float)h[0]) * kLoScale,
                                                                            (w1 - (float)h[1]) * kLoScale));
                            phi[nb][j] = h[0]; phi[nb][j + 1] = h[1];
                            plo[nb][j] = l[0]; plo[nb][j + 1] = l[1];
                        }
                        b_run[nb][gg] += bsum;
                    }
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm) {
                        half2v e[4];
#pragma unroll
                        for (int jp = 0; jp < 4; ++jp)
                            e[jp] = v_pair8(bx[g][2 * jp], bx[g][2 * jp + 1], sel_b[mm], magic16);
                        const half8 bv = cat8(e[0], e[1], e[2], e[3]);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            const int m = 8 * s2 + 4 * g + mm;
                            acc[nb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi[nb], bv, acc[nb][m], 0, 0, 0);
                            accl[nb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(plo[nb], bv, accl[nb][m], 0, 0, 0);
                        }
                    }
                }
            }

            load_tile(ti + PF, kbuf[u], vbuf[u], mbuf[u]);
            stage_meta(slot ^ 1, mbuf[(u + 1) % PF]);
        }
    }

    // ---- normalised outputs: row r = 4 q4 + i is column 16 nb + r
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float l_tot = xrow_sum(l_run[nb]);
        float b_tot[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g)
            b_tot[g] = xrow_sum(b_run[nb][g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * q4 + i;
            const int cc = 16 * nb + r;
            const float inv_l = 1.0f / __shfl(l_tot, r);
            const int rpos = cc / nrep, rhead = cc % nrep;
            const bool on = cc < a.pb * nrep && rpos < npos;
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                const int s2 = gg >> 1, g = gg & 1;
                const float bias = __shfl(b_tot[gg], r);
                // group gg's products of this lane: dimensions 128 s2 + 8 col +
                // 0..3 when its own word is in the set's group g, else
                // 128 s2 + 8 (col ^ 8) + 4..7
                const int d0 = HV ? 8 * (col & 7) + 4 * (col >> 3)  // the column's word
                                  : 128 * s2 + ((g == (low8 ? 0 : 1)) ? 8 * col : 8 * (col ^ 8) + 4);
                float o[4];
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const float hi = acc[nb][8 * s2 + 4 * g + mm][i];
                    const float lo = accl[nb][8 * s2 + 4 * g + mm][i];
                    o[mm] = (fmaf(lo, VU / kLoScale, hi * VU) + bias) * inv_l;
                }
                if (on) {
                    float *dst = a.out + (((int64_t)b * a.Hq + kvh * nrep + rhead) * a.sq + p0 + rpos) * D + d0;
                    *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
                }
            }
        }
    }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// the query-sum piece that each of a group's six score-bias slots multiplies
constexpr int kQPiece[6] = {0, 1, 2, 0, 1, 0};

// v as the sum of three bf16 values (each returned as its 16 bits in the low
// half), exact to all 24 bits of v: each piece is the truncation of what the
// pieces before it leave, and those differences are exact
__device__ __forceinline__ void bf16_split3(float v, uint32_t (&out)[3])
{
    const uint32_t b1 = __builtin_bit_cast(uint32_t, v) & 0xFFFF0000u;
    const float r1 = v - __builtin_bit_cast(float, b1);
    const uint32_t b2 = __builtin_bit_cast(uint32_t, r1) & 0xFFFF0000u;
    const float r2 = r1 - __builtin_bit_cast(float, b2);
    out[0] = b1 >> 16;
    out[1] = b2 >> 16;
    out[2] = __builtin_bit_cast(uint32_t, r2) >> 16;
}

// K word as an MFMA operand of centred codes: k_operand_sub's subnormals
// n 2^-20 less 8 2^-20 (the fp16 subnormal 0x0080), exact
__device__ __forceinline__ half8 k_operand_centred(uint32_t w, uint32_t m_fine)
{
    const half2v c8 = as_h2(0x00800080u);
    return cat8(as_h2((w << 4) & m_fine) - c8, as_h2(w & m_fine) - c8, as_h2((w >> 4) & m_fine) - c8,
                as_h2((w >> 8) & m_fine) - c8);
}

// ---------------------------------------------------------------------------
// int4 codes: the scale and bias factors enter the matrix core
//
// One wavefront per block of 16 NB query columns (NB = 1 at D = 256, where
// the accumulators of one block take as many registers as two do at
// D = 128); the D = 128 kernel below shares the operands of a tile across a
// workgroup. The per-column vector work of a tile is cut to the score's
// per-group scaling, the exponential and one hi/lo split of each weight;
// everything else is a matrix instruction whose operands are exact:
//
// Scores: e[t][c] = sum_g x_{t,g} (Kcodes' . Q[c])_g + Sb[t][c], with the K
// codes centred, n - 8, as the subnormals (n - 8) 2^-20, x = s_k c 2^20 (one
// accumulator per group as before), and Sb = sum_g b'_k c qsum_g + 7 - m,
// b'_k = b_k + 8 s_k (the value of the centre code), from one bf16 matrix
// instruction per 16-row block: b'_k and c qsum_g and 7 - m (fp32) as three
// bf16 pieces each, so every product is exact and the bf16 range takes any
// bias and any query. The matrix core truncates each instruction's sum at
// its largest term; with uncentred codes that term would be b_k c qsum_g,
// which cancels against most of the code products (for the outlier
// workload's K about 150 in log2 units, against scores of about 10), and
// the truncation would show in the weights.
//
// Weights are carried as p' = 2^7 p = exp2(e) (at most 2^(7 - kHeadroom)), as
// an fp16 hi half (truncated) and the exact remainder lo; both halves are at
// the same scale, so lo sinks into the fp16 subnormals only for p' < 2^-4,
// where its absolute error is at most 2^-25 of p'.
//
// Values: the scale goes into the value operand instead of the weights, so
// one (hi, lo) weight pair serves every scale group. s_v (fp16) is split
// into s_hi (its top eight significant bits) and s_lo = s_v - s_hi (three
// bits); a centred code n - 8 times s_hi or s_lo is exact in fp16 (|n - 8|
// is at most 7, or 8, a power of two). Both are halved (so that 8 s_hi stays
// below the fp16 maximum for every fp16 scale); halving is exact except for
// s_lo of scales below 2^-13, where it leaves at most 2^-26 absolute error
// per element. One accumulator per output takes p'_hi V_hi + p'_hi V_lo +
// p'_lo V_hi (p'_lo V_lo, at most 2^-18 of the whole, is left out).
//
// Bias and normaliser: the weight operands times a table whose columns are
// the value a group's centre code stands for, w = b_v + 8 s_v (fp32), as an
// fp16 hi (truncated) and lo pair per group, and ones give sum p' w and
// sum p' = l' in one more accumulator; the output is (2 acc + sum p' w) / l'.
// w lies between the group's extreme values, so its hi half never overflows;
// the pair holds it to 2^-22 relative, or 2^-24 absolute where w is below
// the fp16 normal range. (b_v and 8 s_v in columns of their own would cancel
// in the sum and magnify the matrix core's truncation by |b_v| / |output|.)
template <int PF, int NB, bool Q32, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1)))
void sdpa_prefill_i4_kernel(PrefillArgs a)
{
    constexpr int NG = D / 64;        // scale groups of 64
    constexpr int VS = D / 128;       // sets of 16 value words (two groups each)
    constexpr int W = D / 8;          // words per row
    constexpr int KM = D / 32;        // score products per 16-row block
    constexpr int KPG = KM / NG;      // of them per scale group
    constexpr int PAIRS = PT * NG;
    constexpr int MP = PAIRS / 64;    // (row, group) pairs per lane
    static_assert(PAIRS % 64 == 0, "whole pairs per lane");
    constexpr int QH = Q32 ? 2 : 1;   // query halves: hi (and lo)
    // score-bias operand slots: group g at 6g..6g+5, (b1, b1, b1, b2, b2, b3)
    // against (Q1, Q2, Q3, Q1, Q2, Q1); then three ones against the pieces of
    // 7 - m; the rest zero
    constexpr int SBR = 6 * NG;       // first slot of the reference pieces
    constexpr int SBL = (SBR + 3 + 7) / 8 * 8;  // slots stored per row
    constexpr int NQ4 = SBL / 8;      // lane groups that hold used slots
    constexpr int NVB = 2 * NG + 2;   // value-bias table rows: w hi, w lo per group, ones, zeros
    constexpr float kRef = 7.0f;      // weights are 2^kRef p

    const int lane = threadIdx.x;
    const int q4 = lane >> 4;
    const int col = lane & 15;
    const int kvh = prefill_head(a);
    const int b = blockIdx.z;
    const int nrep = a.n_rep;
    const int p0 = prefill_block(a) * a.pb;
    const int npos = min(a.pb, a.sq - p0);
    const int t_end = (int)a.q_start + p0 + npos;
    const int t_all = (int)a.q_start + p0;
    const int ntile = (t_end + PT - 1) / PT;
    const int64_t kvrow0 = ((int64_t)b * a.Hkv + kvh) * a.cap;
    const bool low8 = (lane & 8) == 0;

    int cpos[NB], chead[NB];
    bool con[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int cc = 16 * nb + col;
        cpos[nb] = cc / nrep;
        chead[nb] = cc % nrep;
        con[nb] = cc < a.pb * nrep && cpos[nb] < npos;
    }

    const uint32_t rows_ok = (uint32_t)t_end;
    const __amdgpu_buffer_rsrc_t kq = make_rsrc(a.k_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t vq = make_rsrc(a.v_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t mres[4] = {
        make_rsrc(a.k_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.k_bias + kvrow0 * NG, rows_ok * NG * 2u),
        make_rsrc(a.v_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.v_bias + kvrow0 * NG, rows_ok * NG * 2u)};

    // per-tile tables, two-slot LDS ring
    __shared__ __align__(16) float xs[2][PT][NG];            // s_k c 2^20
    __shared__ __align__(16) uint16_t sba[2][PT][SBL];       // score-bias operand rows (bf16)
    __shared__ __align__(16) uint16_t vbt[2][NVB][PT];       // value-bias table (fp16), by column
    __shared__ __align__(16) uint16_t svt[2][2 * NG][PT];    // s_hi / 2, then s_lo / 2 (fp16)
    const Unpacker unpack = Unpacker::make();
    const float cs = a.score_scale;
    const float csk = cs * 1048576.0f;
    const uint32_t m_fine = 0x00F000F0u;
    // 1.0 the compiler cannot see: the weights' lo halves w - hi below then
    // stay a multiply-add whose fp16 operand hi is read as it is (one mixed
    // fp16/fp32 FMA instead of a conversion and a subtraction); the product
    // w * 1 and the difference are exact either way
    const float one = __builtin_bit_cast(float, opaque_s(0x3f800000u));

    // the constant parts of the tables, in both slots: ones against the
    // reference pieces, zero slots, the ones and zeros columns
    {
        const int s = lane >> 5, r = lane & 31;
#pragma unroll
        for (int k = SBR; k < SBL; ++k)
            sba[s][r][k] = k < SBR + 3 ? (uint16_t)0x3F80u : (uint16_t)0u;
        vbt[s][2 * NG][r] = 0x3C00u;
        vbt[s][2 * NG + 1][r] = 0u;
    }

    constexpr uint32_t kNoRows = 0x80000000u;
    uint32_t kbuf[PF][2][KM];
    uint32_t vbuf[PF][VS][8];
    uint32_t mbuf[PF][MP][4];
    auto load_tile = [&](int ti, uint32_t (&kt)[2][KM], uint32_t (&vt)[VS][8], uint32_t (&mt)[MP][4]) {
        const bool in = ti < ntile;
#pragma unroll
        for (int pp = 0; pp < MP; ++pp) {
            const uint32_t moff = in ? (uint32_t)((PT * ti) * NG + lane + 64 * pp) * 2u : kNoRows;
#pragma unroll
            for (int arr = 0; arr < 4; ++arr)
                mt[pp][arr] = __builtin_amdgcn_raw_buffer_load_b16(mres[arr], moff, 0, 0);
        }
        const uint32_t base = in ? (uint32_t)(PT * ti) * (uint32_t)(W * 4) : kNoRows;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const uint32_t off = base + (uint32_t)(((16 * blk + col) * W + q4) * 4);
#pragma unroll
            for (int uu = 0; uu < KM; ++uu)
                kt[blk][uu] = __builtin_amdgcn_raw_buffer_load_b32(kq, off + 16 * uu, 0, 0);
        }
#pragma unroll
        for (int s2 = 0; s2 < VS; ++s2) {
            const uint32_t voff = base + (uint32_t)((4 * q4 * W + 16 * s2 + col) * 4);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                vt[s2][j] = __builtin_amdgcn_raw_buffer_load_b32(vq, voff + ((16 * (j >> 2) + (j & 3)) * W) * 4, 0, 0);
        }
    };
    auto stage_meta = [&](int slot, const uint32_t (&mt)[MP][4]) {
#pragma unroll
        for (int pp = 0; pp < MP; ++pp) {
            const int idx = lane + 64 * pp;
            const int r = idx / NG, g = idx % NG;
            const uint16_t ks = (uint16_t)mt[pp][0], kb = (uint16_t)mt[pp][1];
            const uint16_t vsb = (uint16_t)mt[pp][2], vbb = (uint16_t)mt[pp][3];
            xs[slot][r][g] = h_val(ks) * csk;
            uint32_t bp[3];
            bf16_split3(fmaf(8.0f, h_val(ks), h_val(kb)), bp);
            uint32_t *srow = reinterpret_cast<uint32_t *>(&sba[slot][r][6 * g]);
            srow[0] = bp[0] | (bp[0] << 16);
            srow[1] = bp[0] | (bp[1] << 16);
            srow[2] = bp[1] | (bp[2] << 16);
            const float w = fmaf(8.0f, h_val(vsb), h_val(vbb));
            const float whi = (float)__builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(w, 0.0f))[0];
            // (the halves are copied out before the bit casts: a bit cast of a
            // vector element in place reads element 0)
            const half2v wp = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(whi, w - whi));
            const _Float16 wh = wp[0], wl = wp[1];
            vbt[slot][2 * g][r] = __builtin_bit_cast(uint16_t, wh);
            vbt[slot][2 * g + 1][r] = __builtin_bit_cast(uint16_t, wl);
            const float sh = h_val((uint16_t)(vsb & 0xFFF8u));
            const float sl = h_val(vsb) - sh;
            svt[slot][g][r] = __builtin_bit_cast(uint16_t, (_Float16)(0.5f * sh));
            svt[slot][NG + g][r] = __builtin_bit_cast(uint16_t, (_Float16)(0.5f * sl));
        }
        asm volatile("" ::: "memory");
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        load_tile(u, kbuf[u], vbuf[u], mbuf[u]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // query operands (as in the kernel above) and the fp32 group sums of
    // exactly what the matrix core sees
    half8 qop[NB][QH][KM];
    float qsum[NB][NG];
    __shared__ __align__(16) half8 q_lds[NB][QH][KM][64];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t qrow = (((int64_t)b * a.Hq + kvh * nrep + (con[nb] ? chead[nb] : 0)) * a.sq + p0 +
                              (con[nb] ? cpos[nb] : 0)) * D;
        float gs[NG] = {};
#pragma unroll
        for (int uu = 0; uu < KM; ++uu) {
            float x[8];
            if constexpr (Q32) {
                const float *qp = reinterpret_cast<const float *>(a.q) + qrow + 32 * uu + 8 * q4;
                const float4 x0 = *reinterpret_cast<const float4 *>(qp);
                const float4 x1 = *reinterpret_cast<const float4 *>(qp + 4);
                x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
                x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
            } else {
                const half8 h8 = *reinterpret_cast<const half8 *>(reinterpret_cast<const _Float16 *>(a.q) + qrow +
                                                                  32 * uu + 8 * q4);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    x[j] = (float)h8[j];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xv = con[nb] ? x[kPerm[j]] : 0.0f;
                const _Float16 hi = (_Float16)xv;
                qop[nb][0][uu][j] = hi;
                if constexpr (Q32) {
                    const _Float16 lo = (_Float16)(xv - (float)hi);
                    qop[nb][QH - 1][uu][j] = lo;
                    gs[uu / KPG] += (float)hi + (float)lo;
                } else {
                    gs[uu / KPG] += (float)hi;
                }
            }
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
            qsum[nb][g] = xrow_sum(gs[g]);
#pragma unroll
        for (int hl = 0; hl < QH; ++hl)
#pragma unroll
            for (int uu = 0; uu < KM; ++uu)
                q_lds[nb][hl][uu][lane] = qop[nb][hl][uu];
    }
    stage_meta(0, mbuf[0]);

    // the score-bias B operand of block nb: this lane's column, slots
    // 8 q4 .. 8 q4 + 7 (c qsum_g and 7 - m as bf16 pieces)
    float ref[NB];  // 7 - m, this lane's column
    bf16x8 sbb[NB];
    auto build_sbb = [&](int nb) {
        uint32_t qp[NG][3], rp[3];
#pragma unroll
        for (int g = 0; g < NG; ++g)
            bf16_split3(cs * qsum[nb][g], qp[g]);
        bf16_split3(ref[nb], rp);
        auto piece = [&](int k) -> uint32_t {  // k a constant after unrolling
            if (k < SBR)
                return qp[k / 6][kQPiece[k % 6]];
            if (k < SBR + 3)
                return rp[k - SBR];
            return 0u;
        };
        u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int qq = 0; qq < NQ4; ++qq)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint32_t v = piece(8 * qq + 2 * jj) | (piece(8 * qq + 2 * jj + 1) << 16);
                w[jj] = q4 == qq ? v : w[jj];
            }
        sbb[nb] = __builtin_bit_cast(bf16x8, w);
    };

    float4v acc[NB][8 * VS], bacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        ref[nb] = kRef;
        build_sbb(nb);
        bacc[nb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 8 * VS; ++m)
            acc[nb][m] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int vrow = min(col, 2 * NG + 1);  // this lane's value-bias table row

#pragma unroll 1
    for (int kk = 0; kk < ntile; kk += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int ti = kk + u;
            const int slot = u & 1;

            // ---- exponents of the lane's 8 rows (16 blk + 4 q4 + i) for each block's column
            float sc[NB][8];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int ar = 16 * blk + col;
                const u32x4 araw = *reinterpret_cast<const u32x4 *>(&sba[slot][ar][8 * min(q4, NQ4 - 1)]);
                const bf16x8 sa = __builtin_bit_cast(bf16x8, araw);
                float4v s[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    s[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa, sbb[nb], (float4v){0.0f, 0.0f, 0.0f, 0.0f},
                                                                   0, 0, 0);
                float4v sacc[NG][NB];
#pragma unroll
                for (int g = 0; g < NG; ++g) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        sacc[g][nb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int k = 0; k < KPG; ++k) {
                        const half8 ka = k_operand_centred(kbuf[u][blk][g * KPG + k], m_fine);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int hl = 0; hl < QH; ++hl)
                                sacc[g][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, q_lds[nb][hl][g * KPG + k][lane],
                                                                                    sacc[g][nb], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float xg[NG];
#pragma unroll
                    for (int g = 0; g < NG; ++g)
                        xg[g] = xs[slot][16 * blk + 4 * q4 + i][g];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        float e = s[nb][i];
#pragma unroll
                        for (int g = 0; g < NG; ++g)
                            e = fmaf(xg[g], sacc[g][nb][i], e);
                        sc[nb][4 * blk + i] = e;
                    }
                }
            }
            if (PT * ti + PT - 1 > t_all) {  // uniform: some row is past some column's position
                asm volatile("" ::: "memory");
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int lim = t_all + cpos[nb];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int r = PT * ti + 16 * (i >> 2) + 4 * q4 + (i & 3);
                        sc[nb][i] = r <= lim ? sc[nb][i] : -INFINITY;
                    }
                }
            }
            half8 phi[NB], plo[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float mx = max3_raw(max3_raw(sc[nb][0], sc[nb][1], sc[nb][2]),
                                          max3_raw(sc[nb][3], sc[nb][4], sc[nb][5]), max_raw(sc[nb][6], sc[nb][7]));
                // ---- reference raised only when an exponent exceeds kRef (the first tile sets it)
                if (ti == 0 || __builtin_amdgcn_ballot_w64(mx > kRef) != 0) {
                    const float full = xrow_max(mx, -INFINITY);
                    const bool raise = full > kRef || (ti == 0 && full > -INFINITY);
                    const float r_new = raise ? ref[nb] - (full - (kRef - kHeadroom)) : ref[nb];
                    const float delta = ref[nb] - r_new;
                    ref[nb] = r_new;
                    build_sbb(nb);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        sc[nb][i] -= delta;
                    if (ti != 0) {
                        const float corr = __builtin_amdgcn_exp2f(-delta);
                        float4v corr_row;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            corr_row[i] = __shfl(corr, 4 * q4 + i);
                        bacc[nb] *= corr_row;
#pragma unroll
                        for (int m = 0; m < 8 * VS; ++m)
                            acc[nb][m] *= corr_row;
                    }
                }
                // ---- weights 2^7 p as hi (truncated) and lo halves
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const float w0 = __builtin_amdgcn_exp2f(sc[nb][j]);
                    const float w1 = __builtin_amdgcn_exp2f(sc[nb][j + 1]);
                    const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(w0, w1));
                    const half2v l = __builtin_bit_cast(
                        half2v, __builtin_amdgcn_cvt_pkrtz(fmaf(w0, one, -(float)h[0]), fmaf(w1, one, -(float)h[1])));
                    phi[nb][j] = h[0]; phi[nb][j + 1] = h[1];
                    plo[nb][j] = l[0]; plo[nb][j + 1] = l[1];
                }
            }

            // ---- value products: the lane's rows (2 jp, 2 jp + 1) pair up in
            // each fp16 pair of the operand, so the scale halves of a pair of
            // rows multiply one half2
#pragma unroll
            for (int s2 = 0; s2 < VS; ++s2) {
                const uint32_t(&vw)[8] = vbuf[u][s2];
                uint32_t bx[2][4];
#pragma unroll
                for (int jp = 0; jp < 4; ++jp) {
                    const uint32_t xw = __builtin_amdgcn_perm(vw[2 * jp + 1], vw[2 * jp], 0x05040100u);
                    const uint32_t yw = __builtin_amdgcn_perm(vw[2 * jp + 1], vw[2 * jp], 0x07060302u);
                    bx[0][jp] = take_half_row<0xC>(xw, yw);
                    bx[1][jp] = take_half_row<0x3>(xw, yw);
                }
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    const int gg = 2 * s2 + g;
                    const uint2 h0 = *reinterpret_cast<const uint2 *>(&svt[slot][gg][4 * q4]);
                    const uint2 h1 = *reinterpret_cast<const uint2 *>(&svt[slot][gg][16 + 4 * q4]);
                    const uint2 l0 = *reinterpret_cast<const uint2 *>(&svt[slot][NG + gg][4 * q4]);
                    const uint2 l1 = *reinterpret_cast<const uint2 *>(&svt[slot][NG + gg][16 + 4 * q4]);
                    const half2v shi[4] = {as_h2(h0.x), as_h2(h0.y), as_h2(h1.x), as_h2(h1.y)};
                    const half2v slo[4] = {as_h2(l0.x), as_h2(l0.y), as_h2(l1.x), as_h2(l1.y)};
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm) {
                        half2v e[4];
#pragma unroll
                        for (int jp = 0; jp < 4; ++jp)
                            e[jp] = unpack.one(bx[g][jp], mm);
                        const half8 vh = cat8(e[0] * shi[0], e[1] * shi[1], e[2] * shi[2], e[3] * shi[3]);
                        const half8 vl = cat8(e[0] * slo[0], e[1] * slo[1], e[2] * slo[2], e[3] * slo[3]);
                        const int m = 8 * s2 + 4 * g + mm;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[nb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi[nb], vh, acc[nb][m], 0, 0, 0);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[nb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi[nb], vl, acc[nb][m], 0, 0, 0);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            acc[nb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(plo[nb], vh, acc[nb][m], 0, 0, 0);
                    }
                }
            }
            // ---- bias sums and the normaliser: rows 4 q4 .. + 3 and 16 + 4 q4 .. + 3 of table row vrow
            {
                const uint2 c0 = *reinterpret_cast<const uint2 *>(&vbt[slot][vrow][4 * q4]);
                const uint2 c1 = *reinterpret_cast<const uint2 *>(&vbt[slot][vrow][16 + 4 * q4]);
                const half8 bv = __builtin_bit_cast(half8, (u32x4){c0.x, c0.y, c1.x, c1.y});
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    bacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi[nb], bv, bacc[nb], 0, 0, 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    bacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(plo[nb], bv, bacc[nb], 0, 0, 0);
            }

            load_tile(ti + PF, kbuf[u], vbuf[u], mbuf[u]);
            stage_meta(slot ^ 1, mbuf[(u + 1) % PF]);
        }
    }

    // ---- normalised outputs: accumulator row 4 q4 + i is column 16 nb + 4 q4 + i;
    // its bias sums and l' sit in lanes 16 q4 + n of bacc (table column n)
    const int rowbase = lane & 48;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = 16 * nb + 4 * q4 + i;
            const float inv_l = 1.0f / __shfl(bacc[nb][i], rowbase + 2 * NG);
            const int rpos = cc / nrep, rhead = cc % nrep;
            const bool on = cc < a.pb * nrep && rpos < npos;
#pragma unroll
            for (int gg = 0; gg < NG; ++gg) {
                const int s2 = gg >> 1, g = gg & 1;
                const float bias = __shfl(bacc[nb][i], rowbase + 2 * gg) + __shfl(bacc[nb][i], rowbase + 2 * gg + 1);
                const int d0 = 128 * s2 + ((g == (low8 ? 0 : 1)) ? 8 * col : 8 * (col ^ 8) + 4);
                float o[4];
#pragma unroll
                for (int mm = 0; mm < 4; ++mm)
                    o[mm] = fmaf(2.0f, acc[nb][8 * s2 + 4 * g + mm][i], bias) * inv_l;
                if (on) {
                    float *dst = a.out + (((int64_t)b * a.Hq + kvh * nrep + rhead) * a.sq + p0 + rpos) * D + d0;
                    *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// int4 codes, D = 64 and 128: WG wavefronts share each tile's unpacked
// operands
//
// The arithmetic of sdpa_prefill_i4_kernel, with WG wavefronts per
// workgroup on consecutive position blocks of one (batch, KV head): they
// read the same rows, so each builds only 1/WG of a tile's matrix operands
// into LDS: the K operands (centred codes as subnormals) and the V operands
// (centred codes times s_hi / 2 and times s_lo / 2). The factor tables
// are staged in batches into a ring of 2 WG slots: every WG tiles each
// wavefront stages one of the next WG tiles (tiles t + 2 .. t + WG + 1 at
// tile t), so the staging falls on all wavefronts in the same tile (the
// builders of tile t + 1 read its value-scale halves while tile t is being
// computed); one barrier per tile separates building tile t + 1 (into the
// other half of a two-slot operand ring) from the reads of tile t.
// D = 128: WG = 8 with fp16 queries (one workgroup per CU, two wavefronts
// per SIMD); WG = 4 with fp32 queries, whose hi and lo query operands take
// twice the LDS (one wavefront per SIMD). D = 64: WG = 4 (a tile has four K
// and four V operands, one of each per wavefront).
template <int PF, int NB, bool Q32, int WG, int D>
__global__ __launch_bounds__(64 * WG) __attribute__((amdgpu_waves_per_eu(WG / 4)))
void sdpa_prefill_i4_wg_kernel(PrefillArgs a)
{
    // D = 64: one scale group of eight words; each of the 16 value columns is
    // half a word (word col & 7, dimensions 4 (col >> 3) + mm), as in the
    // one-wavefront kernel
    static_assert(D == 128 || D == 64, "two scale groups, or one");
    constexpr bool HV = D == 64;
    constexpr int NG = D / 64, W = D / 8, KM = D / 32, KPG = 2;
    constexpr int QH = Q32 ? 2 : 1;
    constexpr int SBR = 6 * NG;
    constexpr int SBL = (SBR + 3 + 7) / 8 * 8;
    constexpr int NQ4 = SBL / 8;
    constexpr int NVB = 2 * NG + 2;
    constexpr float kRef = 7.0f;
    constexpr int NKO = 2 * KM;   // K operands of a tile: (16-row block, 32 dimensions)
    constexpr int NVO = 4 * NG;   // V operands of a tile, hi and lo each: (scale group, mm)
    constexpr int KO = NKO / WG;  // of them built by each wavefront
    constexpr int VO = NVO / WG;
    static_assert(NKO % WG == 0 && NVO % WG == 0, "operands split evenly");
    static_assert(PT * NG == 64 || PT * NG == 32, "at most one (row, group) pair per lane of the staging wavefront");
    static_assert(PF == 2, "tile j's words in register buffer j % 2");

    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int q4 = lane >> 4;
    const int col = lane & 15;
    const int kvh = prefill_head(a);
    const int b = blockIdx.z;
    const int nrep = a.n_rep;
    const int p0g = prefill_block(a) * WG * a.pb;          // first position of the workgroup
    const int p0 = p0g + wv * a.pb;                        // of this wavefront
    const int npos = max(0, min(a.pb, a.sq - p0));         // this wavefront's positions (may be none)
    const int t_end = (int)a.q_start + min(p0g + WG * a.pb, a.sq);  // rows [0, t_end) are read
    const int t_all = (int)a.q_start + p0;
    const int ntile = (t_end + PT - 1) / PT;
    const int64_t kvrow0 = ((int64_t)b * a.Hkv + kvh) * a.cap;
    const bool low8 = (lane & 8) == 0;

    int cpos[NB], chead[NB];
    bool con[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int cc = 16 * nb + col;
        cpos[nb] = cc / nrep;
        chead[nb] = cc % nrep;
        con[nb] = cc < a.pb * nrep && cpos[nb] < npos;
    }

    const uint32_t rows_ok = (uint32_t)t_end;
    const __amdgpu_buffer_rsrc_t kq = make_rsrc(a.k_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t vq = make_rsrc(a.v_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t mres[4] = {
        make_rsrc(a.k_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.k_bias + kvrow0 * NG, rows_ok * NG * 2u),
        make_rsrc(a.v_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.v_bias + kvrow0 * NG, rows_ok * NG * 2u)};

    __shared__ __align__(16) half8 kop[2][NKO][64];          // K operands
    __shared__ __align__(16) half8 vhi[2][NVO][64];          // V operands, codes x s_hi / 2
    __shared__ __align__(16) half8 vlo[2][NVO][64];          // V operands, codes x s_lo / 2
    // factor tables, a ring of NTS slots (slot of tile t: t % NTS), staged in
    // batches: every WG tiles each wavefront stages one of the next WG tiles
    constexpr int NTS = 2 * WG;
    // rows per table slot: PT, and at D = 64 (32 (row, group) pairs per tile)
    // 8 more that take the stores of the staging lanes 32-63, so that every
    // lane stores (a branch around the stores does not compile here)
    constexpr int PTX = PT * NG < 64 ? PT + 8 : PT;
    __shared__ __align__(16) float xs[NTS][PTX][NG];
    __shared__ __align__(16) uint16_t sba[NTS][PTX][SBL];
    __shared__ __align__(16) uint16_t vbt[NTS][NVB][PTX];
    __shared__ __align__(16) uint16_t svt[NTS][2 * NG][PTX];
    __shared__ __align__(16) half8 q_lds[WG][NB][QH][KM][64];
    const float cs = a.score_scale;
    const float csk = cs * 1048576.0f;
    const uint32_t m_fine = 0x00F000F0u;
    // 1.0 the compiler cannot see: the weights' lo halves w - hi below then
    // stay a multiply-add whose fp16 operand hi is read as it is (one mixed
    // fp16/fp32 FMA instead of a conversion and a subtraction); the product
    // w * 1 and the difference are exact either way
    const float one = __builtin_bit_cast(float, opaque_s(0x3f800000u));

    // this wavefront's V operands are (g, mm) = (v >> 2, v & 3) with
    // v = wv + WG i: the nibble to take is chosen by wave-uniform shift,
    // mask, magic and offset
    static_assert(WG == 8 || WG == 4, "one or two (g, mm) operands per wavefront");

    // the constant parts of the tables, in every slot
    static_assert(NTS * PT <= 64 * WG, "one thread per (slot, row)");
    if (threadIdx.x < NTS * PT) {
        const int s = threadIdx.x / PT, r = threadIdx.x % PT;
#pragma unroll
        for (int k = SBR; k < SBL; ++k)
            sba[s][r][k] = k < SBR + 3 ? (uint16_t)0x3F80u : (uint16_t)0u;
        vbt[s][2 * NG][r] = 0x3C00u;
        vbt[s][2 * NG + 1][r] = 0u;
    }

    constexpr uint32_t kNoRows = 0x80000000u;
    uint32_t kbuf[PF][KO];
    uint32_t vbuf[PF][8];
    auto load_tile = [&](int ti, uint32_t (&kt)[KO], uint32_t (&vt)[8]) {
        const bool in = ti < ntile;
        const uint32_t base = in ? (uint32_t)(PT * ti) * (uint32_t)(W * 4) : kNoRows;
#pragma unroll
        for (int i = 0; i < KO; ++i) {
            const int o = wv + WG * i;  // blk = o / KM, uu = o % KM
            kt[i] = __builtin_amdgcn_raw_buffer_load_b32(
                kq, base + (uint32_t)((((16 * (o / KM) + col) * W + q4) * 4) + 16 * (o % KM)), 0, 0);
        }
        const uint32_t voff = base + (uint32_t)((4 * q4 * W + (HV ? (col & 7) : col)) * 4);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            vt[j] = __builtin_amdgcn_raw_buffer_load_b32(vq, voff + ((16 * (j >> 2) + (j & 3)) * W) * 4, 0, 0);
    };
    // the scale/bias words of tile tj, one (row, group) per lane
    auto load_meta = [&](int tj, uint32_t (&mt)[4]) {
        const uint32_t moff = tj < ntile ? (uint32_t)((PT * tj) * NG + lane) * 2u : kNoRows;
#pragma unroll
        for (int arr = 0; arr < 4; ++arr)
            mt[arr] = __builtin_amdgcn_raw_buffer_load_b16(mres[arr], moff, 0, 0);
    };
    // tile ti's operands into operand slot `slot`; its value-scale halves
    // come from table slot `ts` (staged a tile earlier)
    auto build = [&](int slot, int ts, const uint32_t (&kt)[KO], const uint32_t (&vt)[8]) {
#pragma unroll
        for (int i = 0; i < KO; ++i)
            kop[slot][wv + WG * i][lane] = k_operand_centred(kt[i], m_fine);
        uint32_t bx[2][4];
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) {
            if constexpr (HV) {  // the two bytes of the lane's half word (one group)
                const uint32_t xw = __builtin_amdgcn_perm(vt[2 * jp + 1], vt[2 * jp], 0x05040100u);
                const uint32_t yw = __builtin_amdgcn_perm(vt[2 * jp + 1], vt[2 * jp], 0x07060302u);
                bx[0][jp] = (col >> 3) ? yw : xw;
                bx[1][jp] = bx[0][jp];
            } else {
                const uint32_t xw = __builtin_amdgcn_perm(vt[2 * jp + 1], vt[2 * jp], 0x05040100u);
                const uint32_t yw = __builtin_amdgcn_perm(vt[2 * jp + 1], vt[2 * jp], 0x07060302u);
                bx[0][jp] = take_half_row<0xC>(xw, yw);
                bx[1][jp] = take_half_row<0x3>(xw, yw);
            }
        }
#pragma unroll
        for (int i = 0; i < VO; ++i) {
            const int v = wv + WG * i;
            const int g = v >> 2, mm = v & 3;
            const uint32_t sh = mm >= 2 ? 8u : 0u;
            const uint32_t mask = opaque_s((mm & 1) ? 0x00F000F0u : 0x000F000Fu);
            const uint32_t magic = opaque_v((mm & 1) ? 0x54005400u : 0x64006400u);
            const half2v off = as_h2((mm & 1) ? 0x54805480u : 0x64086408u);  // 72 or 1032
            const uint2 h0 = *reinterpret_cast<const uint2 *>(&svt[ts][g][4 * q4]);
            const uint2 h1 = *reinterpret_cast<const uint2 *>(&svt[ts][g][16 + 4 * q4]);
            const uint2 l0 = *reinterpret_cast<const uint2 *>(&svt[ts][NG + g][4 * q4]);
            const uint2 l1 = *reinterpret_cast<const uint2 *>(&svt[ts][NG + g][16 + 4 * q4]);
            const half2v shi[4] = {as_h2(h0.x), as_h2(h0.y), as_h2(h1.x), as_h2(h1.y)};
            const half2v slo[4] = {as_h2(l0.x), as_h2(l0.y), as_h2(l1.x), as_h2(l1.y)};
            half2v e[4];
#pragma unroll
            for (int jp = 0; jp < 4; ++jp) {
                const uint32_t x = g == 0 ? bx[0][jp] : bx[1][jp];
                e[jp] = as_h2(and_or(x >> sh, mask, magic)) - off;
            }
            vhi[slot][v][lane] = cat8(e[0] * shi[0], e[1] * shi[1], e[2] * shi[2], e[3] * shi[3]);
            vlo[slot][v][lane] = cat8(e[0] * slo[0], e[1] * slo[1], e[2] * slo[2], e[3] * slo[3]);
        }
    };
    // a tile's factor tables into table slot ts, from its scale/bias words
    // mt (load_meta)
    auto stage = [&](int ts, const uint32_t (&mt)[4]) {
        // (D = 64: lanes 32-63 loaded the next tile's words; they store into the spare row PT)
        const int r = PT * NG < 64 && lane >= PT * NG ? PT : lane / NG, g = lane % NG;
        const uint16_t ks = (uint16_t)mt[0], kb = (uint16_t)mt[1];
        const uint16_t vsb = (uint16_t)mt[2], vbb = (uint16_t)mt[3];
        xs[ts][r][g] = h_val(ks) * csk;
        uint32_t bp[3];
        bf16_split3(fmaf(8.0f, h_val(ks), h_val(kb)), bp);
        uint32_t *srow = reinterpret_cast<uint32_t *>(&sba[ts][r][6 * g]);
        srow[0] = bp[0] | (bp[0] << 16);
        srow[1] = bp[0] | (bp[1] << 16);
        srow[2] = bp[1] | (bp[2] << 16);
        const float w = fmaf(8.0f, h_val(vsb), h_val(vbb));
        const float whi = (float)__builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(w, 0.0f))[0];
        // (the halves are copied out before the bit casts: a bit cast of a
        // vector element in place reads element 0)
        const half2v wp = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(whi, w - whi));
        const _Float16 wh = wp[0], wl = wp[1];
        vbt[ts][2 * g][r] = __builtin_bit_cast(uint16_t, wh);
        vbt[ts][2 * g + 1][r] = __builtin_bit_cast(uint16_t, wl);
        const float shv = h_val((uint16_t)(vsb & 0xFFF8u));
        const float slv = h_val(vsb) - shv;
        svt[ts][g][r] = __builtin_bit_cast(uint16_t, (_Float16)(0.5f * shv));
        svt[ts][NG + g][r] = __builtin_bit_cast(uint16_t, (_Float16)(0.5f * slv));
    };

    // query operands (as in the kernels above)
    float qsum[NB][NG];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t qrow = (((int64_t)b * a.Hq + kvh * nrep + (con[nb] ? chead[nb] : 0)) * a.sq +
                              (con[nb] ? p0 + cpos[nb] : 0)) * D;
        float gs[NG] = {};
#pragma unroll
        for (int uu = 0; uu < KM; ++uu) {
            float x[8];
            if constexpr (Q32) {
                const float *qp = reinterpret_cast<const float *>(a.q) + qrow + 32 * uu + 8 * q4;
                const float4 x0 = *reinterpret_cast<const float4 *>(qp);
                const float4 x1 = *reinterpret_cast<const float4 *>(qp + 4);
                x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
                x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
            } else {
                const half8 h8 = *reinterpret_cast<const half8 *>(reinterpret_cast<const _Float16 *>(a.q) + qrow +
                                                                  32 * uu + 8 * q4);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    x[j] = (float)h8[j];
            }
            half8 qh, ql;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xv = con[nb] ? x[kPerm[j]] : 0.0f;
                const _Float16 hi = (_Float16)xv;
                qh[j] = hi;
                if constexpr (Q32) {
                    const _Float16 lo = (_Float16)(xv - (float)hi);
                    ql[j] = lo;
                    gs[uu / KPG] += (float)hi + (float)lo;
                } else {
                    gs[uu / KPG] += (float)hi;
                }
            }
            q_lds[wv][nb][0][uu][lane] = qh;
            if constexpr (Q32)
                q_lds[wv][nb][QH - 1][uu][lane] = ql;
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
            qsum[nb][g] = xrow_sum(gs[g]);
    }

    // prologue: raw words of tiles 0 and 1; the tables of tiles 0 and 1
    // staged by wavefronts 0 and 1, the scale/bias words of the first batch
    // (tiles 2 .. WG + 1, one per wavefront) loaded; then tile 0 built (its
    // builders read its value-scale halves) and tile 2 loaded
    uint32_t mb[4];  // this wavefront's tile of the next batch
#pragma unroll
    for (int u = 0; u < PF; ++u)
        load_tile(u, kbuf[u], vbuf[u]);
    if (wv < 2) {
        uint32_t m0[4];
        load_meta(wv, m0);
        stage(wv, m0);
    }
    load_meta(2 + wv, mb);
    __syncthreads();
    build(0, 0, kbuf[0], vbuf[0]);
    load_tile(2, kbuf[0], vbuf[0]);
    __syncthreads();

    float ref[NB];
    bf16x8 sbb[NB];
    auto build_sbb = [&](int nb) {
        uint32_t qp[NG][3], rp[3];
#pragma unroll
        for (int g = 0; g < NG; ++g)
            bf16_split3(cs * qsum[nb][g], qp[g]);
        bf16_split3(ref[nb], rp);
        auto piece = [&](int k) -> uint32_t {
            if (k < SBR)
                return qp[k / 6][kQPiece[k % 6]];
            if (k < SBR + 3)
                return rp[k - SBR];
            return 0u;
        };
        u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int qq = 0; qq < NQ4; ++qq)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint32_t v = piece(8 * qq + 2 * jj) | (piece(8 * qq + 2 * jj + 1) << 16);
                w[jj] = q4 == qq ? v : w[jj];
            }
        sbb[nb] = __builtin_bit_cast(bf16x8, w);
    };

    float4v acc[NB][8], bacc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        ref[nb] = kRef;
        build_sbb(nb);
        bacc[nb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < 8; ++m)
            acc[nb][m] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int vrow = min(col, 2 * NG + 1);

#pragma unroll 1
    for (int kk = 0; kk < ntile; kk += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int ti = kk + u;
            const int slot = u & 1;
            const int ts = ti & (NTS - 1), ts1 = (ti + 1) & (NTS - 1);  // table slots of tiles ti, ti + 1

            float sc[NB][8];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const u32x4 araw =
                    *reinterpret_cast<const u32x4 *>(&sba[ts][16 * blk + col][8 * min(q4, NQ4 - 1)]);
                const bf16x8 sa = __builtin_bit_cast(bf16x8, araw);
                float4v s[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    s[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa, sbb[nb], (float4v){0.0f, 0.0f, 0.0f, 0.0f},
                                                                   0, 0, 0);
                float4v sacc[NG][NB];
#pragma unroll
                for (int g = 0; g < NG; ++g) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        sacc[g][nb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int k = 0; k < KPG; ++k) {
                        const half8 ka = kop[slot][blk * KM + g * KPG + k][lane];
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int hl = 0; hl < QH; ++hl)
                                sacc[g][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    ka, q_lds[wv][nb][hl][g * KPG + k][lane], sacc[g][nb], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (NG == 2) {
                        const float2 xg = *reinterpret_cast<const float2 *>(&xs[ts][16 * blk + 4 * q4 + i][0]);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            sc[nb][4 * blk + i] = fmaf(xg.x, sacc[0][nb][i], fmaf(xg.y, sacc[1][nb][i], s[nb][i]));
                    } else {
                        const float xg = xs[ts][16 * blk + 4 * q4 + i][0];
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            sc[nb][4 * blk + i] = fmaf(xg, sacc[0][nb][i], s[nb][i]);
                    }
                }
            }
            if (PT * ti + PT - 1 > t_all) {
                asm volatile("" ::: "memory");
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int lim = t_all + cpos[nb];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int r = PT * ti + 16 * (i >> 2) + 4 * q4 + (i & 3);
                        sc[nb][i] = r <= lim ? sc[nb][i] : -INFINITY;
                    }
                }
            }
            half8 phi[NB], plo[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float mx = max3_raw(max3_raw(sc[nb][0], sc[nb][1], sc[nb][2]),
                                          max3_raw(sc[nb][3], sc[nb][4], sc[nb][5]), max_raw(sc[nb][6], sc[nb][7]));
                if (ti == 0 || __builtin_amdgcn_ballot_w64(mx > kRef) != 0) {
                    const float full = xrow_max(mx, -INFINITY);
                    const bool raise = full > kRef || (ti == 0 && full > -INFINITY);
                    const float r_new = raise ? ref[nb] - (full - (kRef - kHeadroom)) : ref[nb];
                    const float delta = ref[nb] - r_new;
                    ref[nb] = r_new;
                    build_sbb(nb);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        sc[nb][i] -= delta;
                    if (ti != 0) {
                        const float corr = __builtin_amdgcn_exp2f(-delta);
                        float4v corr_row;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            corr_row[i] = __shfl(corr, 4 * q4 + i);
                        bacc[nb] *= corr_row;
#pragma unroll
                        for (int m = 0; m < 8; ++m)
                            acc[nb][m] *= corr_row;
                    }
                }
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    const float w0 = __builtin_amdgcn_exp2f(sc[nb][j]);
                    const float w1 = __builtin_amdgcn_exp2f(sc[nb][j + 1]);
                    const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(w0, w1));
                    const half2v l = __builtin_bit_cast(
                        half2v, __builtin_amdgcn_cvt_pkrtz(fmaf(w0, one, -(float)h[0]), fmaf(w1, one, -(float)h[1])));
                    phi[nb][j] = h[0]; phi[nb][j + 1] = h[1];
                    plo[nb][j] = l[0]; plo[nb][j + 1] = l[1];
                }
            }

#pragma unroll
            for (int m = 0; m < NVO; ++m) {
                const half8 vh = vhi[slot][m][lane], vl = vlo[slot][m][lane];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi[nb], vh, acc[nb][m], 0, 0, 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi[nb], vl, acc[nb][m], 0, 0, 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    acc[nb][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(plo[nb], vh, acc[nb][m], 0, 0, 0);
            }
            {
                const uint2 c0 = *reinterpret_cast<const uint2 *>(&vbt[ts][vrow][4 * q4]);
                const uint2 c1 = *reinterpret_cast<const uint2 *>(&vbt[ts][vrow][16 + 4 * q4]);
                const half8 bv = __builtin_bit_cast(half8, (u32x4){c0.x, c0.y, c1.x, c1.y});
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    bacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi[nb], bv, bacc[nb], 0, 0, 0);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    bacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(plo[nb], bv, bacc[nb], 0, 0, 0);
            }

            // tile ti + 1's operands into the other operand slot (its words
            // were loaded two tiles ago, its tables staged at least a tile
            // ago); every WG tiles the batch of tables of tiles ti + 2 ..
            // ti + WG + 1 (this wavefront's: ti + 2 + wv), whose words were
            // loaded a tile earlier, so that the wavefronts share that work
            // evenly; tile ti + 3 into the freed registers; then the barrier
            // that ends the reads of tile ti and publishes what was written.
            // The batch's slots are none of tiles ti and ti + 1 (NTS >= WG + 2).
            const int nu = (u + 1) % PF;
            build(slot ^ 1, ts1, kbuf[nu], vbuf[nu]);
            if (ti % WG == 0)
                stage((ti + 2 + wv) & (NTS - 1), mb);
            else if ((ti + 1) % WG == 0)
                load_meta(ti + 3 + wv, mb);
            load_tile(ti + 3, kbuf[nu], vbuf[nu]);
            __syncthreads();
        }
    }

    const int rowbase = lane & 48;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cc = 16 * nb + 4 * q4 + i;
            const float inv_l = 1.0f / __shfl(bacc[nb][i], rowbase + 2 * NG);
            const int rpos = cc / nrep, rhead = cc % nrep;
            const bool on = cc < a.pb * nrep && rpos < npos;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const float bias = __shfl(bacc[nb][i], rowbase + 2 * g) + __shfl(bacc[nb][i], rowbase + 2 * g + 1);
                const int d0 = HV ? 8 * (col & 7) + 4 * (col >> 3)  // the column's half word
                                  : (g == (low8 ? 0 : 1)) ? 8 * col : 8 * (col ^ 8) + 4;
                float o[4];
#pragma unroll
                for (int mm = 0; mm < 4; ++mm)
                    o[mm] = fmaf(2.0f, acc[nb][4 * g + mm][i], bias) * inv_l;
                if (on) {
                    float *dst = a.out + (((int64_t)b * a.Hq + kvh * nrep + rhead) * a.sq + p0 + rpos) * D + d0;
                    *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 8-bit codes, one block of 16 query columns per wavefront: WG wavefronts
// share each tile's unpacked operands (launched at D = 128 with n_rep <= 16;
// the code also takes D = 64, where the one-wavefront kernel is faster)
//
// The arithmetic of sdpa_prefill_b8_kernel (the codes enter the matrix core
// as exact centred integers; the key scale and bias apply in fp32 after the
// score products, the value scale inside the per-group weights, the value
// bias as a running sum), with WG wavefronts per workgroup on consecutive
// position blocks of one (batch, KV head). They read the same rows, so each
// unpacks 1/WG of a tile's K operands (16-row block x 32 dimensions) and V
// operands (scale group g, dimension mm of the column's four) into a
// two-slot LDS ring, and one wavefront per tile, in turn, stages the tile's
// fp32 factors. One barrier per tile separates building tile t + 1 from the
// reads of tile t.
//
// V operand (g, mm) takes one word per row and lane: lane col reads the word
// of dimensions 64 g + 8 (col & 7) + 4 (col >> 3) .. + 3 (the D = 64 layout
// of the one-wavefront kernel, once per group), so that its builder loads
// only its group's words and needs no lane exchange; value column col of
// the operand is dimension 64 g + 8 (col & 7) + 4 (col >> 3) + mm.
template <int PF, int NB, bool Q32, int WG, int D>
__global__ __launch_bounds__(64 * WG) __attribute__((amdgpu_waves_per_eu(3)))
void sdpa_prefill_b8_wg_kernel(PrefillArgs a)
{
    static_assert(D == 128 || D == 64, "two scale groups, or one");
    static_assert(PF == 2, "tile j's words in register buffer j % 2");
    constexpr int NG = D / 64;   // scale groups of 64
    constexpr int W = D / 4;     // words per row
    constexpr int KM = D / 32;   // score products per 16-row block
    constexpr int KPG = 2;       // of them per scale group
    constexpr float VC = 128.0f;        // centre of the value codes
    constexpr float WS = 64.0f;         // scale of the value weights
    constexpr float VU = 1.0f / 64.0f;  // unit of the value products
    constexpr int PAIRS = PT * NG;      // (row, group) pairs of a tile
    constexpr int NKO = 2 * KM;         // K operands of a tile: (16-row block, 32 dimensions)
    constexpr int NVO = 4 * NG;         // V operands of a tile: (scale group, mm)
    constexpr int KO = NKO / WG;        // of them built by each wavefront
    constexpr int VO = NVO / WG;
    static_assert(NKO % WG == 0 && NVO % WG == 0 && 4 % VO == 0, "operands split evenly, one group per builder");
    static_assert(PAIRS == 64 || PAIRS == 32, "at most one (row, group) pair per lane of the staging wavefront");
    constexpr int QH = Q32 ? 2 : 1;     // query halves: hi (and lo)

    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int q4 = lane >> 4;
    const int col = lane & 15;
    const int kvh = prefill_head(a);
    const int b = blockIdx.z;
    const int nrep = a.n_rep;
    const int p0g = prefill_block(a) * WG * a.pb;                   // first position of the workgroup
    const int p0 = p0g + wv * a.pb;                                 // of this wavefront
    const int npos = max(0, min(a.pb, a.sq - p0));                  // this wavefront's positions (may be none)
    const int t_end = (int)a.q_start + min(p0g + WG * a.pb, a.sq);  // rows [0, t_end) are read
    const int t_all = (int)a.q_start + p0;                          // rows <= t_all are seen by every column
    const int ntile = (t_end + PT - 1) / PT;
    const int64_t kvrow0 = ((int64_t)b * a.Hkv + kvh) * a.cap;

    int cpos[NB], chead[NB];
    bool con[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int cc = 16 * nb + col;
        cpos[nb] = cc / nrep;
        chead[nb] = cc % nrep;
        con[nb] = cc < a.pb * nrep && cpos[nb] < npos;
    }

    const uint32_t rows_ok = (uint32_t)t_end;
    const __amdgpu_buffer_rsrc_t kq = make_rsrc(a.k_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t vq = make_rsrc(a.v_q + kvrow0 * W, rows_ok * W * 4u);
    const __amdgpu_buffer_rsrc_t mres[4] = {
        make_rsrc(a.k_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.k_bias + kvrow0 * NG, rows_ok * NG * 2u),
        make_rsrc(a.v_scale + kvrow0 * NG, rows_ok * NG * 2u), make_rsrc(a.v_bias + kvrow0 * NG, rows_ok * NG * 2u)};

    __shared__ __align__(16) half8 kop[2][NKO][64];  // K operands
    __shared__ __align__(16) half8 vop[2][NVO][64];  // V operands
    // fp32 factors per (row, group) of a tile (c = softmax scale * log2 e):
    // x = s_k c, y = (b_k + 128 s_k) c, z = s_v WS, w = b_v + VC s_v
    __shared__ __align__(16) float4 mring[2][PAIRS];
    __shared__ __align__(16) half8 q_lds[WG][NB][QH][KM][64];
    const float cs = a.score_scale;
    const uint32_t magic8 = opaque_s(kMagic1024x4), magic16 = opaque_s(0x64006400u);
    const uint32_t sel_even = opaque_s(0x04020400u), sel_odd = opaque_s(0x04030401u);
    const uint32_t sel_b[4] = {opaque_s(0x0C040C00u), opaque_s(0x0C050C01u), opaque_s(0x0C060C02u),
                               opaque_s(0x0C070C03u)};

    // this wavefront's operands: K (blk, uu) = (o / KM, o % KM) and V (g, mm)
    // = (v >> 2, v & 3) for o = KO wv + i, v = VO wv + i (one group gv)
    const int gv = (VO * wv) >> 2;
    constexpr uint32_t kNoRows = 0x80000000u;  // > any records size (capacity * D < 2^31 bytes)
    uint32_t kbuf[PF][KO][2];
    uint32_t vbuf[PF][8];
    uint32_t mbuf[PF][4];
    auto load_tile = [&](int ti, uint32_t (&kt)[KO][2], uint32_t (&vt)[8], uint32_t (&mt)[4]) {
        const bool in = ti < ntile;
        const uint32_t moff = in ? (uint32_t)((PT * ti) * NG + lane) * 2u : kNoRows;
#pragma unroll
        for (int arr = 0; arr < 4; ++arr)
            mt[arr] = __builtin_amdgcn_raw_buffer_load_b16(mres[arr], moff, 0, 0);
        const uint32_t base = in ? (uint32_t)(PT * ti) * (uint32_t)(W * 4) : kNoRows;
        // K: row 16 blk + col, dimensions 32 uu + 8 q4 .. + 7 (two words)
#pragma unroll
        for (int i = 0; i < KO; ++i) {
            const int o = KO * wv + i;
            const auto x = __builtin_amdgcn_raw_buffer_load_b64(
                kq, base + (uint32_t)(((16 * (o / KM) + col) * W + 8 * (o % KM) + 2 * q4) * 4), 0, 0);
            kt[i][0] = x[0];
            kt[i][1] = x[1];
        }
        // V: the group-gv word of rows 16 (j >> 2) + 4 q4 + (j & 3)
        const uint32_t voff = base + (uint32_t)((4 * q4 * W + 16 * gv + 2 * (col & 7) + (col >> 3)) * 4);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            vt[j] = __builtin_amdgcn_raw_buffer_load_b32(vq, voff + ((16 * (j >> 2) + (j & 3)) * W) * 4, 0, 0);
    };
    // tile's operands into operand slot `slot`
    auto build = [&](int slot, const uint32_t (&kt)[KO][2], const uint32_t (&vt)[8]) {
#pragma unroll
        for (int i = 0; i < KO; ++i)
            kop[slot][KO * wv + i][lane] = k_operand8(kt[i][0], kt[i][1], magic8, sel_even, sel_odd);
#pragma unroll
        for (int i = 0; i < VO; ++i) {
            const int mm = (VO * wv + i) & 3;
            half2v e[4];
#pragma unroll
            for (int jp = 0; jp < 4; ++jp)
                e[jp] = v_pair8(vt[2 * jp], vt[2 * jp + 1], sel_b[mm], magic16);
            vop[slot][VO * wv + i][lane] = cat8(e[0], e[1], e[2], e[3]);
        }
    };
    // a tile's factors into slot `slot`, from its scale/bias words
    auto stage_meta = [&](int slot, const uint32_t (&mt)[4]) {
        if (PAIRS < 64 && lane >= PAIRS)  // D = 64: lanes 32-63 loaded the next tile's words
            return;
        const float ks = h_val((uint16_t)mt[0]);
        const float kb = h_val((uint16_t)mt[1]);
        const float vs = h_val((uint16_t)mt[2]);
        const float vb = h_val((uint16_t)mt[3]);
        mring[slot][lane] = make_float4(ks * cs, fmaf(128.0f, ks, kb) * cs, vs * WS, fmaf(VC, vs, vb));
    };
    auto fac_xy = [&](int slot, int r, int g) {
        return *reinterpret_cast<const float2 *>(&mring[slot][r * NG + g]);
    };
    auto fac_zw = [&](int slot, int r, int g) {
        return *(reinterpret_cast<const float2 *>(&mring[slot][r * NG + g]) + 1);
    };

    // prologue: tiles 0 and 1 loaded, tile 0 built and staged, tile 2 loaded
#pragma unroll
    for (int u = 0; u < PF; ++u)
        load_tile(u, kbuf[u], vbuf[u], mbuf[u]);
    build(0, kbuf[0], vbuf[0]);
    if (wv == 0)
        stage_meta(0, mbuf[0]);
    load_tile(2, kbuf[0], vbuf[0], mbuf[0]);

    // each block's column query as B operands (kPerm8 order, as in the
    // one-wavefront kernel); qsum: group sums of what the matrix core sees
    float qsum[NB][NG];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int64_t qrow = (((int64_t)b * a.Hq + kvh * nrep + (con[nb] ? chead[nb] : 0)) * a.sq +
                              (con[nb] ? p0 + cpos[nb] : 0)) * D;
        float gs[NG] = {};
#pragma unroll
        for (int uu = 0; uu < KM; ++uu) {
            float x[8];
            if constexpr (Q32) {
                const float *qp = reinterpret_cast<const float *>(a.q) + qrow + 32 * uu + 8 * q4;
                const float4 x0 = *reinterpret_cast<const float4 *>(qp);
                const float4 x1 = *reinterpret_cast<const float4 *>(qp + 4);
                x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
                x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
            } else {
                const half8 h8 = *reinterpret_cast<const half8 *>(reinterpret_cast<const _Float16 *>(a.q) + qrow +
                                                                  32 * uu + 8 * q4);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    x[j] = (float)h8[j];
            }
            half8 qh, ql;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float xv = con[nb] ? x[kPerm8[j]] : 0.0f;
                const _Float16 hi = (_Float16)xv;
                qh[j] = hi;
                if constexpr (Q32) {
                    const _Float16 lo = (_Float16)(xv - (float)hi);
                    ql[j] = lo;
                    gs[uu / KPG] += (float)hi + (float)lo;
                } else {
                    gs[uu / KPG] += (float)hi;
                }
            }
            q_lds[wv][nb][0][uu][lane] = qh;
            if constexpr (Q32)
                q_lds[wv][nb][QH - 1][uu][lane] = ql;
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
            qsum[nb][g] = xrow_sum(gs[g]);
    }
    __syncthreads();

    float m_run[NB], l_run[NB], b_run[NB][NG];
    float4v acc[NB][NVO], accl[NB][NVO];  // [nb][4 g + mm]: hi and lo (x kLoScale) weight halves
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        m_run[nb] = 0.0f;
        l_run[nb] = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g)
            b_run[nb][g] = 0.0f;
#pragma unroll
        for (int m = 0; m < NVO; ++m) {
            acc[nb][m] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
            accl[nb][m] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
        }
    }

#pragma unroll 1
    for (int kk = 0; kk < ntile; kk += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int ti = kk + u;
            const int slot = u;
            const int nu = u ^ 1;

            // tile ti + 1 into the other slot (its words loaded two tiles
            // ago; its factors staged by wavefront (ti + 1) % WG), tile ti + 3
            // into the freed registers
            build(nu, kbuf[nu], vbuf[nu]);
            if (wv == ((ti + 1) & (WG - 1)))
                stage_meta(nu, mbuf[nu]);
            load_tile(ti + 3, kbuf[nu], vbuf[nu], mbuf[nu]);

            // ---- scores of the lane's 8 rows (4 q4 + i, 16 + 4 q4 + i - 4), log2 units
            float sc[NB][8];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                float s[NB][4];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        s[nb][i] = -m_run[nb];
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    float4v sacc[NB];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        sacc[nb] = (float4v){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int k = 0; k < KPG; ++k) {
                        const half8 ka = kop[slot][blk * KM + g * KPG + k][lane];
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int hl = 0; hl < QH; ++hl)
                                sacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                    ka, q_lds[wv][nb][hl][g * KPG + k][lane], sacc[nb], 0, 0, 0);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float2 f = fac_xy(slot, 16 * blk + 4 * q4 + i, g);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            s[nb][i] = fmaf(f.x, sacc[nb][i], fmaf(f.y, qsum[nb][g], s[nb][i]));
                    }
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sc[nb][4 * blk + i] = s[nb][i];
            }
            if (PT * ti + PT - 1 > t_all) {  // uniform: some row is past some column's position
                asm volatile("" ::: "memory");  // keep this a branch
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int lim = t_all + cpos[nb];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int r = PT * ti + 16 * (i >> 2) + 4 * q4 + (i & 3);
                        sc[nb][i] = r <= lim ? sc[nb][i] : -INFINITY;
                    }
                }
            }
            float p[NB][8];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const float mx = max3_raw(max3_raw(sc[nb][0], sc[nb][1], sc[nb][2]),
                                          max3_raw(sc[nb][3], sc[nb][4], sc[nb][5]), max_raw(sc[nb][6], sc[nb][7]));
                // ---- reference raised only when a score exceeds it (the first tile sets it)
                if (ti == 0 || __builtin_amdgcn_ballot_w64(mx > 0.0f) != 0) {
                    const float full = xrow_max(mx, -INFINITY);
                    const bool raise = full > 0.0f || (ti == 0 && full > -INFINITY);
                    const float delta = raise ? full + kHeadroom : 0.0f;
                    m_run[nb] += delta;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        sc[nb][i] -= delta;
                    if (ti != 0) {
                        const float corr = __builtin_amdgcn_exp2f(-delta);
                        l_run[nb] *= corr;
#pragma unroll
                        for (int g = 0; g < NG; ++g)
                            b_run[nb][g] *= corr;
                        float4v corr_row;
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            corr_row[i] = __shfl(corr, 4 * q4 + i);
#pragma unroll
                        for (int m = 0; m < NVO; ++m) {
                            acc[nb][m] *= corr_row;
                            accl[nb][m] *= corr_row;
                        }
                    }
                }
                float lsum = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    p[nb][i] = __builtin_amdgcn_exp2f(sc[nb][i]);
                    lsum += p[nb][i];
                }
                l_run[nb] += lsum;
            }

            // ---- value products, group by group: the weights p s_v WS as hi
            // and lo (x kLoScale) fp16 halves, each V operand serving all NB
            // blocks
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                half8 phi[NB], plo[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    float bsum = 0.0f;
#pragma unroll
                    for (int j = 0; j < 8; j += 2) {
                        const float2 f0 = fac_zw(slot, 16 * (j >> 2) + 4 * q4 + (j & 3), g);
                        const float2 f1 = fac_zw(slot, 16 * ((j + 1) >> 2) + 4 * q4 + ((j + 1) & 3), g);
                        bsum = fmaf(p[nb][j], f0.y, fmaf(p[nb][j + 1], f1.y, bsum));
                        const float w0 = p[nb][j] * f0.x, w1 = p[nb][j + 1] * f1.x;
                        const half2v h = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(w0, w1));
                        const half2v l = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(
                                                                        (w0 - (float)h[0]) * kLoScale,
                                                                        (w1 - (float)h[1]) * kLoScale));
                        phi[nb][j] = h[0]; phi[nb][j + 1] = h[1];
                        plo[nb][j] = l[0]; plo[nb][j + 1] = l[1];
                    }
                    b_run[nb][g] += bsum;
                }
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const half8 bv = vop[slot][4 * g + mm][lane];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        acc[nb][4 * g + mm] =
                            __builtin_amdgcn_mfma_f32_16x16x32_f16(phi[nb], bv, acc[nb][4 * g + mm], 0, 0, 0);
                        accl[nb][4 * g + mm] =
                            __builtin_amdgcn_mfma_f32_16x16x32_f16(plo[nb], bv, accl[nb][4 * g + mm], 0, 0, 0);
                    }
                }
            }
            __syncthreads();  // reads of tile ti done, tile ti + 1 published
        }
    }

    // ---- normalised outputs: row r = 4 q4 + i is column 16 nb + r
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float l_tot = xrow_sum(l_run[nb]);
        float b_tot[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g)
            b_tot[g] = xrow_sum(b_run[nb][g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * q4 + i;
            const int cc = 16 * nb + r;
            const float inv_l = 1.0f / __shfl(l_tot, r);
            const int rpos = cc / nrep, rhead = cc % nrep;
            const bool on = cc < a.pb * nrep && rpos < npos;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const float bias = __shfl(b_tot[g], r);
                const int d0 = 64 * g + 8 * (col & 7) + 4 * (col >> 3);
                float o[4];
#pragma unroll
                for (int mm = 0; mm < 4; ++mm) {
                    const float hi = acc[nb][4 * g + mm][i];
                    const float lo = accl[nb][4 * g + mm][i];
                    o[mm] = (fmaf(lo, VU / kLoScale, hi * VU) + bias) * inv_l;
                }
                if (on) {
                    float *dst = a.out + (((int64_t)b * a.Hq + kvh * nrep + rhead) * a.sq + p0 + rpos) * D + d0;
                    *reinterpret_cast<float4 *>(dst) = make_float4(o[0], o[1], o[2], o[3]);
                }
            }
        }
    }
}

}  // namespace

// n_rep up to the query columns of a wavefront (16 per block: 32 at D = 64
// and 128, 16 at D = 256), where a wavefront then takes one position of all
// its KV head's query heads
bool prefill_supports(int D, int G, int n_rep, int q_dtype, int bits)
{
    return (D == 64 || D == 128 || D == 256) && G == 64 && n_rep >= 1 && n_rep <= (D == 256 ? 16 : 32) &&
           (q_dtype == KVQ_F16 || q_dtype == KVQ_F32) && (bits == 4 || bits == 8);
}

// blocks of 16 query columns per wavefront: two at D = 64 and 128, one at
// D = 256 (8-bit codes in one wavefront with one block at D = 128: 35.8 ms
// against 28.8 ms on the 4096-position chunk); one for 8-bit codes at
// D = 128 with n_rep <= 16, whose workgroups share the tile operands and run
// two wavefronts per SIMD (22.0 ms against 27.9 ms for the chunk; at D = 64
// 6.22 ms against 5.84 ms, so D = 64 keeps the one-wavefront kernel)
constexpr int prefill_nb(int D, int bits, int n_rep)
{
    return D == 256 || (bits == 8 && D == 128 && n_rep <= 16) ? 1 : 2;
}

int prefill_positions_per_block(int n_rep, int D, int bits) { return 16 * prefill_nb(D, bits, n_rep) / n_rep; }

// wavefronts per workgroup (consecutive position blocks of one KV head):
// int4 at D = 128 shares each tile's operands across 8 wavefronts with fp16
// queries, 4 with fp32 queries (whose hi and lo query operands take twice
// the LDS); int4 at D = 64 across 4 (a tile has four K and four V operands);
// 8-bit codes at D = 128 with one block per wavefront across 4 (at most 256
// registers, so that two workgroups share a CU: 22.0 ms on the chunk against
// 23.6 ms in workgroups of 8); one wavefront otherwise
constexpr int prefill_wg(int D, int bits, bool q_f32, int nb)
{
    if (bits == 8)
        return D == 128 && nb == 1 ? 4 : 1;
    return D == 128 ? (q_f32 ? 4 : 8) : D == 64 ? 4 : 1;
}

template <int D>
void launch_prefill_d(const PrefillArgs &a, dim3 grid, hipStream_t s)
{
    constexpr int NB = D == 256 ? 1 : 2;
    constexpr int WG16 = prefill_wg(D, 4, false, NB), WG32 = prefill_wg(D, 4, true, NB);
    constexpr int WB = prefill_wg(D, 8, false, 1);
    if constexpr (D == 128) {
        if (a.bits == 8 && a.pb * a.n_rep <= 16) {
            if (a.q_f32)
                hipLaunchKernelGGL((sdpa_prefill_b8_wg_kernel<2, 1, true, WB, D>), grid, dim3(64 * WB), 0, s, a);
            else
                hipLaunchKernelGGL((sdpa_prefill_b8_wg_kernel<2, 1, false, WB, D>), grid, dim3(64 * WB), 0, s, a);
            return;
        }
    }
    if constexpr (D == 128 || D == 64) {
        if (a.bits == 8 && a.q_f32)
            hipLaunchKernelGGL((sdpa_prefill_b8_kernel<2, NB, true, D>), grid, dim3(64), 0, s, a);
        else if (a.bits == 8)
            hipLaunchKernelGGL((sdpa_prefill_b8_kernel<2, NB, false, D>), grid, dim3(64), 0, s, a);
        else if (a.q_f32)
            hipLaunchKernelGGL((sdpa_prefill_i4_wg_kernel<2, NB, true, WG32, D>), grid, dim3(64 * WG32), 0, s, a);
        else
            hipLaunchKernelGGL((sdpa_prefill_i4_wg_kernel<2, NB, false, WG16, D>), grid, dim3(64 * WG16), 0, s, a);
    } else if (a.bits == 8 && a.q_f32)
        hipLaunchKernelGGL((sdpa_prefill_b8_kernel<2, NB, true, D>), grid, dim3(64), 0, s, a);
    else if (a.bits == 8)
        hipLaunchKernelGGL((sdpa_prefill_b8_kernel<2, NB, false, D>), grid, dim3(64), 0, s, a);
    else if (a.q_f32)
        hipLaunchKernelGGL((sdpa_prefill_i4_kernel<2, NB, true, D>), grid, dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL((sdpa_prefill_i4_kernel<2, NB, false, D>), grid, dim3(64), 0, s, a);
}

hipError_t launch_prefill(const PrefillArgs &a, int batch, hipStream_t s)
{
    const int nb = prefill_nb(a.D, a.bits, a.n_rep);
    if ((a.D != 64 && a.D != 128 && a.D != 256) || (a.bits != 4 && a.bits != 8) || a.pb < 1 ||
        a.pb != 16 * nb / a.n_rep)
        return hipErrorInvalidValue;
    const int64_t per_block = (int64_t)a.pb * prefill_wg(a.D, a.bits, a.q_f32 != 0, nb);
    const int64_t blocks = (a.sq + per_block - 1) / per_block;
    // one row of blocks x Hkv workgroups per batch entry (prefill_head, prefill_block)
    dim3 grid((unsigned)(blocks * a.Hkv), 1u, (unsigned)batch);
    if (a.D == 256)
        launch_prefill_d<256>(a, grid, s);
    else if (a.D == 64)
        launch_prefill_d<64>(a, grid, s);
    else
        launch_prefill_d<128>(a, grid, s);
    return hipGetLastError();
}

}  // namespace kvq
