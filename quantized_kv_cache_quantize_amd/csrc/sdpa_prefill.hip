// Prefill-side attention over the int4 cache, matrix-core kernel for gfx950.
//
// The README's hybrid paragraph routes Sq > 1 (prefill) to a separate
// attention on fp16 K/V and only then quantises the rows into the cache; here
// the prefill block's queries read the quantised cache directly, the same
// packed rows the decode kernel reads. Query i of the block is position
// q_start + i; its K/V row is cache row q_start + i (appended before the
// call), and it attends to rows [0, q_start + i] (causal).
//
// Work split: one wavefront per (32 / n_rep query positions x the n_rep heads
// of a KV head, batch), streaming the rows its positions can see in 32-row
// tiles. With GQA the n_rep heads of a KV head and the block's positions all
// read the same rows, so every K/V tile is fetched and unpacked once for 32
// query columns (two blocks of 16, each the N side of its own matrix
// instructions).
//
// Scores (per tile): S^T[t][c] = Kcodes[t][:] . Q[c][:] on
// v_mfma_f32_16x16x32_f16, A = K codes (16 rows, 32 dimensions), B = the
// queries of a 16-column block. A lane loads the K words of its row strided
// by 4 words, so each instruction's 32 dimensions lie in one scale group and
// the group's scale and bias apply in fp32 afterwards (the factored form of
// the Gemma page's "What I Built Instead"): s = sum_g s_g (q . code)_g +
// b_g (sum q)_g. K codes enter as the fp16 subnormals n * 2^-20, as in the
// decode kernel.
//
// Values: O[c][d] += P'_g[c][t] . Vcodes[t][d] per scale group g, with the
// weights p * s_v of group g as hi and lo fp16 halves (lo scaled by 2^11) in
// separate accumulators, and the value codes centred by 8 (one accumulator
// per output across all the rows: with normal centred operands its error on
// the outlier workload's 65536 rows matches that of fp32 flushes every 512
// rows, measured). A lane's value
// word holds eight dimensions of one group; the operand of group g takes the
// four dimensions it lacks from lane l ^ 8 with a bank-masked DPP move (the
// layout of the decode kernel's two-group path).
//
// Softmax: per query column, relative to a reference raised (with headroom)
// only when a score exceeds it, as in the decode kernel; the output is
// normalised in the kernel (no split over rows, so no partial state).

#include "kvq_internal.h"
#include "mfma_common.h"

namespace kvq {
namespace {

constexpr int PT = 32;  // rows per tile

// D = 128, two scale groups of 64, fp16 queries, int4 codes; NB blocks of
// 16 query columns per wavefront (every unpacked K and V operand feeds NB
// matrix instructions); PF tiles in flight. Operands are unpacked right
// before the instruction that reads them and the scale/bias factors read
// from LDS where they are used. NB = 1 fits a wavefront in 256 registers
// (two per SIMD). NB = 2 runs one wavefront per SIMD; its query operands
// wait in LDS (read back every tile) to ease the register pressure, yet the
// compiler still keeps part of the state in accumulation registers and
// copies it around the matrix instructions. Measured on the Llama layer's
// 4096-position chunk at row 61440: NB = 1 30.4 ms, NB = 2 with the queries
// in registers 26.9 ms, NB = 2 with them in LDS 25.5 ms.
//
// BITS = 8 (byte codes, four per word): the K and V codes enter as the exact
// centred integers n - 128 through the byte permutes of the decode kernel
// (k_operand8, v_pair8), the value weights are carried times WS = 2^6 (as
// there, to keep their fp16 halves clear of the subnormal range) and the
// value products are multiplied by VU = 1 / WS at the end.
//
// Q32 (fp32 queries, e.g. a query rotated for a Hadamard-rotated cache): the
// query is split into fp16 hi and lo halves, hi + lo exact to 22 bits, each
// the B operand of its own score product (as in the decode kernel).
//
// D = 256 (four scale groups): the value words of a row come in VS = D / 128
// sets of 16 words, each set two scale groups handled as the D = 128 layout
// handles its two; NB = 1 there (the accumulators of one block already take
// what two blocks take at D = 128).
template <int PF, int NB, int BITS, bool Q32, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NB == 1 && D == 128 ? 2 : 1)))
void sdpa_prefill_mfma_kernel(PrefillArgs a)
{
    constexpr bool B8 = BITS == 8;
    constexpr int NG = D / 64;   // scale groups of 64
    constexpr int VS = D / 128;  // sets of 16 value words (two groups each)
    constexpr int W = D * BITS / 32;  // words per row
    constexpr int KW = BITS / 4;      // words per eight dimensions
    constexpr int KM = D / 32;        // score products per 16-row block
    constexpr int KPG = KM / NG;      // of them per scale group
    constexpr float VC = B8 ? 128.0f : 8.0f;        // centre of the value codes
    constexpr float WS = B8 ? 64.0f : 1.0f;         // scale of the value weights
    constexpr float VU = B8 ? 1.0f / 64.0f : 1.0f;  // unit of the value products
    constexpr int PAIRS = PT * NG;
    constexpr int MP = PAIRS / 64;  // (row, group) pairs per lane
    static_assert(PAIRS % 64 == 0, "whole pairs per lane");
    constexpr bool QLDS = NB > 1 || D > 128;  // query operands in LDS

    const int lane = threadIdx.x;
    const int q4 = lane >> 4;
    const int col = lane & 15;
    const int kvh = blockIdx.y;
    const int b = blockIdx.z;
    const int nrep = a.n_rep;
    const int p0 = blockIdx.x * a.pb;              // first position of the block
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
    const Unpacker unpack = Unpacker::make();
    const float cs = a.score_scale;
    const float csk = B8 ? cs : cs * 1048576.0f;
    const uint32_t m_fine = opaque_s_if<!B8>(0x00F000F0u);
    // 8-bit operands: the magic exponent bytes and the byte selectors of
    // k_operand8 and v_pair8
    const uint32_t magic8 = opaque_s_if<B8>(kMagic1024x4), magic16 = opaque_s_if<B8>(0x64006400u);
    const uint32_t sel_even = opaque_s_if<B8>(0x04020400u), sel_odd = opaque_s_if<B8>(0x04030401u);
    const uint32_t sel_b[4] = {opaque_s_if<B8>(0x0C040C00u), opaque_s_if<B8>(0x0C050C01u),
                               opaque_s_if<B8>(0x0C060C02u), opaque_s_if<B8>(0x0C070C03u)};

    constexpr uint32_t kNoRows = 0x80000000u;  // > any records size (capacity * D * BITS / 8 < 2^31)
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
                if constexpr (B8) {
                    const auto x = __builtin_amdgcn_raw_buffer_load_b64(kq, off + 16 * KW * uu, 0, 0);
                    kt[blk][uu][0] = x[0];
                    kt[blk][uu][1] = x[1];
                } else {
                    kt[blk][uu][0] = __builtin_amdgcn_raw_buffer_load_b32(kq, off + 16 * uu, 0, 0);
                }
            }
        }
        // V: dimensions 128 s2 + 8 col .. + 7 (KW words) of rows 16 (j >> 2) + 4 q4 + (j & 3)
#pragma unroll
        for (int s2 = 0; s2 < VS; ++s2) {
            const uint32_t voff = base + (uint32_t)((4 * q4 * W + KW * (16 * s2 + col)) * 4);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t o = voff + ((16 * (j >> 2) + (j & 3)) * W) * 4;
                if constexpr (B8) {
                    const auto x = __builtin_amdgcn_raw_buffer_load_b64(vq, o, 0, 0);
                    vt[s2][2 * j] = x[0];
                    vt[s2][2 * j + 1] = x[1];
                } else {
                    vt[s2][j] = __builtin_amdgcn_raw_buffer_load_b32(vq, o, 0, 0);
                }
            }
        }
    };
    auto stage_meta = [&](int slot, const uint32_t (&mt)[MP][4]) {
#pragma unroll
        for (int pp = 0; pp < MP; ++pp) {
            const float ks = h_val((uint16_t)mt[pp][0]);
            const float kb = h_val((uint16_t)mt[pp][1]);
            const float vs = h_val((uint16_t)mt[pp][2]);
            const float vb = h_val((uint16_t)mt[pp][3]);
            mring[slot][lane + 64 * pp] =
                make_float4(ks * csk, (B8 ? fmaf(128.0f, ks, kb) : kb) * cs, vs * WS, fmaf(VC, vs, vb));
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
                const float xv = con[nb] ? x[B8 ? kPerm8[j] : kPerm[j]] : 0.0f;
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
    float4v acc[NB][8 * VS], accl[NB][8 * VS];  // [nb][8 s2 + 4 g + mm]: hi and lo (x kLoScale) weight halves
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        m_run[nb] = 0.0f;
        l_run[nb] = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g)
            b_run[nb][g] = 0.0f;
#pragma unroll
        for (int m = 0; m < 8 * VS; ++m) {
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
                        half8 ka;
                        if constexpr (B8)
                            ka = k_operand8(kw[0], kw[KW - 1], magic8, sel_even, sel_odd);
                        else
                            ka = k_operand_sub(kw[0], m_fine);
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
                        for (int m = 0; m < 8 * VS; ++m) {
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
            // l ^ 8, and every unpacked operand serves all NB blocks. int4:
            // rows (2jp, 2jp + 1) interleaved nibble-pair by nibble-pair;
            // 8-bit: the same exchange on whole words (row r's two words hold
            // dimensions 0..3 and 4..7)
#pragma unroll
            for (int s2 = 0; s2 < VS; ++s2) {
                const uint32_t(&vw)[8 * KW] = vbuf[u][s2];
                uint32_t bx[2][4 * KW];
                if constexpr (B8) {
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        bx[0][r] = take_half_row<0xC>(vw[2 * r], vw[2 * r + 1]);
                        bx[1][r] = take_half_row<0x3>(vw[2 * r], vw[2 * r + 1]);
                    }
                } else {
#pragma unroll
                    for (int jp = 0; jp < 4; ++jp) {
                        const uint32_t xw = __builtin_amdgcn_perm(vw[2 * jp + 1], vw[2 * jp], 0x05040100u);
                        const uint32_t yw = __builtin_amdgcn_perm(vw[2 * jp + 1], vw[2 * jp], 0x07060302u);
                        bx[0][jp] = take_half_row<0xC>(xw, yw);
                        bx[1][jp] = take_half_row<0x3>(xw, yw);
                    }
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
                        for (int jp = 0; jp < 4; ++jp) {
                            if constexpr (B8)
                                e[jp] = v_pair8(bx[g][2 * jp], bx[g][2 * jp + 1], sel_b[mm], magic16);
                            else
                                e[jp] = unpack.one(bx[g][jp], mm);
                        }
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
                const int d0 = 128 * s2 + ((g == (low8 ? 0 : 1)) ? 8 * col : 8 * (col ^ 8) + 4);
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

}  // namespace

bool prefill_supports(int D, int G, int n_rep, int q_dtype, int bits)
{
    return (D == 128 || D == 256) && G == 64 && n_rep >= 1 && n_rep <= 16 &&
           (q_dtype == KVQ_F16 || q_dtype == KVQ_F32) && (bits == 4 || bits == 8);
}

// blocks of 16 query columns per wavefront: two at D = 128 (8-bit codes with
// one block: 35.8 ms against 28.8 ms on the 4096-position chunk), one at
// D = 256
constexpr int prefill_nb(int D) { return D == 256 ? 1 : 2; }

int prefill_positions_per_block(int n_rep, int D) { return 16 * prefill_nb(D) / n_rep; }

template <int D>
void launch_prefill_d(const PrefillArgs &a, dim3 grid, hipStream_t s)
{
    constexpr int NB = prefill_nb(D);
    if (a.bits == 8 && a.q_f32)
        hipLaunchKernelGGL((sdpa_prefill_mfma_kernel<2, NB, 8, true, D>), grid, dim3(64), 0, s, a);
    else if (a.bits == 8)
        hipLaunchKernelGGL((sdpa_prefill_mfma_kernel<2, NB, 8, false, D>), grid, dim3(64), 0, s, a);
    else if (a.q_f32)
        hipLaunchKernelGGL((sdpa_prefill_mfma_kernel<2, NB, 4, true, D>), grid, dim3(64), 0, s, a);
    else
        hipLaunchKernelGGL((sdpa_prefill_mfma_kernel<2, NB, 4, false, D>), grid, dim3(64), 0, s, a);
}

hipError_t launch_prefill(const PrefillArgs &a, int batch, hipStream_t s)
{
    if ((a.D != 128 && a.D != 256) || a.pb < 1 || a.pb * a.n_rep > 16 * prefill_nb(a.D) ||
        (a.bits != 4 && a.bits != 8))
        return hipErrorInvalidValue;
    const int64_t blocks = (a.sq + a.pb - 1) / a.pb;
    dim3 grid((unsigned)blocks, (unsigned)a.Hkv, (unsigned)batch);
    if (a.D == 256)
        launch_prefill_d<256>(a, grid, s);
    else
        launch_prefill_d<128>(a, grid, s);
    return hipGetLastError();
}

}  // namespace kvq
