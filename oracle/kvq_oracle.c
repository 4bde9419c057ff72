/*
 * CPU oracle for int4 group-affine KV-cache quantisation and decode-time
 * attention over the quantised cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it. It shares no code, header, table or constant with
 * the GPU library; it is written from the method's description alone.
 *
 * Sources (page titles as published):
 *  - "Fused int4 Attention for Gemma 4 31B on Apple Silicon", sections
 *    "Background: Why TurboQuant Fails on Gemma 4" (int4 quantisation with a
 *    scale and a bias per group) and "What I Built Instead" (attention
 *    computed on the packed int4 data; the nibble masks 0xF, 0xF0, 0xF00,
 *    0xF000 read the lowest nibble first).
 *  - "turboquant-llama3.170B" README: the kernel paragraph (packed int4 K and
 *    V are dequantised per element, dot product Q.K^T, online softmax, values
 *    accumulated), the split-K paragraph (512-token chunks whose partial
 *    softmax results are reduced in a second phase), the per-layer decode
 *    step (K and V quantised to int4 on append; GQA) and the lesson that
 *    asymmetric int4 quantisation is the practical choice.
 *
 *  - The blog on running Gemma 4 with TurboQuant (devengoratela.com), section
 *    "TurboQuant" with its Hadamard worked example: the normalised Hadamard
 *    rotation applied to K (and here also V and Q) before quantisation.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - Quantiser: per group of G consecutive head-dim values, bias = the group
 *    minimum rounded DOWN to fp16, scale = fl32(fl32(max - bias) / 15)
 *    rounded UP to fp16 (a -0 bias or scale is stored as +0), code = clamp(rint((x - bias) / scale),
 *    0, 15) with every step in IEEE fp32 round-to-nearest-even; code 0 for a
 *    zero scale. The directed fp16 roundings keep [min, max] inside the
 *    representable range [bias, bias + 15 * scale].
 *  - Packing: dimension d of a row goes to word d / 8, bits 4 * (d % 8).
 *  - Cache layout: words [B][Hkv][cap][D/8], scale and bias [B][Hkv][cap][D/G]
 *    (fp16 bits), one row per token.
 *  - 8-bit variant (the Gemma page's "What I Tried" table lists an int8 KV
 *    cache; the blog's decode driver takes 4 or 8 KV bits): the same rule
 *    with 255 in place of 15, codes 0..255, four per word, dimension d at
 *    word d / 4, bits 8 * (d % 4); words [B][Hkv][cap][D/4].
 *  - GQA: query head h reads KV head h / (Hq / Hkv).
 *  - Attention: o = sum_t softmax_t(alpha * q . k^_t) v^_t over all Skv rows,
 *    with k^ = code * scale + bias, evaluated in float64 with an exact
 *    two-pass softmax (max, then exponentials and their sum). The online
 *    softmax of the pages reaches this same value up to rounding.
 *  - Split-K partials of a chunk [c0, c1): m = max_t s_t, l = sum_t
 *    exp(s_t - m), acc_d = sum_t exp(s_t - m) v^_{t,d}; the reduce is
 *    o = sum_c e^{m_c - M} acc_c / sum_c e^{m_c - M} l_c with M = max_c m_c.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fPIC -shared.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ fp16 */
/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits; exponent 0 holds zero and subnormals (quantum 2^-24), exponent 31
 * holds inf and NaN. */

double oracle_f16_to_f64(uint16_t h)
{
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);
    return sign ? -v : v;
}

/* Round a finite or infinite float to the nearest fp16, ties to even.
 * Works on the exact value in double: finds the binade, scales the value so
 * the fp16 quantum of that binade becomes 1, and rounds with rint() (ties to
 * even in the default rounding mode). */
uint16_t oracle_f16_rn(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x))
        return 0x7e00;
    if (a >= 65520.0) /* halfway between 65504 and 2^16 rounds to even = inf */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        /* subnormal range (or zero): quantum 2^-24; a * 2^24 is exact. */
        double q = rint(ldexp(a, 24));
        return sign | (uint16_t)q; /* q == 1024 is the smallest normal */
    }
    int k;
    frexp(a, &k); /* a = f * 2^k, f in [0.5, 1): binade exponent E = k - 1 */
    int E = k - 1;
    double q = rint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E > 15)
        return sign | 0x7c00;
    return sign | (uint16_t)(((E + 15) << 10) | ((int)q - 1024));
}

/* next fp16 toward -inf / +inf (bit patterns; finite inputs) */
static uint16_t f16_next_down(uint16_t h)
{
    if (h == 0x0000 || h == 0x8000)
        return 0x8001;
    return (h & 0x8000) ? (uint16_t)(h + 1) : (uint16_t)(h - 1);
}

static uint16_t f16_next_up(uint16_t h)
{
    if (h == 0x0000 || h == 0x8000)
        return 0x0001;
    return (h & 0x8000) ? (uint16_t)(h - 1) : (uint16_t)(h + 1);
}

/* largest fp16 <= x */
uint16_t oracle_f16_rd(float x)
{
    uint16_t h = oracle_f16_rn(x);
    if (oracle_f16_to_f64(h) > (double)x)
        h = f16_next_down(h);
    return h;
}

/* smallest fp16 >= x */
uint16_t oracle_f16_ru(float x)
{
    uint16_t h = oracle_f16_rn(x);
    if (oracle_f16_to_f64(h) < (double)x)
        h = f16_next_up(h);
    return h;
}

/* ------------------------------------------------------------- quantiser */

/* One group of G values -> G codes in 0..L plus fp16 scale and bias, with
 * L = 2^bits - 1: 15 for the int4 cache, 255 for the int8 variant (the same
 * affine rule with 255 steps; reading for the pages' 8-bit KV option). */
void oracle_quantize_group_bits(const float *x, int G, int bits, uint16_t *scale_out, uint16_t *bias_out,
                                uint8_t *codes)
{
    const float levels = (float)((1 << bits) - 1);
    float lo = x[0], hi = x[0];
    for (int j = 1; j < G; ++j) {
        if (x[j] < lo)
            lo = x[j];
        if (x[j] > hi)
            hi = x[j];
    }
    uint16_t b = oracle_f16_rd(lo);
    if (b == 0x8000)
        b = 0x0000;
    float bf = (float)oracle_f16_to_f64(b);
    float range = hi - bf;      /* fp32, round to nearest */
    float s32 = range / levels; /* fp32, correctly rounded */
    uint16_t s = oracle_f16_ru(s32);
    if (s == 0x8000) /* hi - bias is -0 only when every value is -0 */
        s = 0x0000;
    float sf = (float)oracle_f16_to_f64(s);
    for (int j = 0; j < G; ++j) {
        int q = 0;
        if (sf != 0.0f) {
            float diff = x[j] - bf;
            float u = diff / sf;
            float r = rintf(u);
            if (r < 0.0f)
                r = 0.0f;
            if (r > levels)
                r = levels;
            q = (int)r;
        }
        codes[j] = (uint8_t)q;
    }
    *scale_out = s;
    *bias_out = b;
}

void oracle_quantize_group(const float *x, int G, uint16_t *scale_out, uint16_t *bias_out, uint8_t *codes)
{
    oracle_quantize_group_bits(x, G, 4, scale_out, bias_out, codes);
}

/* codes[D] -> words[D*bits/32]: P = 32/bits codes per word, dimension d at
 * word d/P, bits bits*(d%P) (lowest field first, as the nibble masks of the
 * int4 kernel read; the int8 variant packs bytes the same way) */
void oracle_pack_row_bits(const uint8_t *codes, int D, int bits, uint32_t *words)
{
    const int P = 32 / bits;
    const uint32_t mask = (1u << bits) - 1u;
    for (int w = 0; w < D / P; ++w) {
        uint32_t word = 0;
        for (int j = 0; j < P; ++j)
            word |= ((uint32_t)codes[P * w + j] & mask) << (bits * j);
        words[w] = word;
    }
}

void oracle_unpack_row_bits(const uint32_t *words, int D, int bits, uint8_t *codes)
{
    const int P = 32 / bits;
    const uint32_t mask = (1u << bits) - 1u;
    for (int d = 0; d < D; ++d)
        codes[d] = (uint8_t)((words[d / P] >> (bits * (d % P))) & mask);
}

void oracle_pack_row(const uint8_t *codes, int D, uint32_t *words) { oracle_pack_row_bits(codes, D, 4, words); }

void oracle_unpack_row(const uint32_t *words, int D, uint8_t *codes) { oracle_unpack_row_bits(words, D, 4, codes); }

/* Quantise `rows` rows of D fp32 values (row-major) into packed words
 * [rows][D*bits/32] and fp16 scale/bias [rows][D/G]. */
int oracle_quantize_rows(const float *x, int64_t rows, int D, int G, int bits, uint32_t *words, uint16_t *scale,
                         uint16_t *bias)
{
    if (D <= 0 || G <= 0 || D % G != 0 || D % 8 != 0 || G > 1024 || (bits != 4 && bits != 8))
        return -1;
    const int WR = D * bits / 32;
    uint8_t codes[1024];
    uint8_t rowc[4096];
    if (D > 4096)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * D;
        for (int g = 0; g < D / G; ++g) {
            oracle_quantize_group_bits(xr + g * G, G, bits, &scale[r * (D / G) + g], &bias[r * (D / G) + g],
                                       codes);
            memcpy(rowc + g * G, codes, (size_t)G);
        }
        oracle_pack_row_bits(rowc, D, bits, words + r * WR);
    }
    return 0;
}

/* words/scale/bias of `rows` rows -> float64 values code*scale + bias */
void oracle_dequantize_rows(const uint32_t *words, const uint16_t *scale, const uint16_t *bias, int64_t rows,
                            int D, int G, int bits, double *out)
{
    uint8_t rowc[4096];
    const int WR = D * bits / 32;
    for (int64_t r = 0; r < rows; ++r) {
        oracle_unpack_row_bits(words + r * WR, D, bits, rowc);
        for (int d = 0; d < D; ++d) {
            double s = oracle_f16_to_f64(scale[r * (D / G) + d / G]);
            double b = oracle_f16_to_f64(bias[r * (D / G) + d / G]);
            out[r * D + d] = (double)rowc[d] * s + b;
        }
    }
}

/* ------------------------------------------------------------- attention */

typedef struct {
    const uint32_t *k_q, *v_q;
    const uint16_t *k_scale, *k_bias, *v_scale, *v_bias;
    int B, Hkv, Hq, D, G, bits;
    int64_t cap, skv;
    const double *q; /* [B][Hq][D] */
    double alpha;
    int64_t chunk;   /* 0: whole range, no partials */
    double *out;     /* [B][Hq][D] when chunk == 0 */
    double *part_m, *part_l, *part_acc; /* [B][Hq][C], [B][Hq][C][D] */
    int next_head;   /* work counter, guarded by lock */
    pthread_mutex_t lock;
} attn_job;

/* Dequantised row t of KV head (b, kvh) of one of the two caches. */
static void deq_row(const attn_job *J, int which_v, int b, int kvh, int64_t t, double *row)
{
    int D = J->D, G = J->G, bits = J->bits, P = 32 / bits;
    int64_t base = ((int64_t)b * J->Hkv + kvh) * J->cap + t;
    const uint32_t *w = (which_v ? J->v_q : J->k_q) + base * (D / P);
    const uint16_t *sc = (which_v ? J->v_scale : J->k_scale) + base * (D / G);
    const uint16_t *bi = (which_v ? J->v_bias : J->k_bias) + base * (D / G);
    for (int d = 0; d < D; ++d) {
        unsigned code = (w[d / P] >> (bits * (d % P))) & ((1u << bits) - 1u);
        row[d] = (double)code * oracle_f16_to_f64(sc[d / G]) + oracle_f16_to_f64(bi[d / G]);
    }
}

/* Exact two-pass softmax attention of query head (b, h) over rows [t0, t1):
 * returns m and l, and acc (unnormalised, length D). */
static void attend_range(const attn_job *J, int b, int h, int64_t t0, int64_t t1, double *scores, double *row,
                         double *m_out, double *l_out, double *acc)
{
    int D = J->D;
    int kvh = h / (J->Hq / J->Hkv);
    const double *q = J->q + ((int64_t)b * J->Hq + h) * D;
    double m = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
        deq_row(J, 0, b, kvh, t, row);
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += q[d] * row[d];
        double s = J->alpha * dot;
        scores[t - t0] = s;
        if (s > m)
            m = s;
    }
    double l = 0.0;
    for (int d = 0; d < D; ++d)
        acc[d] = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        double w = exp(scores[t - t0] - m);
        l += w;
        deq_row(J, 1, b, kvh, t, row);
        for (int d = 0; d < D; ++d)
            acc[d] += w * row[d];
    }
    *m_out = m;
    *l_out = l;
}

static void *attn_worker(void *arg)
{
    attn_job *J = (attn_job *)arg;
    int64_t span = J->chunk > 0 ? J->chunk : J->skv;
    double *scores = (double *)malloc(sizeof(double) * (size_t)span);
    double *row = (double *)malloc(sizeof(double) * (size_t)J->D);
    double *acc = (double *)malloc(sizeof(double) * (size_t)J->D);
    if (!scores || !row || !acc) {
        free(scores);
        free(row);
        free(acc);
        return (void *)1;
    }
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int idx = J->next_head++;
        pthread_mutex_unlock(&J->lock);
        if (idx >= J->B * J->Hq)
            break;
        int b = idx / J->Hq, h = idx % J->Hq;
        if (J->chunk <= 0) {
            double m, l;
            attend_range(J, b, h, 0, J->skv, scores, row, &m, &l, acc);
            double *o = J->out + (int64_t)idx * J->D;
            for (int d = 0; d < J->D; ++d)
                o[d] = acc[d] / l;
        } else {
            int64_t C = (J->skv + J->chunk - 1) / J->chunk;
            for (int64_t c = 0; c < C; ++c) {
                int64_t t0 = c * J->chunk;
                int64_t t1 = t0 + J->chunk < J->skv ? t0 + J->chunk : J->skv;
                double m, l;
                attend_range(J, b, h, t0, t1, scores, row, &m, &l, acc);
                J->part_m[(int64_t)idx * C + c] = m;
                J->part_l[(int64_t)idx * C + c] = l;
                memcpy(J->part_acc + ((int64_t)idx * C + c) * J->D, acc, sizeof(double) * (size_t)J->D);
            }
        }
    }
    free(scores);
    free(row);
    free(acc);
    return NULL;
}

static int run_attention(attn_job *J, int nthreads)
{
    if (J->B <= 0 || J->Hkv <= 0 || J->Hq <= 0 || J->Hq % J->Hkv != 0 || J->D <= 0 || J->G <= 0 ||
        J->D % J->G != 0 || J->D % 8 != 0 || J->skv <= 0 || J->skv > J->cap)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    J->next_head = 0;
    pthread_mutex_init(&J->lock, NULL);
    pthread_t th[256];
    int started = 0, rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, attn_worker, J) != 0)
            break;
        ++started;
    }
    if (started == 0)
        rc = attn_worker(J) ? -2 : 0;
    for (int i = 0; i < started; ++i) {
        void *r = NULL;
        pthread_join(th[i], &r);
        if (r)
            rc = -2;
    }
    pthread_mutex_destroy(&J->lock);
    return rc;
}

/* Exact decode attention: out[B][Hq][D] (float64). */
int oracle_sdpa(const uint32_t *k_q, const uint32_t *v_q, const uint16_t *k_scale, const uint16_t *k_bias,
                const uint16_t *v_scale, const uint16_t *v_bias, int B, int Hkv, int D, int G, int bits, int64_t cap,
                int64_t skv, const double *q, int Hq, double alpha, double *out, int nthreads)
{
    if (bits != 4 && bits != 8)
        return -1;
    attn_job J;
    memset(&J, 0, sizeof J);
    J.k_q = k_q; J.v_q = v_q; J.k_scale = k_scale; J.k_bias = k_bias; J.v_scale = v_scale; J.v_bias = v_bias;
    J.B = B; J.Hkv = Hkv; J.Hq = Hq; J.D = D; J.G = G; J.bits = bits; J.cap = cap; J.skv = skv;
    J.q = q; J.alpha = alpha; J.chunk = 0; J.out = out;
    return run_attention(&J, nthreads);
}

/* Split-K partials per chunk of `chunk` rows (the last chunk is shorter). */
int oracle_sdpa_partials(const uint32_t *k_q, const uint32_t *v_q, const uint16_t *k_scale,
                         const uint16_t *k_bias, const uint16_t *v_scale, const uint16_t *v_bias, int B, int Hkv,
                         int D, int G, int bits, int64_t cap, int64_t skv, const double *q, int Hq, double alpha,
                         int64_t chunk, double *part_m, double *part_l, double *part_acc, int nthreads)
{
    if (chunk <= 0 || (bits != 4 && bits != 8))
        return -1;
    attn_job J;
    memset(&J, 0, sizeof J);
    J.k_q = k_q; J.v_q = v_q; J.k_scale = k_scale; J.k_bias = k_bias; J.v_scale = v_scale; J.v_bias = v_bias;
    J.B = B; J.Hkv = Hkv; J.Hq = Hq; J.D = D; J.G = G; J.bits = bits; J.cap = cap; J.skv = skv;
    J.q = q; J.alpha = alpha; J.chunk = chunk;
    J.part_m = part_m; J.part_l = part_l; J.part_acc = part_acc;
    return run_attention(&J, nthreads);
}

/* Combine split-K partials of `heads` heads with C chunks each. */
void oracle_combine_partials(const double *part_m, const double *part_l, const double *part_acc, int64_t heads,
                             int64_t C, int D, double *out)
{
    for (int64_t i = 0; i < heads; ++i) {
        double M = -INFINITY;
        for (int64_t c = 0; c < C; ++c)
            if (part_m[i * C + c] > M)
                M = part_m[i * C + c];
        double den = 0.0;
        for (int d = 0; d < D; ++d)
            out[i * D + d] = 0.0;
        for (int64_t c = 0; c < C; ++c) {
            double f = exp(part_m[i * C + c] - M);
            den += f * part_l[i * C + c];
            for (int d = 0; d < D; ++d)
                out[i * D + d] += f * part_acc[(i * C + c) * D + d];
        }
        for (int d = 0; d < D; ++d)
            out[i * D + d] /= den;
    }
}

/* ----------------------------------------------------- Hadamard rotation */
/* The normalised Hadamard transform of the TurboQuant explainer blog on
 * running Gemma 4 with TurboQuant (devengoratela.com; its "TurboQuant"
 * section, the worked example under it and "Transform Results", and step
 * "1. Vector Rotation"): a row x of length n (a power of two) becomes
 * y = H_n x / sqrt(n), where H_n is the Hadamard matrix in Sylvester order
 * (the matrix of the example: H_2n = [[H_n, H_n], [H_n, -H_n]]), whose entry
 * (i, j) is (-1)^(number of bits set in i & j). The normalised matrix is
 * orthogonal and its own inverse, which is how the blog recovers the vector.
 *
 * Written from the definition: the sum over j is a plain loop in float64,
 * then one multiplication by c = 1.0 / sqrt(n) (correctly rounded sqrt and
 * division). For fp16 inputs every term and partial sum is a multiple of
 * 2^-24 below 2^23 in magnitude, so the sum is exact in float64 whatever the
 * order, and y = fl64(S * c) is a single rounding of the exact value. */
static int parity_of(unsigned v)
{
    int p = 0;
    while (v) {
        p ^= 1;
        v &= v - 1;
    }
    return p;
}

int oracle_hadamard_rows(const double *x, int64_t rows, int n, double *out)
{
    if (n < 1 || (n & (n - 1)) != 0)
        return -1;
    const double c = 1.0 / sqrt((double)n);
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * n;
        double *yr = out + r * n;
        for (int i = 0; i < n; ++i) {
            double s = 0.0;
            for (int j = 0; j < n; ++j)
                s += parity_of((unsigned)(i & j)) ? -xr[j] : xr[j];
            yr[i] = s * c;
        }
    }
    return 0;
}

/* ------------------------------------------------- array forms for tests */

void oracle_f16_to_f64_n(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f16_to_f64(h[i]);
}

/* mode 0: nearest even, 1: down, 2: up */
void oracle_f16_round_n(const float *x, int64_t n, int mode, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = mode == 0 ? oracle_f16_rn(x[i]) : mode == 1 ? oracle_f16_rd(x[i]) : oracle_f16_ru(x[i]);
}
