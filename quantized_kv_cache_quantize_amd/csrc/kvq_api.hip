// C-ABI entry points of libkvq: argument validation on the host, then
// kernel launches on the caller's stream. Nothing here allocates, frees or
// synchronises. Every check runs before the first HIP call, so an invalid
// request returns its status without touching the device (and without
// needing one).
#include <math.h>

#include <mutex>

#include "kvq_internal.h"

using namespace kvq;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// bits per code of a cache: 4 (also the zero of a cache set up before the
// field existed) or 8; 0 for anything else
int cache_bits(const kvq_cache *c) { return c->bits == 0 || c->bits == 4 ? 4 : c->bits == 8 ? 8 : 0; }

int check_cache(const kvq_cache *c)
{
    if (!c)
        return KVQ_E_NULL;
    if (!c->k_q || !c->v_q || !c->k_scale || !c->k_bias || !c->v_scale || !c->v_bias)
        return KVQ_E_NULL;
    if (c->batch < 1 || c->batch > 65535 || c->kv_heads < 1 || c->kv_heads > 65535 || c->capacity < 1)
        return KVQ_E_SHAPE;
    if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
        return KVQ_E_SHAPE;
    if (c->group != 32 && c->group != 64 && c->group != 128)
        return KVQ_E_SHAPE;
    if (c->head_dim % c->group != 0)
        return KVQ_E_SHAPE;
    const int bits = cache_bits(c);
    if (!bits)
        return KVQ_E_SHAPE;
    // keep every element index far inside int64, and the code bytes of one
    // (batch, KV head) addressable with 32-bit offsets (with 64 KiB to spare)
    if (c->capacity > ((int64_t)1 << 40) / ((int64_t)c->batch * c->kv_heads))
        return KVQ_E_SHAPE;
    if (c->capacity * (c->head_dim * bits / 8) > 0x7fff0000)
        return KVQ_E_SHAPE;
    if (!aligned16(c->k_q) || !aligned16(c->v_q) || !aligned16(c->k_scale) || !aligned16(c->k_bias) ||
        !aligned16(c->v_scale) || !aligned16(c->v_bias))
        return KVQ_E_ALIGN;
    return KVQ_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_E_LAUNCH; }

}  // namespace

extern "C" {

const char *kvq_version(void) { return "kvq 0.1.0 gfx950"; }

const char *kvq_status_str(int status)
{
    switch (status) {
    case KVQ_OK:
        return "ok";
    case KVQ_E_NULL:
        return "null pointer";
    case KVQ_E_SHAPE:
        return "invalid size or shape";
    case KVQ_E_ALIGN:
        return "pointer not 16-byte aligned";
    case KVQ_E_CAPACITY:
        return "rows beyond cache capacity";
    case KVQ_E_DTYPE:
        return "unknown element type";
    case KVQ_E_LAUNCH:
        return "kernel launch failed";
    case KVQ_E_UNSUPPORTED:
        return "shape not supported by the requested kernel";
    case KVQ_E_SCRATCH:
        return "request needs more than the library's static scratch";
    default:
        return "unknown status";
    }
}

int64_t kvq_num_chunks(int64_t skv, int32_t chunk)
{
    if (skv <= 0 || chunk <= 0)
        return 0;
    return (skv + chunk - 1) / chunk;
}

int64_t kvq_cache_bytes(int32_t batch, int32_t kv_heads, int32_t head_dim, int32_t group, int64_t capacity,
                        int32_t bits)
{
    if (batch < 1 || kv_heads < 1 || head_dim < 8 || head_dim % 8 || group < 1 || head_dim % group || capacity < 1)
        return 0;
    if (bits == 0)
        bits = 4;
    if (bits != 4 && bits != 8)
        return 0;
    const int64_t rows = (int64_t)batch * kv_heads * capacity;
    const int64_t per_row = head_dim * bits / 8 + 2 * 2 * (head_dim / group);  // codes + fp16 scale and bias
    return 2 * rows * per_row;                                         // K and V
}

}  // extern "C"

namespace {

int append_impl(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int dtype, int64_t n_new,
                void *stream, bool rotate)
{
    int st = check_cache(cache);
    if (st)
        return st;
    if (dtype != KVQ_F16 && (dtype != KVQ_F32 || rotate))
        return KVQ_E_DTYPE;
    if (len < 0 || n_new < 0)
        return KVQ_E_SHAPE;
    if (len > cache->capacity || n_new > cache->capacity - len)
        return KVQ_E_CAPACITY;
    if (n_new == 0)
        return KVQ_OK;
    if (!k_new || !v_new)
        return KVQ_E_NULL;
    if (!aligned16(k_new) || !aligned16(v_new))
        return KVQ_E_ALIGN;
    const int64_t rows = (int64_t)cache->batch * cache->kv_heads * n_new;
    if ((rows * (cache->head_dim / 8) + 255) / 256 > 0x7fffffff)
        return KVQ_E_SHAPE;

    QuantizeArgs a;
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_q = cache->k_q;
    a.v_q = cache->v_q;
    a.k_scale = cache->k_scale;
    a.k_bias = cache->k_bias;
    a.v_scale = cache->v_scale;
    a.v_bias = cache->v_bias;
    a.rows = rows;
    a.n_new = n_new;
    a.len = len;
    a.cap = cache->capacity;
    a.D = cache->head_dim;
    a.G = cache->group;
    a.bits = cache_bits(cache);
    a.rot_scale = rotate ? 1.0 / sqrt((double)cache->head_dim) : 0.0;
    return launch_status(launch_quantize(a, dtype, (hipStream_t)stream));
}

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

}  // namespace

extern "C" {

int kvq_quantize_kv_append(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int dtype,
                           int64_t n_new, void *stream)
{
    return append_impl(cache, len, k_new, v_new, dtype, n_new, stream, false);
}

int kvq_quantize_kv_append_rotated(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new,
                                   int dtype, int64_t n_new, void *stream)
{
    return append_impl(cache, len, k_new, v_new, dtype, n_new, stream, true);
}

int kvq_hadamard_rotate(const void *x, int dtype, int64_t rows, int32_t head_dim, float *out, void *stream)
{
    if (dtype != KVQ_F16 && dtype != KVQ_F32)
        return KVQ_E_DTYPE;
    if (rows < 0 || (head_dim != 64 && head_dim != 128 && head_dim != 256))
        return KVQ_E_SHAPE;
    if (rows == 0)
        return KVQ_OK;
    if (!x || !out)
        return KVQ_E_NULL;
    if (!aligned16(x) || !aligned16(out))
        return KVQ_E_ALIGN;
    if (rows > ((int64_t)1 << 40) / head_dim || (rows * (head_dim / 8) + 255) / 256 > 0x7fffffff)
        return KVQ_E_SHAPE;
    const int64_t n = rows * head_dim;
    // in place only as fp32 -> fp32 on the same rows
    if (overlaps(x, n * (dtype == KVQ_F16 ? 2 : 4), out, n * 4) && !(dtype == KVQ_F32 && (const void *)out == x))
        return KVQ_E_SHAPE;
    RotateArgs a;
    a.x = x;
    a.out = out;
    a.rows = rows;
    a.D = head_dim;
    a.scale = 1.0 / sqrt((double)head_dim);
    return launch_status(launch_rotate(a, dtype, (hipStream_t)stream));
}

namespace {

// A validated partial-phase request: its kernel arguments and whether it runs
// on the matrix cores.
struct PartialPlan {
    PartialArgs a;
    bool use_mfma;
};

int prepare_partial(const kvq_cache *cache, int64_t skv, const void *q, int q_dtype, int32_t Hq, float softmax_scale,
                    int32_t chunk, float *part_m, float *part_l, float *part_acc, int kernel, PartialPlan &p)
{
    int st = check_cache(cache);
    if (st)
        return st;
    if (!q || !part_m || !part_l || !part_acc)
        return KVQ_E_NULL;
    if (q_dtype != KVQ_F16 && q_dtype != KVQ_F32)
        return KVQ_E_DTYPE;
    if (skv < 1 || chunk < 1 || Hq < 1 || Hq % cache->kv_heads != 0 || !isfinite(softmax_scale))
        return KVQ_E_SHAPE;
    if ((int64_t)cache->batch * Hq > 0x7fffffff)
        return KVQ_E_SHAPE;
    if (skv > cache->capacity)
        return KVQ_E_CAPACITY;
    if (!aligned16(q) || !aligned16(part_m) || !aligned16(part_l) || !aligned16(part_acc))
        return KVQ_E_ALIGN;
    const int64_t C = kvq_num_chunks(skv, chunk);
    if (C > 0x7fffffff)
        return KVQ_E_SHAPE;
    if (kernel < KVQ_KERNEL_AUTO || kernel > KVQ_KERNEL_MFMA_WAVE)
        return KVQ_E_SHAPE;
    const int n_rep = Hq / cache->kv_heads;
    const int bits = cache_bits(cache);
    const bool want_mfma = kernel == KVQ_KERNEL_MFMA || kernel == KVQ_KERNEL_MFMA_SPLIT ||
                           kernel == KVQ_KERNEL_MFMA_WAVE;
    // 8-bit caches and head_dim 64 have the one-wavefront matrix-core kernel only
    const bool wave_only = bits == 8 || cache->head_dim == 64;
    if (wave_only && kernel == KVQ_KERNEL_MFMA_SPLIT)
        return KVQ_E_UNSUPPORTED;

    PartialArgs &a = p.a;
    a.k_q = cache->k_q;
    a.v_q = cache->v_q;
    a.k_scale = cache->k_scale;
    a.k_bias = cache->k_bias;
    a.v_scale = cache->v_scale;
    a.v_bias = cache->v_bias;
    a.q = q;
    a.part_m = part_m;
    a.part_l = part_l;
    a.part_acc = part_acc;
    a.cap = cache->capacity;
    a.skv = skv;
    a.num_chunks = C;
    a.chunk = chunk;
    a.Hkv = cache->kv_heads;
    a.Hq = Hq;
    a.n_rep = n_rep;
    a.G = cache->group;
    const int split = mfma_head_split(cache->head_dim, cache->group, n_rep);
    a.head_split = split > 0 ? split : 1;
    a.bits = bits;
    a.score_scale = softmax_scale * kLog2e;
    a.k_new = nullptr;
    a.v_new = nullptr;
    a.append_row = -1;
    a.append_dtype = KVQ_F16;
    a.rotate = 0;
    a.q_f16 = 0;
    a.rot_scale = 0.0;
    a.merge_ws = nullptr;
    a.counters = nullptr;
    a.out = nullptr;
    a.nwg = 0;
    const bool mfma_ok = mfma_supports(cache->head_dim, cache->group, n_rep, chunk) &&
                         (!wave_only || mfma_one_wave_ok(a, cache->head_dim, cache->batch));
    if (want_mfma && !mfma_ok)
        return KVQ_E_UNSUPPORTED;
    if (kernel == KVQ_KERNEL_MFMA_WAVE && !mfma_one_wave_ok(a, cache->head_dim, cache->batch))
        return KVQ_E_UNSUPPORTED;
    p.use_mfma = want_mfma || (kernel == KVQ_KERNEL_AUTO && mfma_ok);
    return KVQ_OK;
}

int launch_plan(const PartialPlan &p, const kvq_cache *cache, int q_dtype, int kernel, const Launch &l)
{
    hipError_t e = p.use_mfma ? launch_partial_mfma(p.a, cache->head_dim, q_dtype, cache->batch, kernel, l)
                              : launch_partial_valu(p.a, cache->head_dim, q_dtype, cache->batch, l);
    return launch_status(e);
}

int partial_impl(const kvq_cache *cache, int64_t skv, const void *q, int q_dtype, int32_t Hq, float softmax_scale,
                 int32_t chunk, float *part_m, float *part_l, float *part_acc, int kernel, const Launch &l)
{
    PartialPlan p;
    const int st = prepare_partial(cache, skv, q, q_dtype, Hq, softmax_scale, chunk, part_m, part_l, part_acc,
                                   kernel, p);
    return st ? st : launch_plan(p, cache, q_dtype, kernel, l);
}

}  // namespace

int kvq_sdpa_int4_partial(const kvq_cache *cache, int64_t skv, const void *q, int q_dtype, int32_t Hq,
                          float softmax_scale, int32_t chunk, float *part_m, float *part_l, float *part_acc,
                          int kernel, void *stream)
{
    const Launch l{(hipStream_t)stream, nullptr, nullptr};
    return partial_impl(cache, skv, q, q_dtype, Hq, softmax_scale, chunk, part_m, part_l, part_acc, kernel, l);
}

int kvq_sdpa_int4_partial_timed(const kvq_cache *cache, int64_t skv, const void *q, int q_dtype, int32_t Hq,
                                float softmax_scale, int32_t chunk, float *part_m, float *part_l, float *part_acc,
                                int kernel, void *stream, void *start_event, void *stop_event)
{
    const Launch l{(hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event};
    return partial_impl(cache, skv, q, q_dtype, Hq, softmax_scale, chunk, part_m, part_l, part_acc, kernel, l);
}

int kvq_sdpa_int4_reduce(const float *part_m, const float *part_l, const float *part_acc, int32_t batch, int32_t Hq,
                         int32_t head_dim, int64_t num_chunks, float *out, void *stream)
{
    if (!part_m || !part_l || !part_acc || !out)
        return KVQ_E_NULL;
    if (batch < 1 || Hq < 1 || num_chunks < 1 || (int64_t)batch * Hq > 0x7fffffff)
        return KVQ_E_SHAPE;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        return KVQ_E_SHAPE;
    if (!aligned16(part_m) || !aligned16(part_l) || !aligned16(part_acc) || !aligned16(out))
        return KVQ_E_ALIGN;
    ReduceArgs a;
    a.part_m = part_m;
    a.part_l = part_l;
    a.part_acc = part_acc;
    a.out = out;
    a.heads = (int64_t)batch * Hq;
    a.C = num_chunks;
    a.D = head_dim;
    a.rot_scale = 0.0;
    return launch_status(launch_reduce(a, (hipStream_t)stream));
}

int kvq_sdpa_int4(const kvq_cache *cache, int64_t skv, const void *q, int q_dtype, int32_t Hq, float softmax_scale,
                  int32_t chunk, float *part_m, float *part_l, float *part_acc, float *out, int kernel, void *stream)
{
    if (!out)
        return KVQ_E_NULL;
    if (!aligned16(out))
        return KVQ_E_ALIGN;
    int st = kvq_sdpa_int4_partial(cache, skv, q, q_dtype, Hq, softmax_scale, chunk, part_m, part_l, part_acc,
                                   kernel, stream);
    if (st)
        return st;
    return kvq_sdpa_int4_reduce(part_m, part_l, part_acc, cache->batch, Hq, cache->head_dim,
                                kvq_num_chunks(skv, chunk), out, stream);
}

int kvq_sdpa_int4_prefill(const kvq_cache *cache, int64_t q_start, int32_t sq, const void *q, int q_dtype, int32_t Hq,
                          float softmax_scale, float *out, void *stream)
{
    int st = check_cache(cache);
    if (st)
        return st;
    if (q_dtype != KVQ_F16 && q_dtype != KVQ_F32)
        return KVQ_E_DTYPE;
    if (q_start < 0 || sq < 1 || Hq < 1 || Hq % cache->kv_heads != 0 || !isfinite(softmax_scale))
        return KVQ_E_SHAPE;
    if (q_start > cache->capacity || sq > cache->capacity - q_start)
        return KVQ_E_CAPACITY;
    if (!q || !out)
        return KVQ_E_NULL;
    if (!aligned16(q) || !aligned16(out))
        return KVQ_E_ALIGN;
    const int n_rep = Hq / cache->kv_heads;
    if (!prefill_supports(cache->head_dim, cache->group, n_rep, q_dtype, cache_bits(cache)))
        return KVQ_E_UNSUPPORTED;
    const int pb = prefill_positions_per_block(n_rep, cache->head_dim, cache_bits(cache));
    if ((int64_t)cache->batch * Hq * sq > ((int64_t)1 << 40) / cache->head_dim || (sq + pb - 1) / pb > 0x7fffffff)
        return KVQ_E_SHAPE;
    PrefillArgs a;
    a.k_q = cache->k_q;
    a.v_q = cache->v_q;
    a.k_scale = cache->k_scale;
    a.k_bias = cache->k_bias;
    a.v_scale = cache->v_scale;
    a.v_bias = cache->v_bias;
    a.q = q;
    a.out = out;
    a.cap = cache->capacity;
    a.q_start = q_start;
    a.sq = sq;
    a.Hkv = cache->kv_heads;
    a.Hq = Hq;
    a.n_rep = n_rep;
    a.pb = pb;
    a.bits = cache_bits(cache);
    a.q_f32 = q_dtype == KVQ_F32;
    a.D = cache->head_dim;
    a.score_scale = softmax_scale * kLog2e;
    return launch_status(launch_prefill(a, cache->batch, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// rows_b[i] = H_D rows_a[i] / sqrt(D) for the query (fp32 out) and the output
// reduce of a rotated decode step
int reduce_rotated(const float *part_m, const float *part_l, const float *part_acc, const kvq_cache *cache, int32_t Hq,
                   int64_t num_chunks, float *out, hipStream_t s)
{
    ReduceArgs ra;
    ra.part_m = part_m;
    ra.part_l = part_l;
    ra.part_acc = part_acc;
    ra.out = out;
    ra.heads = (int64_t)cache->batch * Hq;
    ra.C = num_chunks;
    ra.D = cache->head_dim;
    ra.rot_scale = 1.0 / sqrt((double)cache->head_dim);
    return launch_status(launch_reduce(ra, s));
}

int decode_step_impl(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int kv_dtype,
                     const void *q, int q_dtype, int32_t Hq, float softmax_scale, int32_t chunk, float *part_m,
                     float *part_l, float *part_acc, float *out, int kernel, const Launch &l, bool rotate)
{
    void *stream = (void *)l.s;
    int st = check_cache(cache);
    if (st)
        return st;
    if (kv_dtype != KVQ_F16 && (kv_dtype != KVQ_F32 || rotate))
        return KVQ_E_DTYPE;
    if (len < 0)
        return KVQ_E_SHAPE;
    if (len >= cache->capacity)
        return KVQ_E_CAPACITY;
    if (!k_new || !v_new || !out)
        return KVQ_E_NULL;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(out))
        return KVQ_E_ALIGN;
    if (rotate && (q_dtype != KVQ_F16 && q_dtype != KVQ_F32))
        return KVQ_E_DTYPE;
    if (rotate && (!q || !aligned16(q)))
        return !q ? KVQ_E_NULL : KVQ_E_ALIGN;
    if (rotate) {  // out may hold the rotated query: it must not overlap q, except fp32 q in place
        const int64_t n = (int64_t)cache->batch * Hq * cache->head_dim;
        if (overlaps(q, n * (q_dtype == KVQ_F16 ? 2 : 4), out, n * 4) && !(q_dtype == KVQ_F32 && (const void *)out == q))
            return KVQ_E_SHAPE;
    }
    // a rotated step that cannot rotate the query inside the attention kernel
    // first rotates it into `out` (fp32, the query's size) and attends with that
    PartialPlan p;
    st = prepare_partial(cache, len + 1, q, q_dtype, Hq, softmax_scale, chunk, part_m, part_l, part_acc, kernel, p);
    if (st)
        return st;
    const bool rot_inside = rotate && p.use_mfma && cache->head_dim == 128 &&
                            mfma_one_wave_ok(p.a, cache->head_dim, cache->batch) &&
                            kernel != KVQ_KERNEL_MFMA_SPLIT;
    if (rotate && !rot_inside) {
        st = prepare_partial(cache, len + 1, out, KVQ_F32, Hq, softmax_scale, chunk, part_m, part_l, part_acc, kernel,
                             p);
        if (st)
            return st;
    }
    // AUTO / MFMA: the multi-wavefront workgroups of the single-launch step,
    // each writing one split-K partial for its rows (at most the caller's
    // chunk count of partials per head), the token's row appended inside
    int32_t rows = 0, nwg = 0;
    const bool one_ok = p.use_mfma && mfma_one_wave_ok(p.a, cache->head_dim, cache->batch);
    bool wide = one_ok && (kernel == KVQ_KERNEL_AUTO || kernel == KVQ_KERNEL_MFMA) &&
                decode_single_plan(cache->head_dim, cache->group, Hq / cache->kv_heads, p.a.bits, len + 1,
                                   (int64_t)cache->batch * cache->kv_heads, rows, nwg) &&
                nwg <= p.a.num_chunks;
    // With the query rotated inside, every wavefront rotates it in its
    // prologue: where the workgroups would stream fewer than 512 rows per
    // wavefront and the one-wavefront kernel already has a chunk per SIMD,
    // the one-wavefront kernel's 512-row streams amortise that better.
    if (wide && rot_inside && rows < 512 && p.a.num_chunks * (int64_t)cache->kv_heads * cache->batch >= kOneWaveItems)
        wide = false;
    // fused (append inside the attention launch) whenever a one-wavefront
    // tile kernel runs: the workgroups above; or the one-wavefront kernel:
    // forced, on 8-bit caches and at head_dim 64 (their only matrix-core
    // kernel), with the rotation inside, or under AUTO / MFMA at a chunk per
    // SIMD or more where the workgroups do not fit (more merge groups than
    // they take)
    const int64_t items = p.a.num_chunks * cache->kv_heads * cache->batch;
    const bool fused = one_ok && (wide || kernel == KVQ_KERNEL_MFMA_WAVE || p.a.bits == 8 || cache->head_dim == 64 ||
                                  rot_inside ||
                                  ((kernel == KVQ_KERNEL_AUTO || kernel == KVQ_KERNEL_MFMA) && items >= kOneWaveItems));
    if (fused) {
        p.a.k_new = k_new;
        p.a.v_new = v_new;
        p.a.append_row = len;
        p.a.append_dtype = kv_dtype;
        int launch_q_dtype = q_dtype;
        if (rotate) {
            p.a.rot_scale = 1.0 / sqrt((double)cache->head_dim);
            launch_q_dtype = KVQ_F32;  // the split-query kernel variant
            if (rot_inside) {          // rotate the appended rows and the query (read as given)
                p.a.rotate = kRotateRows | kRotateQuery;
                p.a.q_f16 = q_dtype == KVQ_F16;
            } else {                   // query rotated beforehand (into out); rotate only the rows
                p.a.rotate = kRotateRows;
                p.a.q_f16 = 0;
            }
        }
        if (rotate && !rot_inside) {
            RotateArgs ra{q, out, (int64_t)cache->batch * Hq, cache->head_dim, 1.0 / sqrt((double)cache->head_dim)};
            st = launch_status(launch_rotate(ra, q_dtype, l.s));
            if (st)
                return st;
            p.a.q = out;
        }
        if (wide) {
            p.a.chunk = rows;
            p.a.nwg = nwg;
            p.a.num_chunks = nwg;
            st = launch_status(launch_decode_single(p.a, cache->head_dim, launch_q_dtype, cache->batch, l));
        } else {
            st = launch_status(launch_decode_fused(p.a, cache->head_dim, launch_q_dtype, cache->batch, l));
        }
    } else {
        if (rotate) {
            RotateArgs ra{q, out, (int64_t)cache->batch * Hq, cache->head_dim, 1.0 / sqrt((double)cache->head_dim)};
            st = launch_status(launch_rotate(ra, q_dtype, l.s));
            if (!st)
                st = kvq_quantize_kv_append_rotated(cache, len, k_new, v_new, kv_dtype, 1, stream);
        } else {
            st = kvq_quantize_kv_append(cache, len, k_new, v_new, kv_dtype, 1, stream);
        }
        if (!st)
            st = launch_plan(p, cache, rotate ? KVQ_F32 : q_dtype, kernel, l);
    }
    if (st)
        return st;
    if (rotate)
        return reduce_rotated(part_m, part_l, part_acc, cache, Hq, p.a.num_chunks, out, l.s);
    return kvq_sdpa_int4_reduce(part_m, part_l, part_acc, cache->batch, Hq, cache->head_dim, p.a.num_chunks, out,
                                stream);
}

// Workspace of the single-launch decode step, for steps over at most
// max_rows rows: the arrival counters, one per (batch, grid row), B * Hq at
// most (a grid row is a KV head and a block of its query heads), padded to
// 256 bytes; then room for one merged partial per 512 rows and grid row
// (kMergeHeader + block heads * D floats), which also holds the split-K
// partials (m, l, acc, fp32) of the paths with a separate reduce.
int64_t counter_region(const kvq_cache *c, int32_t Hq) { return ((int64_t)c->batch * Hq * 4 + 255) / 256 * 256; }

int64_t workspace_bytes(const kvq_cache *c, int32_t Hq, int64_t max_rows)
{
    const int64_t n_rep = Hq / c->kv_heads, D = c->head_dim;
    const int split = mfma_head_split(c->head_dim, c->group, (int)n_rep);
    const int64_t blocks = (max_rows + 511) / 512;
    const int64_t merged = (split > 0 ? split : 1) * kMergeHeader + n_rep * D, partials = n_rep * (D + 2);
    return counter_region(c, Hq) +
           (int64_t)c->batch * c->kv_heads * blocks * (merged > partials ? merged : partials) * 4 + 64;
}

int single_launch_impl(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int kv_dtype,
                       const void *q, int q_dtype, int32_t Hq, float softmax_scale, void *workspace, int64_t ws_bytes,
                       float *out, const Launch &l)
{
    int st = check_cache(cache);
    if (st)
        return st;
    if (kv_dtype != KVQ_F16 && kv_dtype != KVQ_F32)
        return KVQ_E_DTYPE;
    if (len < 0 || Hq < 1 || Hq % cache->kv_heads != 0)
        return KVQ_E_SHAPE;
    if (len >= cache->capacity)
        return KVQ_E_CAPACITY;
    if (!workspace || !out || !k_new || !v_new || !q)
        return KVQ_E_NULL;
    if (!aligned16(workspace) || !aligned16(out) || !aligned16(k_new) || !aligned16(v_new))
        return KVQ_E_ALIGN;
    const int64_t skv = len + 1;
    if (ws_bytes < workspace_bytes(cache, Hq, skv))
        return KVQ_E_SHAPE;
    // the split-K workspace of the three-launch path, inside the same bytes
    char *base = (char *)workspace + counter_region(cache, Hq);
    const int64_t C = kvq_num_chunks(skv, 512);
    const int64_t nm = ((int64_t)cache->batch * Hq * C + 3) / 4 * 4;
    float *part_m = (float *)base, *part_l = part_m + nm, *part_acc = part_l + nm;
    PartialPlan p;
    st = prepare_partial(cache, skv, q, q_dtype, Hq, softmax_scale, 512, part_m, part_l, part_acc, KVQ_KERNEL_AUTO,
                         p);
    if (st)
        return st;
    int32_t rows = 0, nwg = 0;
    const int64_t heads = (int64_t)cache->batch * cache->kv_heads;
    if (p.use_mfma && decode_single_plan(cache->head_dim, cache->group, Hq / cache->kv_heads, cache_bits(cache), skv,
                                         heads, rows, nwg)) {
        p.a.chunk = rows;
        p.a.num_chunks = (int64_t)nwg * (cache->head_dim <= 128 ? 8 : 4);  // wavefronts: eight per workgroup up to D 128
        p.a.k_new = k_new;
        p.a.v_new = v_new;
        p.a.append_row = len;
        p.a.append_dtype = kv_dtype;
        p.a.merge_ws = (float *)base;
        p.a.counters = (uint32_t *)workspace;
        p.a.out = out;
        p.a.nwg = nwg;
        p.a.part_m = p.a.part_l = p.a.part_acc = nullptr;  // the merge inside the launch
        return launch_status(launch_decode_single(p.a, cache->head_dim, q_dtype, cache->batch, l));
    }
    return decode_step_impl(cache, len, k_new, v_new, kv_dtype, q, q_dtype, Hq, softmax_scale, 512, part_m, part_l,
                            part_acc, out, KVQ_KERNEL_AUTO, l, false);
}

// Scratch of kvq_decode_step_noalloc: a file-scope device array (each GPU
// that loads the library holds its own copy until the process ends). Host
// code never uses the array's name as an address: on first use on a device,
// with that device current, its device address is looked up once and kept
// per device (g_scratch), and kernels receive that pointer.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float *g_scratch[kMaxDevices] = {};

int noalloc_scratch(float **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return KVQ_E_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return KVQ_E_LAUNCH;
        g_scratch[dev] = static_cast<float *>(ptr);
    }
    *out = g_scratch[dev];
    return KVQ_OK;
}

}  // namespace

extern "C" {

int kvq_decode_step(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int kv_dtype,
                    const void *q, int q_dtype, int32_t Hq, float softmax_scale, int32_t chunk, float *part_m,
                    float *part_l, float *part_acc, float *out, int kernel, void *stream)
{
    const Launch l{(hipStream_t)stream, nullptr, nullptr};
    return decode_step_impl(cache, len, k_new, v_new, kv_dtype, q, q_dtype, Hq, softmax_scale, chunk, part_m, part_l,
                            part_acc, out, kernel, l, false);
}

int kvq_decode_step_rotated(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int kv_dtype,
                            const void *q, int q_dtype, int32_t Hq, float softmax_scale, int32_t chunk, float *part_m,
                            float *part_l, float *part_acc, float *out, int kernel, void *stream)
{
    const Launch l{(hipStream_t)stream, nullptr, nullptr};
    return decode_step_impl(cache, len, k_new, v_new, kv_dtype, q, q_dtype, Hq, softmax_scale, chunk, part_m, part_l,
                            part_acc, out, kernel, l, true);
}

int64_t kvq_decode_workspace_bytes(const kvq_cache *cache, int32_t Hq, int64_t max_rows)
{
    if (check_cache(cache) || Hq < 1 || Hq % cache->kv_heads != 0 || max_rows < 1)
        return 0;
    return workspace_bytes(cache, Hq, max_rows);
}

int kvq_decode_step_single_launch(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new,
                                  int kv_dtype, const void *q, int q_dtype, int32_t Hq, float softmax_scale,
                                  void *workspace, int64_t workspace_bytes, float *out, void *stream,
                                  void *start_event, void *stop_event)
{
    const Launch l{(hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event};
    return single_launch_impl(cache, len, k_new, v_new, kv_dtype, q, q_dtype, Hq, softmax_scale, workspace,
                              workspace_bytes, out, l);
}

int kvq_decode_step_noalloc(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int kv_dtype,
                            const void *q, int q_dtype, int32_t Hq, float softmax_scale, int32_t chunk, float *out,
                            int kernel, void *stream)
{
    int st = check_cache(cache);
    if (st)
        return st;
    if (len < 0 || chunk < 1 || Hq < 1 || Hq % cache->kv_heads != 0)
        return KVQ_E_SHAPE;
    if (len >= cache->capacity)
        return KVQ_E_CAPACITY;
    // the split-K partials of kvq_decode_step, laid out in the scratch array
    const int64_t C = kvq_num_chunks(len + 1, chunk);
    const int64_t nm = ((int64_t)cache->batch * Hq * C + 63) / 64 * 64;  // floats of m (and of l), 256-byte multiple
    const int64_t nacc = (int64_t)cache->batch * Hq * C * cache->head_dim;
    if ((2 * nm + nacc) * 4 > KVQ_NOALLOC_SCRATCH_BYTES)
        return KVQ_E_SCRATCH;
    float *base = nullptr;
    st = noalloc_scratch(&base);
    if (st)
        return st;
    const Launch l{(hipStream_t)stream, nullptr, nullptr};
    return decode_step_impl(cache, len, k_new, v_new, kv_dtype, q, q_dtype, Hq, softmax_scale, chunk, base, base + nm,
                            base + 2 * nm, out, kernel, l, false);
}

int kvq_decode_step_timed(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int kv_dtype,
                          const void *q, int q_dtype, int32_t Hq, float softmax_scale, int32_t chunk, float *part_m,
                          float *part_l, float *part_acc, float *out, int kernel, void *stream, void *start_event,
                          void *stop_event)
{
    const Launch l{(hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event};
    return decode_step_impl(cache, len, k_new, v_new, kv_dtype, q, q_dtype, Hq, softmax_scale, chunk, part_m, part_l,
                            part_acc, out, kernel, l, false);
}

}  // extern "C"
