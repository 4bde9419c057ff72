/*
 * kvq.h - C ABI for decode-time attention on an int4 group-affine KV cache
 * on AMD Instinct MI355X (gfx950).
 *
 * What the operations are, from the source pages:
 *  - "Fused int4 Attention for Gemma 4 31B on Apple Silicon", "Background:
 *    Why TurboQuant Fails on Gemma 4": K/V stored as int4 codes with a scale
 *    and a bias per group; "What I Built Instead": attention computed as
 *    sdpa_int4(Q, K_int4, V_int4) -> output, dequantising in registers with
 *    no float temporaries, nibbles read lowest first.
 *  - "turboquant-llama3.170B" README: the kernel paragraph (per-element
 *    dequantisation, Q.K^T, online softmax, no score matrix), the split-K
 *    paragraph (512-token chunks computed independently, then a second phase,
 *    run after the first, that merges the per-chunk softmax states), the
 *    decode-step listing (K and V quantised to int4 on append; GQA).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or synchronises, and keeps no global state, with
 *    one exception: kvq_decode_step_noalloc's static device scratch and the
 *    address it looks up once per GPU. It is safe to call from several
 *    threads.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *    work is enqueued asynchronously on it; calls on one stream run in order,
 *    so the reduce launched after the partial kernel on the same stream sees
 *    its results without any event or host synchronisation.
 *  - Arguments are validated on the host before anything is enqueued; on a
 *    negative status nothing was written. A fault during execution surfaces
 *    at the caller's next synchronisation of the stream.
 *  - Inputs must be finite and within fp16 range (|x| <= 65504); this is not
 *    checked.
 *
 * Cache format (one layer):
 *  - k_q, v_q: uint32 [B][Hkv][cap][D/8]. Dimension d of a row is code
 *    (word[d/8] >> (4*(d%8))) & 0xF: eight codes per word, lowest nibble first.
 *  - k_scale, k_bias, v_scale, v_bias: fp16 bit patterns [B][Hkv][cap][D/G];
 *    element (t, d) dequantises to code * scale[t][d/G] + bias[t][d/G].
 *  - Quantiser (per group of G values x): bias = largest fp16 <= min(x);
 *    scale = smallest fp16 >= fl32(fl32(max(x) - bias) / 15); code =
 *    clamp(rint(fl32(fl32(x - bias) / scale)), 0, 15), 0 if scale == 0;
 *    fp32 round-to-nearest-even at every step; -0 metadata stored as +0.
 *    This rule is this library's reading of "per-group scale + bias"; it is
 *    bit-exact and keeps every value within scale/2 of its reconstruction.
 *  - 8-bit variant (kvq_cache.bits == 8; the Gemma page's "What I Tried"
 *    table lists an int8 KV cache and the blog's decode driver takes 4 or 8
 *    KV bits): the same rule with 255 in place of 15, codes 0..255, k_q and
 *    v_q uint32 [B][Hkv][cap][D/4] with dimension d at
 *    (word[d/4] >> (8*(d%4))) & 0xFF. Every entry point that takes a cache
 *    reads and writes this format. Of the split-K kernels, the vector-ALU
 *    and the one-wavefront matrix-core kernel (KVQ_KERNEL_MFMA_WAVE) read
 *    8-bit codes; AUTO and MFMA run 8-bit caches on the latter when the chunk
 *    layout fits it, else on the vector-ALU kernel. The same holds for
 *    head_dim 64 at either code width.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_E_NULL = -1,        /* a required pointer is NULL */
    KVQ_E_SHAPE = -2,       /* a size is out of range or inconsistent */
    KVQ_E_ALIGN = -3,       /* a pointer is not 16-byte aligned */
    KVQ_E_CAPACITY = -4,    /* rows beyond the cache capacity */
    KVQ_E_DTYPE = -5,       /* unknown element type */
    KVQ_E_LAUNCH = -6,      /* the HIP runtime rejected a launch */
    KVQ_E_UNSUPPORTED = -7, /* valid request that no kernel variant handles */
    KVQ_E_SCRATCH = -8      /* kvq_decode_step_noalloc: partials beyond its static scratch */
} kvq_status;

/* Bytes of the static device scratch that kvq_decode_step_noalloc uses. */
#define KVQ_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)

typedef enum kvq_dtype { KVQ_F16 = 0, KVQ_F32 = 1 } kvq_dtype;

/* Kernel choice for the partial (split-K) phase. */
typedef enum kvq_kernel {
    KVQ_KERNEL_AUTO = 0,        /* fastest variant that supports the shape */
    KVQ_KERNEL_VALU = 1,        /* vector-ALU kernel: any supported shape */
    KVQ_KERNEL_MFMA = 2,        /* matrix-core kernels, D in {64, 128, 256}, D/G <= 4 (any Hq/Hkv: the
                                   query heads of a KV head run in blocks of at most 8 / (D/G)
                                   heads, 16 / (D/G) at D = 128 with D/G = 2, each block its own
                                   grid row); the variant below is chosen by grid size */
    KVQ_KERNEL_MFMA_SPLIT = 3,  /* matrix-core, four wavefronts per chunk (any chunk length); int4
                                   codes at D in {128, 256} only */
    KVQ_KERNEL_MFMA_WAVE = 4    /* matrix-core, one wavefront per chunk: chunk <= 512 */
    /* any other value returns KVQ_E_SHAPE (5 named a two-wavefront variant, since removed) */
} kvq_kernel;

/* One layer's quantised cache (all device pointers, 16-byte aligned). */
typedef struct kvq_cache {
    uint32_t *k_q;
    uint32_t *v_q;
    uint16_t *k_scale;
    uint16_t *k_bias;
    uint16_t *v_scale;
    uint16_t *v_bias;
    int32_t batch;     /* B >= 1 */
    int32_t kv_heads;  /* Hkv >= 1 */
    int32_t head_dim;  /* D in {64, 128, 256} */
    int32_t group;     /* G in {32, 64, 128}, D % G == 0 */
    int64_t capacity;  /* rows per (batch, KV head), >= 1; capacity * D * bits/8 <= 2^31 - 2^16 */
    int32_t bits;      /* bits per code: 4 (0 means 4) or 8 */
} kvq_cache;

/* Library version string, e.g. "kvq 0.1.0 gfx950". */
const char *kvq_version(void);

/* Human-readable name of a status code (never NULL). */
const char *kvq_status_str(int status);

/* Number of split-K chunks: ceil(skv / chunk); 0 if skv <= 0 or chunk <= 0. */
int64_t kvq_num_chunks(int64_t skv, int32_t chunk);

/* Bytes of one layer's cache: codes plus fp16 scale and bias for K and V,
 * capacity rows per (batch, KV head), bits per code 4 (or 0) or 8; 0 for
 * invalid sizes. */
int64_t kvq_cache_bytes(int32_t batch, int32_t kv_heads, int32_t head_dim, int32_t group, int64_t capacity,
                        int32_t bits);

/*
 * Measurement helper, not a step of the method: read `bytes` bytes of device
 * memory once with a plain grid-stride kernel (16-byte loads, 2048
 * workgroups of 256 threads) and discard them. Timing it over a buffer no
 * cache holds (>= 1 GB) gives the HBM read rate this GPU reaches, beside
 * which the attention kernel's algorithmic bytes per second are compared.
 *  buf:  device memory, 16-byte aligned; bytes: a multiple of 16, >= 0
 *        (0: no-op returning KVQ_OK).
 *  sink: one device uint32, 4-byte aligned; written only when a thread's XOR
 *        of its words equals `key` (a caller-chosen value, so no load can be
 *        dropped); the caller owns both buffers.
 * KVQ_E_NULL / KVQ_E_SHAPE / KVQ_E_ALIGN before anything is enqueued;
 * KVQ_E_LAUNCH if the launch fails. Asynchronous on `stream`.
 */
int kvq_hbm_read(const void *buf, int64_t bytes, uint32_t key, uint32_t *sink, void *stream);

/*
 * Quantise n_new new rows of K and V and store them at rows
 * [len, len + n_new) of the cache ("quantize K,V to int4" in the README's
 * decode-step listing; prefill rows are appended the same way).
 *
 *  k_new, v_new: [B][Hkv][n_new][D] row-major, element type `dtype`
 *                (KVQ_F16 or KVQ_F32), 16-byte aligned.
 *  len:          rows already in the cache (0 <= len, len + n_new <= cap).
 *  n_new == 0 is a no-op returning KVQ_OK.
 * Rows outside [len, len + n_new) are not touched. The caller advances its
 * own length; the library does not track it.
 */
int kvq_quantize_kv_append(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new,
                           int dtype, int64_t n_new, void *stream);

/*
 * Hadamard-rotated append: the rotation of the blog on running Gemma 4 with
 * TurboQuant (devengoratela.com; its "TurboQuant" section with the worked
 * example and step "1. Vector Rotation"), which spreads outlier channels
 * before quantisation. Each K and V row x is replaced by
 *   r = fp32( fp64(H_D x) * fp64(1 / sqrt(D)) ),
 * H_D the Sylvester-ordered Hadamard matrix (entry (i, j) = (-1)^popcount(i & j));
 * the sum is exact for fp16 rows, then one rounding to float64 and one to
 * fp32, and r is quantised exactly as kvq_quantize_kv_append quantises its
 * rows. Arguments, layout and errors as kvq_quantize_kv_append, but the rows
 * must be fp16 (KVQ_E_DTYPE otherwise) and the rotated values within
 * +-65504 (not checked). A rotated cache is read with a rotated query and
 * gives a rotated output: rotate q with kvq_hadamard_rotate, run the
 * attention calls unchanged, rotate the output back (the rotation is its own
 * inverse).
 */
int kvq_quantize_kv_append_rotated(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new,
                                   int dtype, int64_t n_new, void *stream);

/*
 * out[r][:] = H_D x[r][:] / sqrt(D) in fp32, for rows r < rows (the rotation
 * above, computed in float64 and rounded once to fp32; for fp16 rows the
 * result equals the values kvq_quantize_kv_append_rotated quantises).
 *  x:   [rows][D], KVQ_F16 or KVQ_F32; out: fp32 [rows][D]; both 16-byte
 *       aligned. out may be x itself when x is fp32 (in place); any other
 *       overlap returns KVQ_E_SHAPE.
 *  D:   64, 128 or 256. rows == 0 is a no-op returning KVQ_OK.
 */
int kvq_hadamard_rotate(const void *x, int dtype, int64_t rows, int32_t head_dim, float *out, void *stream);

/*
 * Phase 1 of split-K decode attention ("turboquant-llama3.170B" README,
 * split-K paragraph): one query row per head over cache rows [0, skv),
 * cut into C = kvq_num_chunks(skv, chunk) chunks of `chunk` rows (the last
 * may be shorter). For query head h (KV head h / (Hq / Hkv)) and chunk c,
 * with scores s_t = softmax_scale * q_h . k^_t over the chunk's rows:
 *   part_m[b][h][c]      = max_t s_t
 *   part_l[b][h][c]      = sum_t exp(s_t - part_m)
 *   part_acc[b][h][c][d] = sum_t exp(s_t - part_m) * v^_t[d]
 * with k^, v^ dequantised in registers (no float K/V temporaries).
 *
 *  q:       [B][Hq][D], element type q_dtype (KVQ_F16 or KVQ_F32), 16-byte aligned.
 *  Hq:      query heads, a multiple of Hkv.
 *  chunk:   rows per chunk, >= 1 (512 is the tuned default).
 *  part_*:  fp32 outputs sized [B][Hq][C] and [B][Hq][C][D], 16-byte aligned.
 *  kernel:  KVQ_KERNEL_AUTO, or a forced variant (KVQ_E_UNSUPPORTED if it
 *           cannot run this shape; MFMA_SPLIT refuses 8-bit caches).
 */
int kvq_sdpa_int4_partial(const kvq_cache *cache, int64_t skv, const void *q, int q_dtype, int32_t Hq,
                          float softmax_scale, int32_t chunk, float *part_m, float *part_l, float *part_acc,
                          int kernel, void *stream);

/*
 * kvq_sdpa_int4_partial with its kernel timed: start_event and stop_event
 * (hipEvent_t, created by the caller with timing enabled; either may be
 * NULL) are recorded in the kernel's own dispatch, at the start and the end of
 * its execution, so their elapsed time is the kernel's duration without the
 * dispatch and completion latency an event recorded before and after the
 * call would include. Same arguments, results and errors otherwise; the
 * events are not touched when the call returns an error.
 */
int kvq_sdpa_int4_partial_timed(const kvq_cache *cache, int64_t skv, const void *q, int q_dtype, int32_t Hq,
                                float softmax_scale, int32_t chunk, float *part_m, float *part_l, float *part_acc,
                                int kernel, void *stream, void *start_event, void *stop_event);

/*
 * Phase 2: combine the partials of kvq_sdpa_int4_partial (README split-K
 * paragraph): with M = max_c m_c,
 *   out[b][h][d] = sum_c e^{m_c - M} acc_c[d] / sum_c e^{m_c - M} l_c.
 * Launch it on the same stream after the partial call.
 *  out: fp32 [B][Hq][D], 16-byte aligned. C >= 1.
 */
int kvq_sdpa_int4_reduce(const float *part_m, const float *part_l, const float *part_acc, int32_t batch,
                         int32_t Hq, int32_t head_dim, int64_t num_chunks, float *out, void *stream);

/*
 * Convenience: both phases back to back on `stream` (the pages' single
 * sdpa_int4 call). The caller provides the partials workspace, sized as for
 * kvq_sdpa_int4_partial.
 */
int kvq_sdpa_int4(const kvq_cache *cache, int64_t skv, const void *q, int q_dtype, int32_t Hq,
                  float softmax_scale, int32_t chunk, float *part_m, float *part_l, float *part_acc, float *out,
                  int kernel, void *stream);

/*
 * Prefill-side attention on the quantised cache (the README's hybrid
 * paragraph sends Sq > 1 to a separate fp16 attention before quantising;
 * here the block's queries read the packed cache itself): the queries of
 * positions q_start .. q_start + sq - 1, whose K/V rows must already be cache
 * rows [q_start, q_start + sq) (append them first), with query i attending
 * to rows [0, q_start + i] (causal):
 *   out[b][h][i][:] = sum_{t <= q_start + i} softmax_t(softmax_scale * q_hi . k^_t) v^_t
 *  q:    [B][Hq][sq][D], q_dtype KVQ_F16 or KVQ_F32 (fp32: split into fp16
 *        hi and lo halves, e.g. a query rotated for a Hadamard-rotated
 *        cache), 16-byte aligned; Hq a multiple of Hkv.
 *  out:  [B][Hq][sq][D] fp32, normalised, 16-byte aligned.
 * One launch, no workspace. Supported: D = 64, 128 or 256, G = 64, 4- or
 * 8-bit codes, Hq / Hkv <= 32 at D = 64 and 128 and <= 16 at D = 256
 * (KVQ_E_UNSUPPORTED otherwise). q_start + sq beyond the capacity returns
 * KVQ_E_CAPACITY. On a Hadamard-rotated cache: rotate q with
 * kvq_hadamard_rotate (fp32 out), call this with KVQ_F32, rotate out back.
 */
int kvq_sdpa_int4_prefill(const kvq_cache *cache, int64_t q_start, int32_t sq, const void *q, int q_dtype,
                          int32_t Hq, float softmax_scale, float *out, void *stream);

/*
 * One decode step (the README's decode-step listing: quantise the current
 * token's K and V into the cache, then the fused int4 attention with GQA):
 * writes k_new / v_new ([B][Hkv][D], kv_dtype, one row per (batch, KV head))
 * into cache row `len` with the rule of kvq_quantize_kv_append, then
 * computes out over the len + 1 rows 0..len as kvq_sdpa_int4 would.
 * When the one-wavefront matrix-core kernel takes the shape, the append runs
 * inside the attention kernel, in the wavefront that owns the new row, so the
 * step is two launches (attention, reduce) instead of three:
 *  - AUTO / MFMA: workgroups of eight wavefronts (four at D = 256), each
 *    wavefront streaming every eighth 32-row tile of the workgroup's rows
 *    (a power of two from 512 down to 64 rows per wavefront, 128 at
 *    D = 256: the most that still gives two wavefronts per SIMD, a
 *    workgroup covering at least 512 rows), merged in LDS into one partial
 *    per workgroup, so
 *    the reduce reads at most as many partials as there are chunks; out
 *    matches kvq_sdpa_int4 within the attention tolerance (a different
 *    split of the rows);
 *  - MFMA_WAVE (or AUTO / MFMA where the partials would outnumber the
 *    chunks): one wavefront per chunk; out is kvq_sdpa_int4's with that
 *    kernel, bit for bit (also for 8-bit caches).
 * Otherwise it is the three calls in order. The cache row is bit for bit
 * the append's either way. All arguments are validated before anything is
 * enqueued: len + 1 <= capacity (else KVQ_E_CAPACITY), k_new, v_new and out
 * 16-byte aligned, the partials workspace sized for C = ceil((len+1)/chunk)
 * (its contents after the call are the step's own partials).
 */
int kvq_decode_step(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int kv_dtype,
                    const void *q, int q_dtype, int32_t Hq, float softmax_scale, int32_t chunk, float *part_m,
                    float *part_l, float *part_acc, float *out, int kernel, void *stream);

/*
 * One decode step on a Hadamard-rotated cache (the rotation of
 * kvq_quantize_kv_append_rotated; blog on running Gemma 4 with TurboQuant,
 * "TurboQuant" section): the token's fp16 K/V rows are rotated and
 * quantised into row `len`, the query is rotated, attention runs over rows
 * 0..len, and the output is rotated back, so `out` is the attention output
 * in the original coordinates. Arguments as kvq_decode_step, but k_new and
 * v_new must be fp16 (KVQ_E_DTYPE otherwise), and `out` must not overlap q
 * unless q is fp32 and out == q (KVQ_E_SHAPE).
 * At D = 128 on the matrix-core tile kernels (the one-wavefront kernel, or
 * under AUTO / MFMA the eight-wavefront workgroups of kvq_decode_step; AUTO
 * keeps the one-wavefront kernel where the workgroups would stream fewer
 * than 512 rows per wavefront and it already has a chunk per SIMD) the step
 * is two launches: the attention kernel rotates the query (fp32
 * butterflies, a relative error of a few 2^-24) in its prologue and the
 * appended rows (float64, exact for fp16 rows) in its fused append, and the
 * reduce rotates each head's output (fp32) before storing it. Otherwise the
 * query is first rotated into `out` (four launches).
 */
int kvq_decode_step_rotated(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int kv_dtype,
                            const void *q, int q_dtype, int32_t Hq, float softmax_scale, int32_t chunk,
                            float *part_m, float *part_l, float *part_acc, float *out, int kernel, void *stream);

/*
 * Bytes of workspace that kvq_decode_step_single_launch needs for steps over
 * at most max_rows cache rows (len + 1 <= max_rows) with Hq query heads; 0
 * for an invalid cache or sizes. Grows with max_rows: a workspace sized for
 * the longest context serves every shorter one.
 */
int64_t kvq_decode_workspace_bytes(const kvq_cache *cache, int32_t Hq, int64_t max_rows);

/*
 * One decode step in a single kernel launch: the step of kvq_decode_step
 * (the README's decode-step listing: quantise the token's K and V into cache
 * row len, then attention with GQA over rows 0..len), with the split-K merge
 * (README split-K paragraph: per-chunk softmax states, then a merge that
 * must follow them) inside the same launch. Each workgroup streams a few
 * consecutive chunks of one (batch, KV head), one wavefront per chunk,
 * merges its wavefronts' states in LDS and stores one partial state in the
 * workspace; the last workgroup of each (batch, KV head) to finish (an
 * arrival counter in the workspace) merges those partials into out.
 *  k_new, v_new: [B][Hkv][D], kv_dtype KVQ_F16 or KVQ_F32, 16-byte aligned.
 *  q:            [B][Hq][D], q_dtype KVQ_F16 or KVQ_F32; out: [B][Hq][D] fp32
 *                normalised, 16-byte aligned.
 *  workspace:    device memory owned by the caller, 16-byte aligned, at least
 *                kvq_decode_workspace_bytes(cache, Hq, len + 1) bytes
 *                (KVQ_E_SHAPE otherwise). Its first 4 * B * Hq bytes hold
 *                the arrival counters (uint32, one per batch, KV head and
 *                block of its query heads, at most B * Hq of them): zero
 *                them once before the first call (e.g. hipMemset);
 *                every call leaves them at zero again. Calls that use one
 *                workspace must not overlap in time (one stream, or ordered
 *                by events); after a call that did not complete (a fault),
 *                zero them again.
 *  start_event, stop_event: optional hipEvent_t (timing enabled, either may
 *                be NULL), recorded in the kernel's own dispatch as in
 *                kvq_sdpa_int4_partial_timed.
 * The matrix-core shapes of the one-wavefront kernel run in one launch
 * (D 64, 128 or 256, D/G <= 4, 4- or 8-bit codes); other shapes run as
 * kvq_decode_step with 512-row
 * chunks (append, partial and reduce), inside the same workspace. The cache
 * row written is the one kvq_quantize_kv_append writes, bit for bit; out
 * matches kvq_sdpa_int4 within the attention tolerance (the merge order
 * differs). Validated before anything is enqueued, as kvq_decode_step.
 */
int kvq_decode_step_single_launch(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new,
                                  int kv_dtype, const void *q, int q_dtype, int32_t Hq, float softmax_scale,
                                  void *workspace, int64_t workspace_bytes, float *out, void *stream,
                                  void *start_event, void *stop_event);

/*
 * kvq_decode_step for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step, arguments and results, but its split-K partials live in a static
 * device array of KVQ_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds
 * on each GPU it runs on until the process ends, so the caller passes no
 * workspace. The request must fit it: B * Hq * C * (D + 2) floats, C =
 * ceil((len + 1) / chunk), with m and l each rounded up to 64 floats (the
 * Llama layer, B 1, Hq 64, D 128, chunk 512: up to 258,048 rows); larger ones
 * return KVQ_E_SCRATCH before anything is enqueued. Nothing is allocated:
 * on its first call on a device, with that device current, the call looks
 * up the array's device address once and keeps it. Every call on one GPU
 * shares the array (it holds the last call's partials, all written before
 * they are read within a call), so calls that overlap in time on one GPU
 * race: issue them on one stream or order them.
 */
int kvq_decode_step_noalloc(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int kv_dtype,
                            const void *q, int q_dtype, int32_t Hq, float softmax_scale, int32_t chunk, float *out,
                            int kernel, void *stream);

/*
 * kvq_decode_step with its attention kernel timed: start_event / stop_event
 * (hipEvent_t with timing, either may be NULL) are recorded in that kernel's
 * own dispatch, as in kvq_sdpa_int4_partial_timed (in the fused step this is
 * the kernel that also appends the row). Otherwise identical.
 */
int kvq_decode_step_timed(const kvq_cache *cache, int64_t len, const void *k_new, const void *v_new, int kv_dtype,
                          const void *q, int q_dtype, int32_t Hq, float softmax_scale, int32_t chunk, float *part_m,
                          float *part_l, float *part_acc, float *out, int kernel, void *stream, void *start_event,
                          void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
