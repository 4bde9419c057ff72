// Internal declarations shared by the kvq HIP sources (not part of the ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// log2(e) in fp32; scores are kept pre-multiplied by it so that softmax
// weights come from the hardware exp2.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// AUTO picks the one-wavefront matrix-core kernel from this many (chunk, KV
// head, batch) items on: one wavefront per SIMD of the 256-CU chip.
constexpr int64_t kOneWaveItems = 1024;

struct QuantizeArgs {
    const void *k_new;
    const void *v_new;
    uint32_t *k_q;
    uint32_t *v_q;
    uint16_t *k_scale;
    uint16_t *k_bias;
    uint16_t *v_scale;
    uint16_t *v_bias;
    int64_t rows;     // B * Hkv * n_new
    int64_t n_new;
    int64_t len;
    int64_t cap;
    int32_t D;
    int32_t G;
    int32_t bits;      // 4 or 8 bits per code
    double rot_scale;  // nonzero: rotate each row by H_D * rot_scale (1 / sqrt(D)) before quantising
};

struct RotateArgs {
    const void *x;
    float *out;
    int64_t rows;
    int32_t D;
    double scale;  // 1 / sqrt(D)
};
hipError_t launch_rotate(const RotateArgs &a, int dtype, hipStream_t s);

struct PartialArgs {
    const uint32_t *k_q;
    const uint32_t *v_q;
    const uint16_t *k_scale;
    const uint16_t *k_bias;
    const uint16_t *v_scale;
    const uint16_t *v_bias;
    const void *q;
    float *part_m;
    float *part_l;
    float *part_acc;
    int64_t cap;
    int64_t skv;
    int64_t num_chunks;
    int32_t chunk;
    int32_t Hkv;
    int32_t Hq;
    int32_t n_rep;
    int32_t G;
    // matrix-core kernels: the n_rep query heads of a KV head run as head_split
    // blocks of n_rep / head_split heads, one grid row each (mfma_head_split)
    int32_t head_split;
    int32_t bits;       // 4 or 8 bits per code (the matrix-core kernels take 4 only)
    float score_scale;  // softmax_scale * log2(e)
    // Fused decode step (one-wavefront kernel only): when append_row >= 0,
    // the wavefront whose chunk holds that row first quantises k_new / v_new
    // ([B][Hkv][D], append_dtype) into it. -1: no append.
    const void *k_new;
    const void *v_new;
    int64_t append_row;
    int32_t append_dtype;
    // Hadamard-rotated cache (one-wavefront kernel): kRotateRows rotates the
    // appended rows, kRotateQuery (D = 128, split-query variant) the query
    // (read as fp16 when q_f16, else fp32), each by H_D * rot_scale in
    // float64 before use; 0: no rotation.
    int32_t rotate;
    int32_t q_f16;
    double rot_scale;
    // Single-launch decode step (workgroups of several wavefronts, each
    // streaming `chunk` rows): each workgroup merges its wavefronts' states
    // and stores them as partial wg of its (batch, KV head) in merge_ws
    // (kMergeHeader + n_rep * D tagged 64-bit words: (m, l) pairs in log2
    // units, then the value sums) and takes a ticket from
    // counters[b * grid rows + row]; the workgroup with the last ticket
    // merges all nwg partials into out and sets the counter back to zero.
    float *merge_ws;
    uint32_t *counters;
    float *out;
    int32_t nwg;
};

constexpr int32_t kRotateRows = 1, kRotateQuery = 2;
// words before the value sums in a merged partial: (m, l) of up to 16 heads
constexpr int kMergeHeader = 32;
// most workgroups per (batch, KV head) in the single-launch step (longer
// contexts take the three-launch step)
constexpr int kMaxMergeGroups = 256;

struct ReduceArgs {
    const float *part_m;
    const float *part_l;
    const float *part_acc;
    float *out;
    int64_t heads;  // B * Hq
    int64_t C;
    int32_t D;
    double rot_scale;  // nonzero: store H_D * out * rot_scale (the output of a rotated cache, rotated back)
};

// Prefill-side attention: queries of positions q_start .. q_start + sq - 1
// (q [B][Hq][sq][D] fp16), each over cache rows [0, q_start + i]; out fp32
// [B][Hq][sq][D], normalised.
struct PrefillArgs {
    const uint32_t *k_q;
    const uint32_t *v_q;
    const uint16_t *k_scale;
    const uint16_t *k_bias;
    const uint16_t *v_scale;
    const uint16_t *v_bias;
    const void *q;
    float *out;
    int64_t cap;
    int64_t q_start;
    int32_t sq;
    int32_t Hkv;
    int32_t Hq;
    int32_t n_rep;
    int32_t pb;         // positions per wavefront (prefill_positions_per_block)
    int32_t bits;       // 4 or 8
    int32_t q_f32;      // queries fp32 (else fp16)
    int32_t D;          // head dimension: 128 or 256
    float score_scale;  // softmax_scale * log2(e)
};
bool prefill_supports(int D, int G, int n_rep, int q_dtype, int bits);
int prefill_positions_per_block(int n_rep, int D, int bits);
hipError_t launch_prefill(const PrefillArgs &a, int batch, hipStream_t s);

// Where a partial-phase launch goes: the stream and, optionally, two events
// recorded at the kernel's own dispatch start and end (hipExtLaunchKernel).
struct Launch {
    hipStream_t s;
    hipEvent_t start;
    hipEvent_t stop;
};

hipError_t launch_quantize(const QuantizeArgs &a, int dtype, hipStream_t s);
hipError_t launch_partial_valu(const PartialArgs &a, int D, int q_dtype, int batch, const Launch &l);
bool mfma_supports(int D, int G, int n_rep, int chunk);
int mfma_head_split(int D, int G, int n_rep);
hipError_t launch_partial_mfma(const PartialArgs &a, int D, int q_dtype, int batch, int variant, const Launch &l);
bool mfma_one_wave_ok(const PartialArgs &a, int D, int batch);
// the fused decode step: append (a.append_row) + partial with the one-wavefront kernel
hipError_t launch_decode_fused(const PartialArgs &a, int D, int q_dtype, int batch, const Launch &l);
// the single-launch decode step: rows per wavefront and workgroups per
// (batch, KV head) for a step over skv rows, or false if the shape does not
// take it
bool decode_single_plan(int D, int G, int n_rep, int bits, int64_t skv, int64_t heads, int32_t &rows, int32_t &nwg);
hipError_t launch_decode_single(const PartialArgs &a, int D, int q_dtype, int batch, const Launch &l);
hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s);

}  // namespace kvq
