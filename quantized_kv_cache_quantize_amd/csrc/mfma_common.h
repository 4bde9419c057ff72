// Helpers shared by the matrix-core attention kernels (decode and prefill):
// fp16 operand builders for packed codes, lane exchanges, buffer resources
// and the small numeric tricks they rely on. Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// word 3 of a raw (unswizzled, 32-bit element) buffer resource on gfx9
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ float h_val(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferFlags);
}

// (x & mask) | magic, meant for one v_and_or_b32. A gfx9 VOP3 encoding takes
// no 32-bit literal, so with constant operands the compiler would split it
// into an AND and an OR that each carry a literal; the Unpacker therefore
// holds mask and magic as opaque register values (mask in a scalar register,
// magic in a vector register). Plain code, not inline asm, so that the
// compiler's hazard tracking sees every write next to the matrix instructions.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic)
{
    return (x & mask) | magic;
}

// x as a value the compiler cannot see through, in a scalar or a vector
// register (an empty asm statement; no instruction is emitted)
__device__ __forceinline__ uint32_t opaque_s(uint32_t x)
{
    asm volatile("" : "+s"(x));
    return x;
}
__device__ __forceinline__ uint32_t opaque_v(uint32_t x)
{
    asm volatile("" : "+v"(x));
    return x;
}
// opaque_s where ON, else x as a plain constant (no asm statement at all)
template <bool ON>
__device__ __forceinline__ uint32_t opaque_s_if(uint32_t x)
{
    if constexpr (ON)
        return opaque_s(x);
    else
        return x;
}

// Four half2 registers -> one MFMA operand.
__device__ __forceinline__ half8 cat8(half2v a, half2v b, half2v c, half2v d)
{
    half8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// The four nibbles of each 16-bit half of x as exact fp16 values n - 8:
// out[m] = (nibble m of the low half, nibble m of the high half) - 8.
// A nibble placed in mantissa bits 0-3 under exponent 2^10 (0x6400) reads as
// 1024 + n; in bits 4-7 under 2^6 (0x5400) as 64 + n. Nibbles 2 and 3 are
// first shifted down by 8 (an fp16 mantissa has only bits 0-9). The fp16
// subtraction of 1032 or 72 is exact.
//
// Why centred codes: the matrix core aligns the 32 products of one
// instruction to the largest and truncates the rest, which biases sums of
// same-signed products toward zero. Codes in [-8, 7] give products of both
// signs and half the magnitude, and the 8 * scale they drop moves into the
// bias term: code * s + b = (code - 8) * s + (b + 8 s).
struct Unpacker {
    uint32_t m1024, m64;  // magic exponents 0x6400 / 0x5400 (vector registers)
    uint32_t lo4, hi4;    // nibble masks 0x000F000F / 0x00F000F0 (scalar registers)
    __device__ static Unpacker make()
    {
        return Unpacker{opaque_v(0x64006400u), opaque_v(0x54005400u), opaque_s(0x000F000Fu), opaque_s(0x00F000F0u)};
    }
    __device__ __forceinline__ void operator()(uint32_t x, half2v (&out)[4]) const
    {
        const half2v k1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
        const half2v k72 = {(_Float16)72.0f, (_Float16)72.0f};
        const uint32_t y = x >> 8;
        out[0] = as_h2(and_or(x, lo4, m1024)) - k1032;
        out[1] = as_h2(and_or(x, hi4, m64)) - k72;
        out[2] = as_h2(and_or(y, lo4, m1024)) - k1032;
        out[3] = as_h2(and_or(y, hi4, m64)) - k72;
    }
    // out[m] of operator() alone (m a compile-time constant)
    __device__ __forceinline__ half2v one(uint32_t x, int m) const
    {
        const half2v k1032 = {(_Float16)1032.0f, (_Float16)1032.0f};
        const half2v k72 = {(_Float16)72.0f, (_Float16)72.0f};
        const uint32_t z = m >= 2 ? x >> 8 : x;
        return (m & 1) ? as_h2(and_or(z, hi4, m64)) - k72 : as_h2(and_or(z, lo4, m1024)) - k1032;
    }
};

// One K word (dimensions 8w..8w+7 of one row) as an MFMA operand; element j
// holds dimension 8w + kPerm[j].
constexpr int kPerm[8] = {0, 4, 1, 5, 2, 6, 3, 7};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Sum over the NG adjacent lanes that hold the groups of one head.
template <int NG>
__device__ __forceinline__ float group_sum(float v)
{
    if constexpr (NG >= 2)
        v += dpp_f<0xB1>(v);  // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (NG >= 4)
        v += dpp_f<0x4E>(v);  // quad_perm [2,3,0,1]: lane ^ 2
    return v;
}

// Headroom (log2 units) above a head's running maximum when its softmax
// reference is raised: weights are at most 2^-kHeadroom of their largest
// possible value, which costs nothing in fp32 and about 2 bits at the fp16
// subnormal floor of the value weights' lo halves.
constexpr float kHeadroom = 2.0f;
// With the hi and lo halves of the value weights in separate operand rows,
// the lo halves are stored scaled by 2^11: lo is at most half an fp16 ulp of
// hi, so lo * 2^11 stays within hi's magnitude (no overflow) and, for any
// weight above 2^-13, in the normal fp16 range instead of the subnormals.
constexpr float kLoScale = 2048.0f;

// Sum / max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 with the gfx950 row
// swaps: with both operands equal, the two results of a swap hold a lane's
// own value and its partner's, in some order. (Each element is copied to a
// scalar before the bit cast: a bit cast of a vector element in place reads
// element 0.)
__device__ __forceinline__ void row_swap16(float v, float &x, float &y)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    x = __builtin_bit_cast(float, r0);
    y = __builtin_bit_cast(float, r1);
}

__device__ __forceinline__ void row_swap32(float v, float &x, float &y)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    x = __builtin_bit_cast(float, r0);
    y = __builtin_bit_cast(float, r1);
}

// Maxima of values the compiler cannot prove canonical (results of lane
// swaps and DPP sums, or joined across the tail branch): fmaxf would first
// canonicalise every operand with an extra v_max. The NaN-propagating
// maximum needs no canonical operands and maps to gfx950's v_maximum3_f32;
// scores are finite or -inf, never NaN, so it is the same maximum.
__device__ __forceinline__ float max_raw(float x, float y) { return __builtin_elementwise_maximum(x, y); }

__device__ __forceinline__ float max3_raw(float x, float y, float z) { return max_raw(max_raw(x, y), z); }

// max(m, maximum of v over the four lanes l, l ^ 16, l ^ 32, l ^ 48)
__device__ __forceinline__ float xrow_max(float v, float m)
{
    float x, y;
    row_swap16(v, x, y);
    row_swap32(max_raw(x, y), x, y);
    return max3_raw(m, x, y);
}

// Multiply an accumulator tile in place. Tied asm operands keep the products
// in the accumulator's own registers: as plain code the compiler writes them
// to new registers and, on the far more common path that skips the rescale,
// copies every accumulator across (one move per accumulator element and tile).
// The compiler's hazard tracking does not see into inline asm, so a rescale
// starts with mfma_result_wait(): more wait states than any matrix
// instruction here needs before a vector instruction may read its result.
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"); }

__device__ __forceinline__ void scale_in_place(float4v &v, const float4v &c)
{
    float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
    asm volatile("v_mul_f32 %0, %0, %4\n\tv_mul_f32 %1, %1, %5\n\tv_mul_f32 %2, %2, %6\n\tv_mul_f32 %3, %3, %7"
                 : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3)
                 : "v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]));
    v = (float4v){x0, x1, x2, x3};
}


// One DPP move inside each row of 16 lanes: lanes in the banks of BANKS
// (bank b = lanes 4b..4b+3 of a row) take src from lane l ^ 8 (row_ror:8);
// the other lanes keep old.
template <int BANKS>
__device__ __forceinline__ uint32_t take_half_row(uint32_t old, uint32_t src)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, 0x128, 0xF, BANKS, false);
}

__device__ __forceinline__ float xrow_sum(float v)
{
    float x, y;
    row_swap16(v, x, y);
    row_swap32(x + y, x, y);
    return x + y;
}

// K words as MFMA operands with the nibbles read as fp16 subnormals: a
// nibble n moved into mantissa bits 4-7 of a half whose exponent field is
// zero is the exact value n * 2^-20 (one AND for nibbles 1 and 5, a shift
// and an AND for each other pair). Element j of the operand holds dimension
// kPerm[j]; the score factor carries the 2^20. Only this placement: the
// matrix core sums products of operands at the bottom of the subnormal range
// (n * 2^-24, bits 0-3) with about 2^-16 of the largest product's precision
// (measured), against 2^-21 for n * 2^-20 and for normal operands. The codes
// enter with no offset, so the products are at most 15 |q|.
__device__ __forceinline__ half8 k_operand_sub(uint32_t w, uint32_t m_fine)
{
    return cat8(as_h2((w << 4) & m_fine), as_h2(w & m_fine), as_h2((w >> 4) & m_fine), as_h2((w >> 8) & m_fine));
}

// Exponent bits of 1024 in both halves, and 1024 + 128 (8-bit codes): a byte
// n placed in bits 0-7 under the exponent of 1024 reads as 1024 + n (exact
// for n <= 255), and subtracting 1152 leaves the centred code n - 128, an
// exact normal fp16 integer.
constexpr uint32_t kMagic1024x4 = 0x64646464u;

// 8-bit codes. Two K words (dimensions 8o..8o+7 of one row, four bytes each)
// as an MFMA operand: a byte permute against the magic exponent bytes gives
// each pair of codes as (1024 + n) halves, one packed subtraction centres
// them. Element j holds dimension kPerm8[j]. sel_even / sel_odd pick bytes
// (0, 2) / (1, 3) of the word into the low byte of each half and the magic
// byte into the high one.
constexpr int kPerm8[8] = {0, 2, 1, 3, 4, 6, 5, 7};

__device__ __forceinline__ half8 k_operand8(uint32_t w0, uint32_t w1, uint32_t magic, uint32_t sel_even,
                                            uint32_t sel_odd)
{
    const half2v c1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
    return cat8(as_h2(__builtin_amdgcn_perm(magic, w0, sel_even)) - c1152,
                as_h2(__builtin_amdgcn_perm(magic, w0, sel_odd)) - c1152,
                as_h2(__builtin_amdgcn_perm(magic, w1, sel_even)) - c1152,
                as_h2(__builtin_amdgcn_perm(magic, w1, sel_odd)) - c1152);
}

// Byte m of the value words of two rows (r0 in the low half, r1 in the high
// half) as the exact centred codes n - 128: a byte permute places the two
// codes in the low bytes of the halves, the magic exponent bits are ORed in
// (1024 + n) and one packed subtraction of 1152 centres them. Centred codes,
// as for int4: the matrix core truncates the aligned products of one
// instruction, which biases sums of same-signed products toward zero.
__device__ __forceinline__ half2v v_pair8(uint32_t r0, uint32_t r1, uint32_t sel, uint32_t magic16)
{
    const half2v c1152 = {(_Float16)1152.0f, (_Float16)1152.0f};
    return as_h2(__builtin_amdgcn_perm(r1, r0, sel) | magic16) - c1152;
}

}  // namespace
}  // namespace kvq
