// Device helpers shared by the gfx950 kernels of the library: wave64 lane
// arithmetic, MFMA fragment types, fast exp2/log2, bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace locks {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short bf16x4 __attribute__((ext_vector_type(4)));  // 4 bf16 bit patterns
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// 2^x and log2(x) on the transcendental unit (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Cross-lane exchange through the LDS crossbar (ds_bpermute); general lanes.
__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// DPP row permutes (rows = 16 lanes), applied inside the VALU instruction.
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i -> 7 - i within each 8-lane half
constexpr int kDppMirror = 0x140;      // lane i -> 15 - i within each row
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xf, 0xf, false);
}

// Max / sum over the 16 lanes of one row: butterflies inside each quad, then
// quad pairs (half mirror) and halves (mirror); every lane gets the result.
__device__ __forceinline__ float max_in_row(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    return fmaxf(v, dpp<kDppMirror>(v));
}
__device__ __forceinline__ float sum_in_row(float v) {
    v += dpp<kDppXor1>(v);
    v += dpp<kDppXor2>(v);
    v += dpp<kDppHalfMirror>(v);
    return v + dpp<kDppMirror>(v);
}
__device__ __forceinline__ uint32_t umax_in_row(uint32_t v) {
    uint32_t o = dpp_u<kDppXor1>(v);
    v = o > v ? o : v;
    o = dpp_u<kDppXor2>(v);
    v = o > v ? o : v;
    o = dpp_u<kDppHalfMirror>(v);
    v = o > v ? o : v;
    o = dpp_u<kDppMirror>(v);
    return o > v ? o : v;
}

// Combine lane l with lanes l^16 and l^32 (the same column of the four
// rows) with the gfx950 row-swap instructions: swapping a register with a
// copy of itself leaves each lane holding its own value in one output and
// its partner row's value in the other.
__device__ __forceinline__ float max_over_rows(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float sum_over_rows(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float wave_max(float v) { return max_over_rows(max_in_row(v)); }
__device__ __forceinline__ float wave_sum(float v) { return sum_over_rows(sum_in_row(v)); }

// D(16x16) += A(16x4) * B(4x16), fp32.  Lane l supplies A[l%16][l/16] and
// B[l/16][l%16]; it receives D[4*(l/16) + v][l%16] in element v.
__device__ __forceinline__ f32x4 mfma_16x16x4_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.  Lane l
// supplies 8 consecutive k of row l%16 of A and of column l%16 of B, k-group
// l/16; it receives D[4*(l/16) + v][l%16] in element v.
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x16) * B(16x16), bf16 inputs, fp32 accumulate.  Lane l
// supplies 4 consecutive k of row l%16 of A and of column l%16 of B, k-group
// l/16; it receives D[4*(l/16) + v][l%16] in element v.
__device__ __forceinline__ f32x4 mfma_16x16x16_bf16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x64) * B(64x16), int8 inputs, int32 accumulate (exact).
// Lane l supplies 16 int8 of row l%16 of A and of column l%16 of B, k-group
// l/16 (A and B share the lane and byte order of k); it receives
// D[4*(l/16) + v][l%16] in element v.
__device__ __forceinline__ i32x4 mfma_16x16x64_i8(i32x4 a, i32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
// Two floats -> packed bf16 pair (low half = first).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16_bits(lo)) |
           (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
}

// Round to nearest even on the conversion unit (the gfx950 bf16 convert):
// the same bits as f32_to_bf16_bits for every finite value, in one
// instruction per pair.
__device__ __forceinline__ uint16_t bf16_rne(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
// Split x into hi + lo, both bf16-representable, hi = rne(x), lo = rne(x - hi):
// the pair carries ~16 significant bits.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
    hi = bf16_rne(x);
    lo = bf16_rne(x - bf16_bits_to_f32(hi));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x4 as_bf16x4(u32x2 v) { return __builtin_bit_cast(bf16x4, v); }

// Pages of a sequence that compete for the budget: its full pages (seq / P,
// clamped to [0, max_pages]) whose summaries exist (the first `summ` pages;
// summ_valid false: all of them).  Pages from there to the end are attended
// outside the budget.
__device__ __forceinline__ int candidate_pages(int seq_raw, int summ, bool summ_valid, int P,
                                               int max_pages) {
    int full = seq_raw / P;
    full = full < 0 ? 0 : (full > max_pages ? max_pages : full);
    if (summ_valid) full = summ < 0 ? 0 : (summ < full ? summ : full);
    return full;
}

// Monotone map of a float's bits to uint32 (ascending floats -> ascending
// keys; -0 is first folded onto +0).  NaN inputs are not ordered.
__device__ __forceinline__ uint32_t orderable_bits(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace locks
