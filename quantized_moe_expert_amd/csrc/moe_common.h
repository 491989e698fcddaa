// Device helpers shared by the HIP kernels of libmoe_q4 (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq4 {

constexpr int WAVE = 64;

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;    // MFMA bf16 operand
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t; // MFMA f16 operand
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;    // 32x32 accumulator
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// --------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// binary32 -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Orderable key of a bf16 logit: a larger value gives a larger key and equal
// values give equal keys, so that the expert index appended below the key
// decides every tie.  -0 takes the key of +0 (they are equal), and a NaN
// takes the key of -inf: it ranks as -inf and ties with it.
__device__ __forceinline__ uint32_t bf16_order(uint32_t b) {
    b &= 0xffffu;
    if ((b & 0x7fffu) > 0x7f80u) b = 0xff80u;   // NaN -> -inf
    if (b == 0x8000u) b = 0u;                   // -0 -> +0
    return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
}
// The bf16 bits of an order key (inverse of bf16_order on the values it
// keeps: a NaN comes back as -inf, -0 as +0).
__device__ __forceinline__ uint32_t bf16_from_order(uint32_t o) {
    o &= 0xffffu;
    return (o & 0x8000u) ? (o & 0x7fffu) : (~o & 0xffffu);
}

// Two floats rounded to f16 (nearest even) as one packed pair, a in the low half.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// 2^s as a float, s clamped to the normal range [-126, 127].
__device__ __forceinline__ float exp2i(int s) {
    s = s < -126 ? -126 : (s > 127 ? 127 : s);
    return __uint_as_float((uint32_t)(s + 127) << 23);
}

// The power of two 2^s that puts values whose largest magnitude is m in
// [2^14, 2^15) before rounding them to f16: s = 14 - floor(log2 m), clamped
// to [-64, 64] (largest magnitudes between 2^-50 and 2^78 reach the range
// exactly).  Zero gets s = 64, the largest, so that among blocks scaled this
// way an all-zero block never sets the common unit.
struct RowScale {
    float sc;  // 2^s
    int s;
};
__device__ __forceinline__ RowScale row_scale(float m) {
    int be = (int)((__float_as_uint(m) >> 23) & 0xffu);  // 127 + floor(log2 m) for normal m
    be = be < 77 ? 77 : (be > 205 ? 205 : be);
    return RowScale{__uint_as_float((uint32_t)(268 - be) << 23), 141 - be};
}

// ---------------------------------------------------------------- nibbles
//
// A packed dword holds 8 consecutive codes, code j in bits [4j, 4j+4).
// unpack_pair(w, j) puts codes j and j+4 into the low 4 mantissa bits of two
// 16-bit floats whose exponent field comes from `magic`:
//   bf16 0x4300 = 128 (unit step from 128 to 256)  -> value 128 + q
//   f16  0x6400 = 1024 (unit step from 1024 to 2048) -> value 1024 + q
// so each half is exactly OFFSET + q.  Over j = 0..3 the 16-bit lanes carry
// the codes in the order 0,4,1,5,2,6,3,7 (PERM8); activations are put in the
// same order so that a dot product pairs each code with its own input.

template <uint32_t MAGIC>
__device__ __forceinline__ uint32_t unpack_pair(uint32_t w, int j) {
    return ((w >> (4 * j)) & 0x000f000fu) | MAGIC;
}
// The same with one bitfield insert (v_bfi_b32): (w & MASK) | (magic & ~MASK),
// where magic comes from opaque_magic() once per kernel.  Kept opaque, the
// constant is not folded into the and + or pair the compiler otherwise
// emits.  MASK 0x000f000f takes codes 0 and 4 of w (value OFFSET + q); for
// f16, MASK 0x00f000f0 takes codes 1 and 5 in place, bits 4..7 of the
// mantissa, value 1024 + 16 q (exact: 1024..1264 are f16 integers).
template <uint32_t MASK>
__device__ __forceinline__ uint32_t insert_codes(uint32_t w, uint32_t magic) {
    return (w & MASK) | (magic & ~MASK);
}
__device__ __forceinline__ uint32_t opaque_magic(uint32_t magic) {
    asm volatile("" : "+v"(magic));
    return magic;
}
constexpr uint32_t MAGIC_BF16 = 0x43004300u;   // 128 + q
constexpr uint32_t MAGIC_F16 = 0x64006400u;    // 1024 + q
constexpr float OFFSET_BF16 = 128.0f;
constexpr float OFFSET_F16 = 1024.0f;

// 8 consecutive 16-bit values in 4 dwords (v0 = elements 0,1; v1 = 2,3; ...)
// reordered to 0,4 | 1,5 | 2,6 | 3,7.
__device__ __forceinline__ void perm8(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t v3,
                                      uint32_t &o0, uint32_t &o1, uint32_t &o2, uint32_t &o3) {
    o0 = (v0 & 0xffffu) | (v2 << 16);
    o1 = (v0 >> 16) | (v2 & 0xffff0000u);
    o2 = (v1 & 0xffffu) | (v3 << 16);
    o3 = (v1 >> 16) | (v3 & 0xffff0000u);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Sum of the two bf16 halves of a dword, in float.
__device__ __forceinline__ float bf16_pair_sum(uint32_t v) {
    return __uint_as_float(v << 16) + __uint_as_float(v & 0xffff0000u);
}

// --------------------------------------------------------------- reductions

template <int WIDTH>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

// DPP-moved copy of v (lanes outside row_mask read 0).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                                 0xf, false));
}

// Largest value over each row of 16 lanes, in every lane of it (DPP moves;
// for non-negative values, as lanes outside the row mask read 0).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f32<0xb1>(v));   // lane ^ 1
    v = fmaxf(v, dpp_f32<0x4e>(v));   // lane ^ 2
    v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
    v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
    return v;
}

// Sum over aligned segments of W lanes with DPP moves only (no LDS).  For
// W <= 16 every lane of the segment holds the sum; for W = 32 and 64 the last
// lane of the segment does (lanes 31 / 63).
template <int W>
__device__ __forceinline__ float seg_sum_dpp(float v) {
    if (W >= 2) v += dpp_f32<0xb1>(v);          // quad_perm [1,0,3,2]: lane ^ 1
    if (W >= 4) v += dpp_f32<0x4e>(v);          // quad_perm [2,3,0,1]: lane ^ 2
    if (W >= 8) v += dpp_f32<0x141>(v);         // row_half_mirror: 8-lane groups
    if (W >= 16) v += dpp_f32<0x140>(v);        // row_mirror: 16-lane rows
    if (W >= 32) v += dpp_f32<0x142, 0xa>(v);   // row_bcast:15 into rows 1, 3
    if (W >= 64) v += dpp_f32<0x143, 0xc>(v);   // row_bcast:31 into rows 2, 3
    return v;
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROW_MASK, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Whole-wave double sum with DPP moves; the result is valid in lane 63.
__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
    v += dpp_f64<0xb1>(v);
    v += dpp_f64<0x4e>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    v += dpp_f64<0x142, 0xa>(v);
    v += dpp_f64<0x143, 0xc>(v);
    return v;
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// The double sum of the whole wave in every lane.
__device__ __forceinline__ double wave_allsum_f64_dpp(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, wave_sum_f64_dpp(v));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Inclusive prefix sum over the wave with DPP moves: shifts by 1, 2, 4, 8
// inside each row of 16 lanes (lanes shifted in from outside the row add 0),
// then the last lane of row 0 / 2 added into rows 1 / 3 and lane 31 into
// rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_scan_i32(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Whole-wave unsigned max with DPP moves, returned to every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    uint32_t t;
    t = dpp_u32<0xb1>(v); v = v > t ? v : t;
    t = dpp_u32<0x4e>(v); v = v > t ? v : t;
    t = dpp_u32<0x141>(v); v = v > t ? v : t;
    t = dpp_u32<0x140>(v); v = v > t ? v : t;
    t = dpp_u32<0x142, 0xa>(v); v = v > t ? v : t;
    t = dpp_u32<0x143, 0xc>(v); v = v > t ? v : t;
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = WAVE / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

}  // namespace moeq4
