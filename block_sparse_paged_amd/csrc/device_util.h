// Device helpers for gfx950 (CDNA4, wave64): FP8/bf16 conversions and
// cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Two OCP E4M3FN codes (byte pair 0-1 or 2-3 of `w`) -> two bf16.  Exact: every
// E4M3FN value (normal, subnormal, NaN) is representable in bf16.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// Two E4M3FN codes -> two fp32 (exact).
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2_to_f32x2(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Two fp32 -> packed bf16 with the hardware converter (v_cvt_pk_bf16_f32,
// round to nearest even).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// 2^x on the transcendental unit, no denormal fix-up (for x <= 0 whose result
// only feeds softmax weights; -inf gives 0).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Compile-time loop: f(Int<I>{}) for I = B .. E-1 (the index can be a template
// argument inside f).
template <int I>
struct Int {
    static constexpr int value = I;
};
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(Int<B>{});
        static_for<B + 1, E>(f);
    }
}

// Lane permutes through DPP (row = 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;       // lane i <-> 15-i within 16

// Inclusive prefix sum over the 64 lanes (lane l gets lanes 0..l): row scans
// with row_shr (zero fill), then row_bcast15 / row_bcast31 across rows.
__device__ __forceinline__ int wave_prefix_sum(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Lane l's value combined with lane l ^ 16's (l ^ 32's) by gfx950's lane
// swaps, without LDS: permlane16_swap (permlane32_swap) of a value with itself
// returns the lane's own value and its partner's as the two results (which is
// which depends on the lane); their sum and max are the same in both lanes.
__device__ __forceinline__ float sum_xor16(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}

// Sum over aligned groups of W lanes (W power of two, <= 64); every lane of a
// group ends with the group sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (W >= 2) v += dpp_f32<kDppXor1>(v);
    if constexpr (W >= 4) v += dpp_f32<kDppXor2>(v);
    if constexpr (W >= 8) v += dpp_f32<kDppHalfMirror>(v);
    if constexpr (W >= 16) v += dpp_f32<kDppMirror>(v);
    if constexpr (W >= 32) v = sum_xor16(v);
    if constexpr (W >= 64) v = sum_xor32(v);
    return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (W >= 2) v = fmaxf(v, dpp_f32<kDppXor1>(v));
    if constexpr (W >= 4) v = fmaxf(v, dpp_f32<kDppXor2>(v));
    if constexpr (W >= 8) v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    if constexpr (W >= 16) v = fmaxf(v, dpp_f32<kDppMirror>(v));
    if constexpr (W >= 32) v = max_xor16(v);
    if constexpr (W >= 64) v = max_xor32(v);
    return v;
}

// max of three as IEEE maximum (v_maximum3_f32, no quieting of the operands
// first, unlike fmaxf); the operands are dot products or -inf, never NaN (a
// NaN dot product is outside the contract)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// Max over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four 16-lane groups).
__device__ __forceinline__ float max_over_lane_groups(float v) { return max_xor16(max_xor32(v)); }

// Sum over lanes l, l ^ 16, l ^ 32 and l ^ 48, the l ^ 16 pairs first.
__device__ __forceinline__ float sum_over_lane_groups(float v) { return sum_xor32(sum_xor16(v)); }

// Max over lanes whose index differs only in bits >= log2(FROM) (all lanes
// holding equal values within groups of FROM).
template <int FROM>
__device__ __forceinline__ float max_across_groups(float v) {
#pragma unroll
    for (int off = FROM; off < 16; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
    if constexpr (FROM <= 16) v = max_xor16(v);
    if constexpr (FROM <= 32) v = max_xor32(v);
    return v;
}

}  // namespace msa
