// device_common.hpp -- gfx950 device helpers shared by the quantize and GEMM
// kernels: the OCP FP8 codec on the hardware convert instructions, bf16
// unpacking and wave64 reductions.
//
// Formats ([DeepL bets on FP8, hmyw.cn] 2.1; [H100 FP8 acceleration, measured,
// scrxy.com] formats paragraph): E4M3 = 1/4/3 bits, no Inf, max 448;
// E5M2 = 1/5/2 bits, max 57344.  gfx950's v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32
// produce exactly these OCP encodings with round-to-nearest-even.  The
// instructions are not relied on for out-of-range inputs: the encoder clamps
// |v| > max (Inf included) to +-max first, so that every non-NaN input takes
// the saturating reading; NaN codes are written from the inputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mi {

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;

template <int FMT> struct FmtTraits;
template <> struct FmtTraits<kE4M3> {
    static constexpr uint32_t kMaxBits = 0x43E00000u;  // 448.0f
    static constexpr float kMax = 448.0f;
};
template <> struct FmtTraits<kE5M2> {
    static constexpr uint32_t kMaxBits = 0x47600000u;  // 57344.0f
    static constexpr float kMax = 57344.0f;
};

constexpr uint32_t kInfBits = 0x7F800000u;
constexpr float kFltMax = 3.40282346638528859812e+38f;

// Four binary32 values -> four codes, byte i = code of v_i.  Every value
// is first clamped to [-max, max] by one median-of-three (so +-Inf and
// every |v| > max take the saturating reading), then converted with
// round-to-nearest-even.  A NaN input yields an unspecified byte: the
// callers rewrite NaN codes from their inputs.
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float v0, float v1, float v2, float v3) {
    constexpr float mx = FmtTraits<FMT>::kMax;
    v0 = __builtin_amdgcn_fmed3f(v0, -mx, mx);
    v1 = __builtin_amdgcn_fmed3f(v1, -mx, mx);
    v2 = __builtin_amdgcn_fmed3f(v2, -mx, mx);
    v3 = __builtin_amdgcn_fmed3f(v3, -mx, mx);
    int w;
    if constexpr (FMT == kE4M3) {
        w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
    } else {
        w = __builtin_amdgcn_cvt_pk_bf8_f32(v0, v1, 0, false);
        w = __builtin_amdgcn_cvt_pk_bf8_f32(v2, v3, w, true);
    }
    return (uint32_t)w;
}

// Scale from an amax given as binary32 bits ([DeepL] 2.3: the factor maps
// the values into FP8's representable interval): s = fl32(max / amax) by one
// correctly rounded division; amax == 0 or non-finite -> 1; overflow ->
// FLT_MAX; POW2 ([Soup] rowwise recipe) clears the mantissa bits.
// (Selects, not branches: the division runs for every lane.)
template <int FMT>
__device__ __forceinline__ float scale_from_amax_bits(uint32_t amax_bits, bool pow2) {
    const float q = FmtTraits<FMT>::kMax / __uint_as_float(amax_bits);
    float s = __float_as_uint(q) == kInfBits ? kFltMax : q;
    s = (amax_bits == 0u || amax_bits >= kInfBits) ? 1.0f : s;
    if (pow2) s = __uint_as_float(__float_as_uint(s) & 0xFF800000u);
    return s;
}

__device__ __forceinline__ float recip_rn(float s) { return 1.0f / s; }

// ---------------------------------------------------------------- wave64 --
// Reductions with DPP lane permutations inside each row of 16 lanes (a
// register-to-register move, no LDS round trip).  Every lane of the wave must
// be active: a permutation reads the source lane's register whatever its
// exec bit.

// v from lane (lane ^ 1), (lane ^ 2) within its quad; from the mirrored lane
// of its 8-lane half row (i <-> 7 - i) and of its 16-lane row (i <-> 15 - i)
__device__ __forceinline__ uint32_t dpp_quad_xor1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
}
__device__ __forceinline__ uint32_t dpp_quad_xor2(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
}
__device__ __forceinline__ uint32_t dpp_half_mirror(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);  // row_half_mirror
}
__device__ __forceinline__ uint32_t dpp_row_mirror(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);  // row_mirror
}

// max over aligned groups of `width` lanes (width a power of two <= 64),
// returned to every lane of the group.  Up to 16 lanes: DPP only (after the
// quad steps each quad holds its max, the half-row mirror pairs quad 0 with
// quad 1, the row mirror half 0 with half 1); wider groups then combine
// rows through lane shuffles.
template <int WIDTH>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    if constexpr (WIDTH >= 2) v = max(v, dpp_quad_xor1(v));
    if constexpr (WIDTH >= 4) v = max(v, dpp_quad_xor2(v));
    if constexpr (WIDTH >= 8) v = max(v, dpp_half_mirror(v));
    if constexpr (WIDTH >= 16) v = max(v, dpp_row_mirror(v));
    if constexpr (WIDTH >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
    if constexpr (WIDTH >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32, 64));
    return v;
}

// max over the wave, returned to every lane: the rows' maxima by DPP, then
// the four rows combined from lanes 0, 16, 32 and 48 (scalar reads)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = group_max_u32<16>(v);
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
    return v;
}

}  // namespace fp8mi
