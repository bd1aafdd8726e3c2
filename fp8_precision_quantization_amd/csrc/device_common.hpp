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
// the saturating reading; NaN passes through unchanged.
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

// |v| > max and not NaN -> +-max (binary32 bit compare: for non-negative
// floats the unsigned order of the bits is the numeric order).
template <int FMT>
__device__ __forceinline__ float sat_clamp(float v) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t a = b & 0x7FFFFFFFu;
    const uint32_t c = (b & 0x80000000u) | FmtTraits<FMT>::kMaxBits;
    return (a > FmtTraits<FMT>::kMaxBits && a <= kInfBits) ? __uint_as_float(c) : v;
}

// Four binary32 values -> four codes, byte i = code of v_i.
template <int FMT>
__device__ __forceinline__ uint32_t encode4(float v0, float v1, float v2, float v3) {
    v0 = sat_clamp<FMT>(v0);
    v1 = sat_clamp<FMT>(v1);
    v2 = sat_clamp<FMT>(v2);
    v3 = sat_clamp<FMT>(v3);
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
template <int FMT>
__device__ __forceinline__ float scale_from_amax_bits(uint32_t amax_bits, bool pow2) {
    float s;
    if (amax_bits == 0u || amax_bits >= kInfBits) {
        s = 1.0f;
    } else {
        s = FmtTraits<FMT>::kMax / __uint_as_float(amax_bits);
        if (__float_as_uint(s) == kInfBits) s = kFltMax;
    }
    if (pow2) s = __uint_as_float(__float_as_uint(s) & 0xFF800000u);
    return s;
}

__device__ __forceinline__ float recip_rn(float s) { return 1.0f / s; }

// ---------------------------------------------------------------- wave64 --
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

// max over aligned groups of `width` lanes (width a power of two <= 64)
template <int WIDTH>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
#pragma unroll
    for (int off = WIDTH / 2; off >= 1; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, 64);
    return v;
}

}  // namespace fp8mi
