// cast_unit.hpp -- the 8-element unit of the element-wise cast kernels
// (quantize.hip, kvcache.hip): 16-byte loads of bf16 or fp32 data, the
// scaled saturating encode with the NaN sign fix-up, 8-byte code stores and
// the optional diagnostic counters.
//
// [DeepL bets on FP8, hmyw.cn] 2.3: q = cast(x * s) with the group's scale;
// 4.2 / 6.2: max-abs, overflow and underflow are the quantities to watch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "fp8mi.h"

namespace fp8mi {
namespace cast {

// ------------------------------------------------------------ data units --
template <typename InT> struct Pack;

template <> struct Pack<uint16_t> {          // 8 bf16 values packed in 4 words
    uint32_t w[4];
    __device__ __forceinline__ float get(int i) const {
        const uint32_t v = w[i >> 1];
        return __uint_as_float((i & 1) ? (v & 0xFFFF0000u) : (v << 16));
    }
    // max |x| as binary32 bits: the 16-bit magnitudes compared two at a time
    // (packed unsigned 16-bit max), then widened
    __device__ __forceinline__ uint32_t abs_max() const {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        auto mag = [](uint32_t v) { return __builtin_bit_cast(u16x2, v & 0x7FFF7FFFu); };
        const u16x2 t = __builtin_elementwise_max(__builtin_elementwise_max(mag(w[0]), mag(w[1])),
                                                  __builtin_elementwise_max(mag(w[2]), mag(w[3])));
        return (uint32_t)max(t[0], t[1]) << 16;
    }
};

template <> struct Pack<float> {             // 8 fp32 values
    uint32_t w[8];
    __device__ __forceinline__ float get(int i) const { return __uint_as_float(w[i]); }
    __device__ __forceinline__ uint32_t abs_max() const {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = max(m, w[i] & 0x7FFFFFFFu);
        return m;
    }
};

// One 16-byte load; NT: non-temporal (streaming), so a tensor read once
// does not displace the cache's lines (a line already cached still hits).
// Measured per kernel: the flat per-tensor passes, the block casts and the
// transposed cast gain from it; the row cast and the KV store lose, and
// keep ordinary loads.
template <bool NT>
__device__ __forceinline__ uint4 load16(const void* p) {
    if constexpr (NT) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        return make_uint4(t.x, t.y, t.z, t.w);
    } else {
        return *reinterpret_cast<const uint4*>(p);
    }
}

// Load `nvalid` (0..8) elements starting at x + off; missing ones are 0.
// `vec`: x + off is 16-byte aligned and the unit is whole.
template <typename InT, bool NT = false>
__device__ __forceinline__ Pack<InT> load_unit(const InT* __restrict__ x, int64_t off, int nvalid,
                                               bool vec) {
    Pack<InT> p;
    if constexpr (sizeof(InT) == 2) {
        if (vec && nvalid == 8) {
            const uint4 r = load16<NT>(x + off);
            p.w[0] = r.x; p.w[1] = r.y; p.w[2] = r.z; p.w[3] = r.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t lo = (2 * i < nvalid) ? (uint32_t)x[off + 2 * i] : 0u;
                const uint32_t hi = (2 * i + 1 < nvalid) ? (uint32_t)x[off + 2 * i + 1] : 0u;
                p.w[i] = lo | (hi << 16);
            }
        }
    } else {
        if (vec && nvalid == 8) {
            const uint4 r0 = load16<NT>(x + off);
            const uint4 r1 = load16<NT>(x + off + 4);
            p.w[0] = r0.x; p.w[1] = r0.y; p.w[2] = r0.z; p.w[3] = r0.w;
            p.w[4] = r1.x; p.w[5] = r1.y; p.w[6] = r1.z; p.w[7] = r1.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) p.w[i] = (i < nvalid) ? __float_as_uint(x[off + i]) : 0u;
        }
    }
    return p;
}

// Whole unit u of a contiguous, 16-byte aligned tensor: elements
// [8u, 8u + 8) with plain non-temporal 16-byte loads (the flat fast path).
template <typename InT>
__device__ __forceinline__ Pack<InT> load_flat(const InT* __restrict__ x, uint32_t u) {
    Pack<InT> p;
    const uint4* src = reinterpret_cast<const uint4*>(x);
    if constexpr (sizeof(InT) == 2) {
        const uint4 r = load16<true>(src + u);
        p.w[0] = r.x; p.w[1] = r.y; p.w[2] = r.z; p.w[3] = r.w;
    } else {
        const uint4 r0 = load16<true>(src + 2 * (uint64_t)u), r1 = load16<true>(src + 2 * (uint64_t)u + 1);
        p.w[0] = r0.x; p.w[1] = r0.y; p.w[2] = r0.z; p.w[3] = r0.w;
        p.w[4] = r1.x; p.w[5] = r1.y; p.w[6] = r1.z; p.w[7] = r1.w;
    }
    return p;
}

// The 8 codes of whole unit u of a contiguous, 8-byte aligned code array.
__device__ __forceinline__ void store_flat(uint8_t* __restrict__ q, uint32_t u, uint2 codes) {
    reinterpret_cast<uint2*>(q)[u] = codes;
}

struct Counters {
    uint32_t sat = 0, nonfinite = 0, under = 0;
};

// Encode a unit with scale s; optionally count the diagnostics.  A NaN
// input makes the unit's max |x| bits exceed Inf's; only then does the
// rare fix-up run, writing the NaN code 0x7F with the input's sign (the
// clamp and convert leave an unspecified byte for a NaN).
template <int FMT, bool DIAG, typename InT>
__device__ __forceinline__ uint2 encode_unit(const Pack<InT>& p, float s, Counters& cnt) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p.get(i) * s;
    uint2 out;
    out.x = encode4<FMT>(v[0], v[1], v[2], v[3]);
    out.y = encode4<FMT>(v[4], v[5], v[6], v[7]);
    if (__builtin_expect(p.abs_max() > kInfBits, 0)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t bx = __float_as_uint(p.get(i));
            if ((bx & 0x7FFFFFFFu) > kInfBits) {
                const uint32_t code = 0x7Fu | ((bx >> 24) & 0x80u);
                const int sh = 8 * (i & 3);
                uint32_t& w = (i < 4) ? out.x : out.y;
                w = (w & ~(0xFFu << sh)) | (code << sh);
            }
        }
    }
    if constexpr (DIAG) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t ax = __float_as_uint(p.get(i)) & 0x7FFFFFFFu;
            const uint32_t av = __float_as_uint(v[i]) & 0x7FFFFFFFu;
            const uint32_t code = ((i < 4 ? out.x : out.y) >> (8 * (i & 3))) & 0xFFu;
            cnt.nonfinite += (ax >= kInfBits) ? 1u : 0u;
            cnt.sat += (av > FmtTraits<FMT>::kMaxBits && av <= kInfBits) ? 1u : 0u;
            cnt.under += (ax != 0u && ax <= kInfBits && (code & 0x7Fu) == 0u) ? 1u : 0u;
        }
    }
    return out;
}

__device__ __forceinline__ void store_unit(uint8_t* __restrict__ q, int64_t off, int nvalid,
                                           bool vec, uint2 codes) {
    if (vec && nvalid == 8) {
        *reinterpret_cast<uint2*>(q + off) = codes;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < nvalid) q[off + i] = (uint8_t)(((i < 4 ? codes.x : codes.y) >> (8 * (i & 3))) & 0xFFu);
    }
}


// Adds a 256-thread block's counters to *diag: one atomic per counter per
// block, and only when a caller asks for the counters.
__device__ __forceinline__ void block_add_diag(Counters c, uint32_t* lds, fp8_diag* diag) {
    c.sat = wave_sum_u32(c.sat);
    c.nonfinite = wave_sum_u32(c.nonfinite);
    c.under = wave_sum_u32(c.under);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) { lds[4 + w] = c.sat; lds[8 + w] = c.nonfinite; lds[12 + w] = c.under; }
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t s = lds[4] + lds[5] + lds[6] + lds[7];
        const uint32_t n = lds[8] + lds[9] + lds[10] + lds[11];
        const uint32_t u = lds[12] + lds[13] + lds[14] + lds[15];
        if (s) atomicAdd(&diag->sat_count, s);
        if (n) atomicAdd(&diag->nonfinite_count, n);
        if (u) atomicAdd(&diag->underflow_count, u);
    }
}


}  // namespace cast
}  // namespace fp8mi
