// kvcache.hip -- FP8 KV cache on gfx950: the scatter-store of new tokens' K
// (or V) vectors into one layer's cache, with a scale per (token, head) taken
// at store time or a fixed per-head scale, or kept in bf16 (the per-layer
// fallback); and the gather-dequantize that reads cache rows back as bf16 or
// fp32.
//
// [DeepL bets on FP8, hmyw.cn] 3.1: FP8 K/V caches halve their memory against
// BF16; K's precision drives the attention scores, V's the mixed output; one
// layer's K cache kept in BF16 removed a long-sequence degradation.
//
// Layout: a cache is [capacity x heads x head_dim], head_dim contiguous; a
// (slot, head) vector of head_dim elements is one "row".  A row gets LPR
// lanes, LPR the power of two (8..64) that covers its head_dim/8 units, so a
// 64-lane wave moves 64/LPR rows with 16-byte input and 8-byte code accesses
// (with LPR = 64 a lane takes up to 4 units: head_dim <= 2048).  The host
// checks that every access is aligned: head_dim, ld and ld_out are multiples
// of 8 and the base pointers 16-byte aligned.  Both kernels are memory bound:
// a stored element moves in_bytes + 1 (bf16 storage: in_bytes + 2) and a row
// 4 more for its scale; a loaded element 1 (or 2) + out_bytes.
#include <hip/hip_runtime.h>

#include "cast_unit.hpp"
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

using namespace cast;
constexpr int kThreads = 256;
constexpr int kStoreBf16 = 2;   // storage code beside kE4M3 / kE5M2

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 b2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even) in one word, low element first.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    const f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// Row r of a batch of n tokens x heads -> token, head and cache slot.  A slot
// outside [0, capacity) is padding: the row is neither stored nor loaded.
struct RowMap {
    int64_t t = 0, slot = -1;
    int h = 0;
    bool active = false;
    __device__ __forceinline__ RowMap(int64_t r, int64_t rows, int heads, const int64_t* __restrict__ slots,
                                      int64_t capacity) {
        if (r < rows) {
            const uint32_t rr = (uint32_t)r, hh = (uint32_t)heads;
            t = rr / hh;
            h = (int)(rr - (uint32_t)t * hh);
            slot = slots ? slots[t] : t;
            active = slot >= 0 && slot < capacity;
        }
    }
};

// Store: x row t holds the heads' vectors back to back (x + t*ld + h*hd).
template <typename InT, int ST, int LPR, bool DIAG>
__global__ __launch_bounds__(kThreads) void k_kv_store(
    const InT* __restrict__ x, int64_t ld, int64_t rows, int heads, int hd,
    const int64_t* __restrict__ slots, int64_t capacity, bool per_head, bool pow2,
    void* __restrict__ cache, float* __restrict__ scale_inv, fp8_diag* diag) {
    constexpr int UPL = LPR == 64 ? 4 : 1;
    __shared__ uint32_t lds[16];
    const int j = threadIdx.x & (LPR - 1);
    const RowMap rm((int64_t)blockIdx.x * (kThreads / LPR) + threadIdx.x / LPR, rows, heads, slots, capacity);
    const int upr = hd >> 3;
    const InT* xr = x + rm.t * ld + (int64_t)rm.h * hd;
    const int64_t dst = (rm.slot * heads + rm.h) * (int64_t)hd;
    Pack<InT> p[UPL];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        const int u = j + i * LPR;
        if (rm.active && u < upr) {
            p[i] = load_unit<InT>(xr, (int64_t)u * 8, 8, true);
            m = max(m, p[i].abs_max());
        }
    }
    if constexpr (ST == kStoreBf16) {
        uint16_t* cr = reinterpret_cast<uint16_t*>(cache) + dst;
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
            const int u = j + i * LPR;
            if (rm.active && u < upr) {
                uint4 w;
                if constexpr (sizeof(InT) == 2) {
                    w = make_uint4(p[i].w[0], p[i].w[1], p[i].w[2], p[i].w[3]);
                } else {
                    w.x = pack_bf16(p[i].get(0), p[i].get(1));
                    w.y = pack_bf16(p[i].get(2), p[i].get(3));
                    w.z = pack_bf16(p[i].get(4), p[i].get(5));
                    w.w = pack_bf16(p[i].get(6), p[i].get(7));
                }
                *reinterpret_cast<uint4*>(cr + (int64_t)u * 8) = w;
            }
        }
    } else {
        // all LPR lanes of a row take part (inactive rows contribute 0)
        m = group_max_u32<LPR>(m);
        float s = 1.0f;
        if (per_head) {
            if (rm.active) s = recip_rn(scale_inv[rm.h]);
        } else {
            s = scale_from_amax_bits<ST>(m, pow2);
            if (rm.active && j == 0) scale_inv[rm.slot * heads + rm.h] = recip_rn(s);
        }
        uint8_t* qr = reinterpret_cast<uint8_t*>(cache) + dst;
        Counters cnt;
#pragma unroll
        for (int i = 0; i < UPL; ++i) {
            const int u = j + i * LPR;
            if (rm.active && u < upr)
                store_unit(qr, (int64_t)u * 8, 8, true, encode_unit<ST, DIAG>(p[i], s, cnt));
        }
        if constexpr (DIAG) block_add_diag(cnt, lds, diag);
    }
}

// Decode 4 codes (one word) to fp32 with the hardware converts.
template <int FMT>
__device__ __forceinline__ void decode4(uint32_t w, float* v) {
    f2 lo, hi;
    if constexpr (FMT == kE4M3) {
        lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    } else {
        lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
        hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
    }
    v[0] = lo.x; v[1] = lo.y; v[2] = hi.x; v[3] = hi.y;
}

// Load: out row t receives cache row slots[t] (out + t*ld_out + h*hd).
template <int ST, bool OUT_BF16, int LPR>
__global__ __launch_bounds__(kThreads) void k_kv_load(
    const void* __restrict__ cache, const float* __restrict__ scale_inv, bool per_head, int64_t capacity,
    int heads, int hd, const int64_t* __restrict__ slots, int64_t rows, void* __restrict__ out,
    int64_t ld_out) {
    constexpr int UPL = LPR == 64 ? 4 : 1;
    const int j = threadIdx.x & (LPR - 1);
    const RowMap rm((int64_t)blockIdx.x * (kThreads / LPR) + threadIdx.x / LPR, rows, heads, slots, capacity);
    if (!rm.active) return;
    const int upr = hd >> 3;
    const int64_t src = (rm.slot * heads + rm.h) * (int64_t)hd;
    const int64_t dst = rm.t * ld_out + (int64_t)rm.h * hd;
    float sinv = 1.0f;
    if constexpr (ST != kStoreBf16) sinv = per_head ? scale_inv[rm.h] : scale_inv[rm.slot * heads + rm.h];
#pragma unroll
    for (int i = 0; i < UPL; ++i) {
        const int u = j + i * LPR;
        if (u >= upr) break;
        float v[8];
        uint4 raw16;
        if constexpr (ST == kStoreBf16) {
            raw16 = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(cache) + src + (int64_t)u * 8);
            if constexpr (!OUT_BF16) {
                const uint32_t w[4] = {raw16.x, raw16.y, raw16.z, raw16.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = __uint_as_float(w[e] << 16);
                    v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                }
            }
        } else {
            const uint2 c = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(cache) + src +
                                                            (int64_t)u * 8);
            decode4<ST>(c.x, v);
            decode4<ST>(c.y, v + 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = v[e] * sinv;
        }
        if constexpr (OUT_BF16) {
            uint4 w;
            if constexpr (ST == kStoreBf16) {
                w = raw16;
            } else {
                w.x = pack_bf16(v[0], v[1]);
                w.y = pack_bf16(v[2], v[3]);
                w.z = pack_bf16(v[4], v[5]);
                w.w = pack_bf16(v[6], v[7]);
            }
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + dst + (int64_t)u * 8) = w;
        } else {
            float* o = reinterpret_cast<float*>(out) + dst + (int64_t)u * 8;
            *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
    }
}

int lanes_per_row(int hd) {
    const int upr = hd / 8;
    return upr <= 8 ? 8 : upr <= 16 ? 16 : upr <= 32 ? 32 : 64;
}

unsigned blocks_for(int64_t rows, int lpr) {
    const int64_t per = kThreads / lpr;
    return (unsigned)((rows + per - 1) / per);
}

template <typename InT, int ST, bool DIAG>
hipError_t store_lpr(const KvStoreArgs& a) {
    const int lpr = lanes_per_row(a.head_dim);
    const int64_t rows = a.n_tokens * a.heads;
    const dim3 grid(blocks_for(rows, lpr)), block(kThreads);
    const InT* x = static_cast<const InT*>(a.x);
#define FP8MI_KV_STORE(L)                                                                                    \
    hipLaunchKernelGGL((k_kv_store<InT, ST, L, DIAG>), grid, block, 0, a.stream, x, a.ld, rows, a.heads,    \
                       a.head_dim, a.slots, a.capacity, a.per_head, a.pow2, a.cache, a.scale_inv, a.diag)
    switch (lpr) {
    case 8: FP8MI_KV_STORE(8); break;
    case 16: FP8MI_KV_STORE(16); break;
    case 32: FP8MI_KV_STORE(32); break;
    default: FP8MI_KV_STORE(64); break;
    }
#undef FP8MI_KV_STORE
    return hipGetLastError();
}

template <typename InT>
hipError_t store_in(const KvStoreArgs& a) {
    const bool d = a.diag != nullptr;
    switch (a.storage) {
    case FP8_KV_E4M3: return d ? store_lpr<InT, kE4M3, true>(a) : store_lpr<InT, kE4M3, false>(a);
    case FP8_KV_E5M2: return d ? store_lpr<InT, kE5M2, true>(a) : store_lpr<InT, kE5M2, false>(a);
    default: return store_lpr<InT, kStoreBf16, false>(a);
    }
}

template <int ST, bool OUT_BF16>
hipError_t load_lpr(const KvLoadArgs& a) {
    const int lpr = lanes_per_row(a.head_dim);
    const int64_t rows = a.n_tokens * a.heads;
    const dim3 grid(blocks_for(rows, lpr)), block(kThreads);
#define FP8MI_KV_LOAD(L)                                                                                      \
    hipLaunchKernelGGL((k_kv_load<ST, OUT_BF16, L>), grid, block, 0, a.stream, a.cache, a.scale_inv,         \
                       a.per_head, a.capacity, a.heads, a.head_dim, a.slots, rows, a.out, a.ld_out)
    switch (lpr) {
    case 8: FP8MI_KV_LOAD(8); break;
    case 16: FP8MI_KV_LOAD(16); break;
    case 32: FP8MI_KV_LOAD(32); break;
    default: FP8MI_KV_LOAD(64); break;
    }
#undef FP8MI_KV_LOAD
    return hipGetLastError();
}

template <bool OUT_BF16>
hipError_t load_out(const KvLoadArgs& a) {
    switch (a.storage) {
    case FP8_KV_E4M3: return load_lpr<kE4M3, OUT_BF16>(a);
    case FP8_KV_E5M2: return load_lpr<kE5M2, OUT_BF16>(a);
    default: return load_lpr<kStoreBf16, OUT_BF16>(a);
    }
}

}  // namespace

hipError_t launch_kv_store(const KvStoreArgs& a) {
    if (a.n_tokens == 0 || a.heads == 0) return hipSuccess;
    return a.in_bf16 ? store_in<uint16_t>(a) : store_in<float>(a);
}

hipError_t launch_kv_load(const KvLoadArgs& a) {
    if (a.n_tokens == 0 || a.heads == 0) return hipSuccess;
    return a.out_bf16 ? load_out<true>(a) : load_out<false>(a);
}

}  // namespace fp8mi
