// quantize.hip -- amax reduction, scale and saturating RNE cast to E4M3/E5M2
// on gfx950, at tensor / row / 1x128 / 128x128 granularity, just in time or
// delayed from an amax-history ring, optionally written transposed.
//
// Method ([DeepL bets on FP8, hmyw.cn] 2.3): a scaling factor per tensor, per
// row or per block maps the values into FP8's range; delayed scaling takes the
// factor from previous steps' statistics instead of a synchronous amax.
// [Soup, lbrq.cn] recipe table: rowwise scales are powers of two.
//
// All kernels stream HBM with 16-byte loads along rows: a "unit" is 8
// consecutive elements of one row (16 B of bf16, 32 B of fp32) that becomes
// 8 code bytes.  amax is a max over binary32 magnitude bits (exact, order
// free).  Every kernel is memory bound; the per-element ALU work is a bf16
// unpack, one multiply, a 4-instruction saturation clamp and half a packed
// convert.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "cast_unit.hpp"
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

constexpr int kThreads = 256;
using namespace cast;

// Unit u of a [rows x cols] matrix: rows == 1 is the flat (contiguous) case.
struct UnitGeom {
    int64_t rows, cols, ld, ldq;
    uint32_t upr;      // units per row
    uint32_t units;    // rows * upr
    __device__ __forceinline__ void locate(uint32_t u, int64_t& off, int64_t& qoff, int& nvalid) const {
        int64_t r, c;
        if (rows == 1) {
            r = 0;
            c = (int64_t)u * 8;
        } else {
            const uint32_t rr = u / upr;
            r = rr;
            c = (int64_t)(u - rr * upr) * 8;
        }
        off = r * ld + c;
        qoff = r * ldq + c;
        const int64_t rem = cols - c;
        nvalid = rem >= 8 ? 8 : (int)rem;
    }
};

// Block-wide max into thread 0 (256 threads = 4 waves).
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* lds) {
    v = wave_max_u32(v);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) lds[w] = v;
    __syncthreads();
    uint32_t r = 0;
    if (threadIdx.x == 0) r = max(max(lds[0], lds[1]), max(lds[2], lds[3]));
    return r;
}

// Max over partials[0..n) computed by the whole block, returned to every
// thread.  This is how per-tensor maxima are combined: each producer block
// stores its own partial with a plain store and the consumer reduces them,
// so no kernel issues same-address device-scope atomics (those serialize
// across the 8 XCDs).
__device__ __forceinline__ uint32_t reduce_partials(const uint32_t* __restrict__ partials, int n,
                                                    uint32_t* lds) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) m = max(m, partials[i]);
    m = wave_max_u32(m);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) lds[w] = m;
    __syncthreads();
    m = max(max(lds[0], lds[1]), max(lds[2], lds[3]));
    __syncthreads();
    return m;
}

// Delayed scale ([DeepL] 2.3): max over the history window; with an empty
// history, the just-in-time amax of the current step (bootstrap partials).
template <int FMT>
__device__ __forceinline__ float delayed_scale(const fp8_amax_history* h, const uint32_t* boot, int n_boot,
                                               bool pow2, uint32_t* lds) {
    const int32_t count = h->count;
    uint32_t basis = 0;
    if (count <= 0) {
        basis = reduce_partials(boot, n_boot, lds);
    } else {
        const int n = count > 16 ? 16 : count;
        for (int i = 0; i < n; ++i) basis = max(basis, __float_as_uint(h->amax[i]) & 0x7FFFFFFFu);
    }
    return scale_from_amax_bits<FMT>(basis, pow2);
}

// ------------------------------------------------------------------ kernels --
// Per-tensor cast modes: just in time (scale from this call's amax pass),
// delayed (scale from the history), and the spike guard's re-cast (scale
// recorded by the finish kernel; does nothing unless that kernel saw a spike).
constexpr int kModeJit = 0, kModeDelayed = 1, kModeRecast = 2;

__global__ void k_history_init(fp8_amax_history* h, int32_t len) {
    uint32_t* w = reinterpret_cast<uint32_t*>(h);
    const int i = threadIdx.x;
    if (i < (int)(sizeof(fp8_amax_history) / 4)) w[i] = 0u;
    __syncthreads();
    if (i == 0) {
        h->len = len;
        h->scale = 1.0f;
        h->scale_inv = 1.0f;
    }
}

constexpr int kUnroll = 4;

// Per-tensor amax, pass 1: grid-stride over units, one partial per block.
// `gate` non-null: run only while the history is empty (delayed bootstrap).
// FLAT: the tensor is one contiguous, 16-byte aligned run of g.cols
// elements (g.rows == 1, vec_in), so every unit but a ragged last one is
// whole and loads with plain indexing; block 0's thread 0 takes the last.
template <typename InT, bool FLAT>
__global__ __launch_bounds__(kThreads) void k_amax_partials(const InT* __restrict__ x, UnitGeom g,
                                                            bool vec_in, uint32_t* __restrict__ partials,
                                                            const fp8_amax_history* gate) {
    __shared__ uint32_t lds[16];
    if (gate != nullptr && gate->count != 0) return;
    const uint32_t stride = gridDim.x * kThreads;
    uint32_t m = 0;
    if constexpr (FLAT) {
        const uint32_t whole = (uint32_t)(g.cols / 8);
        for (uint32_t u0 = blockIdx.x * kThreads + threadIdx.x; u0 < whole; u0 += stride * kUnroll) {
            Pack<InT> p[kUnroll];
#pragma unroll
            for (int i = 0; i < kUnroll; ++i) {
                const uint32_t u = u0 + i * stride;
                p[i] = u < whole ? load_flat<InT>(x, u) : Pack<InT>{};
            }
#pragma unroll
            for (int i = 0; i < kUnroll; ++i) m = max(m, p[i].abs_max());
        }
        if (whole < g.units && blockIdx.x == 0 && threadIdx.x == 0) {
            int64_t off, qoff;
            int nv;
            g.locate(whole, off, qoff, nv);
            m = max(m, load_unit<InT>(x, off, nv, false).abs_max());
        }
    } else for (uint32_t u0 = blockIdx.x * kThreads + threadIdx.x; u0 < g.units; u0 += stride * kUnroll) {
        Pack<InT> p[kUnroll];
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const uint32_t u = u0 + i * stride;
            if (u < g.units) {
                int64_t off, qoff; int nv;
                g.locate(u, off, qoff, nv);
                p[i] = load_unit<InT>(x, off, nv, vec_in);
            }
        }
#pragma unroll
        for (int i = 0; i < kUnroll; ++i)
            if (u0 + i * stride < g.units) m = max(m, p[i].abs_max());
    }
    const uint32_t bm = block_max(m, lds);
    if (threadIdx.x == 0) partials[blockIdx.x] = bm;
}

// Pass 2 of the standalone per-tensor amax.
__global__ __launch_bounds__(kThreads) void k_reduce_amax(const uint32_t* __restrict__ partials, int n,
                                                          float* amax_out) {
    __shared__ uint32_t lds[16];
    const uint32_t m = reduce_partials(partials, n, lds);
    if (threadIdx.x == 0) amax_out[0] = __uint_as_float(m);
}

__global__ void k_history_set_guard(fp8_amax_history* h, float threshold) {
    if (threadIdx.x == 0) h->spike_threshold = threshold;
}

__global__ void k_zero_words(uint32_t* w, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) w[i] = 0u;
}

// After a delayed cast: combine the cast blocks' partials into this step's
// amax, push it into the ring and precompute the next scale (one block).
// GUARD ([DeepL bets on FP8] 2.3, recovery from a distribution jump): when
// this amax exceeds spike_threshold x the window max (fp32 product; only with
// a non-empty window and a positive threshold), record the just-in-time
// scale for the re-cast kernel and give scale_inv_out its inverse.  The
// first cast counted its diagnostics into `diag_tmp`; they reach `diag` only
// when that cast stands.
template <int FMT, bool GUARD>
__global__ __launch_bounds__(kThreads) void k_delayed_finish(fp8_amax_history* h,
                                                             const uint32_t* __restrict__ partials, int n,
                                                             bool pow2, float* amax_out, float* scale_inv_out,
                                                             fp8_diag* diag, fp8_diag* diag_tmp) {
    __shared__ uint32_t lds[16];
    const uint32_t cur = reduce_partials(partials, n, lds);
    if (threadIdx.x != 0) return;
    const float amax_now = __uint_as_float(cur);
    amax_out[0] = amax_now;
    int32_t len = h->len;
    len = len < 1 ? 1 : (len > 16 ? 16 : len);
    int32_t pos = h->pos;
    pos = (pos < 0 || pos >= len) ? 0 : pos;
    if constexpr (GUARD) {
        const int32_t count0 = h->count < 0 ? 0 : (h->count > len ? len : h->count);
        uint32_t wbits = 0;
        for (int i = 0; i < count0; ++i) wbits = max(wbits, __float_as_uint(h->amax[i]) & 0x7FFFFFFFu);
        const float thr = h->spike_threshold;
        const bool spiked = count0 > 0 && thr > 0.0f && amax_now > thr * __uint_as_float(wbits);
        h->internal[0] = spiked ? 1u : 0u;
        if (spiked) {
            const float sj = scale_from_amax_bits<FMT>(cur, pow2);
            h->internal[1] = __float_as_uint(sj);
            scale_inv_out[0] = recip_rn(sj);
            h->spikes = h->spikes + 1u;
        }
        if (diag_tmp != nullptr) {
            if (!spiked && diag != nullptr) {
                diag->sat_count += diag_tmp->sat_count;
                diag->nonfinite_count += diag_tmp->nonfinite_count;
                diag->underflow_count += diag_tmp->underflow_count;
            }
            diag_tmp->sat_count = 0u;
            diag_tmp->nonfinite_count = 0u;
            diag_tmp->underflow_count = 0u;
        }
    }
    h->amax[pos] = amax_now;
    h->pos = (pos + 1) % len;
    const int32_t count = h->count < len ? h->count + 1 : len;
    h->count = count;
    uint32_t basis = 0;
    for (int i = 0; i < count; ++i) basis = max(basis, __float_as_uint(h->amax[i]) & 0x7FFFFFFFu);
    const float s = scale_from_amax_bits<FMT>(basis, pow2);
    h->scale = s;
    h->scale_inv = 1.0f / s;
    h->steps = h->steps + 1;
}

// Per-tensor cast.  JIT: s from the amax partials of pass 1 (block 0 also
// writes amax_out).  DELAYED: s from the history (or the bootstrap partials
// while it is empty); each block stores its own amax partial for the finish
// kernel.  RECAST: s recorded by a guarded finish kernel, or nothing to do.
template <typename InT, int FMT, int MODE, bool DIAG, bool FLAT>
__global__ __launch_bounds__(kThreads) void k_cast_tensor(
    const InT* __restrict__ x, UnitGeom g, bool vec_in, uint8_t* __restrict__ q, bool vec_out,
    const uint32_t* __restrict__ partials_in, int n_in, const fp8_amax_history* hist, bool pow2,
    float* __restrict__ scale_inv_out, float* __restrict__ amax_out, fp8_diag* diag,
    uint32_t* __restrict__ partials_out) {
    __shared__ uint32_t lds[16];
    constexpr bool DELAYED = MODE == kModeDelayed;
    float s;
    if constexpr (MODE == kModeRecast) {
        if (hist->internal[0] == 0u) return;
        s = __uint_as_float(hist->internal[1]);
    } else if constexpr (DELAYED) {
        s = delayed_scale<FMT>(hist, partials_in, n_in, pow2, lds);
    } else {
        const uint32_t am = reduce_partials(partials_in, n_in, lds);
        s = scale_from_amax_bits<FMT>(am, pow2);
        if (blockIdx.x == 0 && threadIdx.x == 0) amax_out[0] = __uint_as_float(am);
    }
    if (MODE != kModeRecast && blockIdx.x == 0 && threadIdx.x == 0) scale_inv_out[0] = recip_rn(s);

    const uint32_t stride = gridDim.x * kThreads;
    uint32_t m = 0;
    Counters cnt;
    if constexpr (FLAT) {     // contiguous input and codes: whole units, then the ragged last one
        const uint32_t whole = (uint32_t)(g.cols / 8);
        for (uint32_t u0 = blockIdx.x * kThreads + threadIdx.x; u0 < whole; u0 += stride * kUnroll) {
            Pack<InT> p[kUnroll];
#pragma unroll
            for (int i = 0; i < kUnroll; ++i) {
                const uint32_t u = u0 + i * stride;
                p[i] = u < whole ? load_flat<InT>(x, u) : Pack<InT>{};
            }
#pragma unroll
            for (int i = 0; i < kUnroll; ++i) {
                const uint32_t u = u0 + i * stride;
                if (u < whole) {
                    if constexpr (DELAYED) m = max(m, p[i].abs_max());
                    store_flat(q, u, encode_unit<FMT, DIAG>(p[i], s, cnt));
                }
            }
        }
        if (whole < g.units && blockIdx.x == 0 && threadIdx.x == 0) {
            int64_t off, qoff;
            int nv;
            g.locate(whole, off, qoff, nv);
            const Pack<InT> p = load_unit<InT>(x, off, nv, false);
            if constexpr (DELAYED) m = max(m, p.abs_max());
            store_unit(q, qoff, nv, false, encode_unit<FMT, DIAG>(p, s, cnt));
        }
    } else for (uint32_t u0 = blockIdx.x * kThreads + threadIdx.x; u0 < g.units; u0 += stride * kUnroll) {
        Pack<InT> p[kUnroll];
        int64_t qo[kUnroll];
        int nv[kUnroll];
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const uint32_t u = u0 + i * stride;
            nv[i] = 0;
            qo[i] = 0;
            if (u < g.units) {
                int64_t off;
                g.locate(u, off, qo[i], nv[i]);
                p[i] = load_unit<InT>(x, off, nv[i], vec_in);
            }
        }
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            if (nv[i] > 0) {
                if constexpr (DELAYED) m = max(m, p[i].abs_max());
                store_unit(q, qo[i], nv[i], vec_out, encode_unit<FMT, DIAG>(p[i], s, cnt));
            }
        }
    }
    if constexpr (DIAG) block_add_diag(cnt, lds, diag);
    if constexpr (DELAYED) {
        const uint32_t bm = block_max(m, lds);
        if (threadIdx.x == 0) partials_out[blockIdx.x] = bm;
    }
}

// Per-tensor cast written transposed: q[c][r] (the wgrad operands).  Blocks
// walk 128x128 tiles grid-stride; codes go through LDS with a 16-chunk XOR
// swizzle so that both the row-wise writes and the column gathers are
// conflict free, and each output row segment leaves as 16-byte stores
// (128 B per 8 lanes).  q2 != nullptr: the codes also go out untransposed
// (q2[r][c], ld ldq2) from the same pass, for a gradient that feeds both
// backward GEMMs.
template <typename InT, int FMT, int MODE, bool DIAG>
__global__ __launch_bounds__(kThreads) void k_cast_tensor_t(
    const InT* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, bool vec_in,
    uint8_t* __restrict__ q, int64_t ldq, bool vec_out16, const uint32_t* __restrict__ partials_in,
    int n_in, const fp8_amax_history* hist, bool pow2, float* __restrict__ scale_inv_out,
    float* __restrict__ amax_out, fp8_diag* diag, uint32_t* __restrict__ partials_out,
    uint8_t* __restrict__ q2, int64_t ldq2, bool vec_out2) {
    __shared__ uint32_t lds[16];
    __shared__ __attribute__((aligned(16))) uint8_t tile[128 * 128];
    constexpr bool DELAYED = MODE == kModeDelayed;
    float s;
    if constexpr (MODE == kModeRecast) {
        if (hist->internal[0] == 0u) return;
        s = __uint_as_float(hist->internal[1]);
    } else if constexpr (DELAYED) {
        s = delayed_scale<FMT>(hist, partials_in, n_in, pow2, lds);
    } else {
        const uint32_t am = reduce_partials(partials_in, n_in, lds);
        s = scale_from_amax_bits<FMT>(am, pow2);
        if (blockIdx.x == 0 && threadIdx.x == 0) amax_out[0] = __uint_as_float(am);
    }
    if (MODE != kModeRecast && blockIdx.x == 0 && threadIdx.x == 0) scale_inv_out[0] = recip_rn(s);

    const int t = threadIdx.x;
    const int cu = t & 15, rr = t >> 4;
    const int64_t tiles_c = (cols + 127) / 128;
    const int64_t tiles = ((rows + 127) / 128) * tiles_c;
    uint32_t m = 0;
    Counters cnt;
    // this thread's 8 units of tile tl (zeros past the matrix)
    Pack<InT> p[8];
    auto load_tile = [&](int64_t tl) {
        const int64_t r0 = (tl / tiles_c) * 128, c = (tl % tiles_c) * 128 + cu * 8;
        const int nvc = (int)(cols - c >= 8 ? 8 : (cols - c > 0 ? cols - c : 0));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = r0 + rr + 16 * i;
            const int nv = (r < rows) ? nvc : 0;
            if (nv > 0) {
                p[i] = load_unit<InT, true>(x, r * ld + c, nv, vec_in);
            } else {
#pragma unroll
                for (int k = 0; k < (int)(sizeof(p[i].w) / 4); ++k) p[i].w[k] = 0u;
            }
        }
    };
    // grid-stride over tiles; the next tile's loads are issued as soon as
    // this tile's codes are in LDS, so they overlap its transposed stores
    if ((int64_t)blockIdx.x < tiles) load_tile(blockIdx.x);
    for (int64_t tl = blockIdx.x; tl < tiles; tl += gridDim.x) {
        const int64_t r0 = (tl / tiles_c) * 128, c0 = (tl % tiles_c) * 128;
        const int64_t c = c0 + cu * 8;
        const int nvc = (int)(cols - c >= 8 ? 8 : (cols - c > 0 ? cols - c : 0));
        __syncthreads();   // the previous tile's gathers are done with `tile`
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = rr + 16 * i;
            if constexpr (DELAYED) m = max(m, p[i].abs_max());
            const uint2 codes = encode_unit<FMT, DIAG>(p[i], s, cnt);
            const int pos = cu ^ ((r >> 4) & 15);
            *reinterpret_cast<uint2*>(&tile[r * 128 + pos * 8]) = codes;
            if (q2 != nullptr && r0 + r < rows && nvc > 0) store_unit(q2, (r0 + r) * ldq2 + c, nvc, vec_out2, codes);
        }
        __syncthreads();
        if (tl + gridDim.x < tiles) load_tile(tl + gridDim.x);
        // gather: thread (rs = t % 8, cl4 = t / 8) takes input rows rs*16 ..
        // rs*16+15 of input columns 4*cl4 .. 4*cl4+3 as 16 words (one row
        // each), transposes the four 4x4 byte blocks with byte permutes and
        // leaves 16 bytes for each of the 4 output rows; 8 consecutive lanes
        // write one 128-byte output row segment.
        {
            const int rs = t & 7, cl4 = t >> 3;
            const int chunk = (cl4 >> 1) ^ rs;          // the write swizzle; row >> 4 == rs here
            uint32_t wv[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                wv[k] = *reinterpret_cast<const uint32_t*>(&tile[(rs * 16 + k) * 128 + chunk * 8 + (cl4 & 1) * 4]);
            uint32_t o[4][4];   // [output row c][input rows 4*blk .. 4*blk+3]
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const uint32_t w0 = wv[4 * blk], w1 = wv[4 * blk + 1], w2 = wv[4 * blk + 2], w3 = wv[4 * blk + 3];
                // byte i of perm(a, b, sel) is byte sel_i of the 8 bytes {b (0..3), a (4..7)}
                const uint32_t lo01 = __builtin_amdgcn_perm(w1, w0, 0x05010400u);   // w0.0 w1.0 w0.1 w1.1
                const uint32_t lo23 = __builtin_amdgcn_perm(w3, w2, 0x05010400u);   // w2.0 w3.0 w2.1 w3.1
                const uint32_t hi01 = __builtin_amdgcn_perm(w1, w0, 0x07030602u);   // w0.2 w1.2 w0.3 w1.3
                const uint32_t hi23 = __builtin_amdgcn_perm(w3, w2, 0x07030602u);   // w2.2 w3.2 w2.3 w3.3
                o[0][blk] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);          // column 0 of rows 0..3
                o[1][blk] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
                o[2][blk] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
                o[3][blk] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
            }
            const int64_t ocol = r0 + rs * 16;
            const int64_t remr = rows - ocol;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t orow = c0 + cl4 * 4 + c;
                if (orow < cols && remr > 0) {
                    uint8_t* dst = q + orow * ldq + ocol;
                    if (vec_out16 && remr >= 16) {
                        *reinterpret_cast<uint4*>(dst) = make_uint4(o[c][0], o[c][1], o[c][2], o[c][3]);
                    } else {
                        for (int b = 0; b < 16 && b < remr; ++b)
                            dst[b] = (uint8_t)((o[c][b >> 2] >> (8 * (b & 3))) & 0xFFu);
                    }
                }
            }
        }
    }
    if constexpr (DIAG) block_add_diag(cnt, lds, diag);
    if constexpr (DELAYED) {
        const uint32_t bm = block_max(m, lds);
        if (threadIdx.x == 0) partials_out[blockIdx.x] = bm;
    }
}

// Row-wise: a persistent grid of waves, wave w taking rows w, w + W, w + 2W
// ... (W waves in all).  A row of at most 64*NU units is held in registers,
// and the next row's loads are in flight while this one is reduced and
// encoded (two register sets, alternating); longer rows are read twice.
// [DeepL] 2.3 (per-row scaling of activations); [Soup] rowwise recipe
// (power-of-two scales).
template <typename InT, int FMT, bool DIAG, bool WRITE_Q, int NU = 8>
__global__ __launch_bounds__(kThreads) void k_cast_rows(
    const InT* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, bool vec_in,
    uint8_t* __restrict__ q, int64_t ldq, bool vec_out, bool pow2,
    float* __restrict__ scale_inv_out, float* __restrict__ amax_out, fp8_diag* diag) {
    __shared__ uint32_t lds[16];
    const int lane = threadIdx.x & 63;
    const int64_t W = (int64_t)gridDim.x * 4;
    const int64_t r0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t upr = (cols + 7) / 8;
    Counters cnt;
    auto nvalid = [&](int64_t c) { return cols - c >= 8 ? 8 : (int)(cols - c); };
    // the row's amax, its scale, and (WRITE_Q) its codes from units held in p
    auto finish = [&](const Pack<InT>* p, int64_t r) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < NU; ++i)
            if (lane + 64 * i < upr) m = max(m, p[i].abs_max());
        m = wave_max_u32(m);
        const float s = scale_from_amax_bits<FMT>(m, pow2);
        if (lane == 0) {
            amax_out[r] = __uint_as_float(m);
            if (WRITE_Q) scale_inv_out[r] = recip_rn(s);
        }
        if constexpr (WRITE_Q) {
            uint8_t* qr = q + r * ldq;
#pragma unroll
            for (int i = 0; i < NU; ++i) {
                const int64_t u = lane + 64 * i;
                if (u < upr) store_unit(qr, u * 8, nvalid(u * 8), vec_out, encode_unit<FMT, DIAG>(p[i], s, cnt));
            }
        }
    };
    auto load = [&](Pack<InT>* p, int64_t r) {
        const InT* xr = x + r * ld;
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int64_t u = lane + 64 * i;
            if (u < upr) p[i] = load_unit<InT>(xr, u * 8, nvalid(u * 8), vec_in);
        }
    };
    if (upr <= 64 * NU) {
        Pack<InT> pa[NU], pb[NU];
        if (r0 < rows) load(pa, r0);
        for (int64_t r = r0; r < rows; r += 2 * W) {
            const int64_t r1 = r + W, r2 = r + 2 * W;
            if (r1 < rows) load(pb, r1);
            finish(pa, r);
            if (r2 < rows) load(pa, r2);
            if (r1 < rows) finish(pb, r1);
        }
    } else {
        for (int64_t r = r0; r < rows; r += W) {
            const InT* xr = x + r * ld;
            uint32_t m = 0;
            for (int64_t u = lane; u < upr; u += 64)
                m = max(m, load_unit<InT>(xr, u * 8, nvalid(u * 8), vec_in).abs_max());
            m = wave_max_u32(m);
            const float s = scale_from_amax_bits<FMT>(m, pow2);
            if (lane == 0) {
                amax_out[r] = __uint_as_float(m);
                if (WRITE_Q) scale_inv_out[r] = recip_rn(s);
            }
            if constexpr (WRITE_Q) {
                uint8_t* qr = q + r * ldq;
                for (int64_t u = lane; u < upr; u += 64)
                    store_unit(qr, u * 8, nvalid(u * 8), vec_out,
                               encode_unit<FMT, DIAG>(load_unit<InT>(xr, u * 8, nvalid(u * 8), vec_in), s, cnt));
            }
        }
    }
    if constexpr (DIAG) block_add_diag(cnt, lds, diag);
}

// 1x128 blocks: 16 lanes per block of 128 elements, UNR blocks per lane in
// flight.  amax/scale arrays are [rows x ceil(cols/128)].
template <typename InT, int FMT, bool DIAG, bool WRITE_Q>
__global__ __launch_bounds__(kThreads) void k_cast_1x128(
    const InT* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, bool vec_in,
    uint8_t* __restrict__ q, int64_t ldq, bool vec_out, bool pow2,
    float* __restrict__ scale_inv_out, float* __restrict__ amax_out, fp8_diag* diag) {
    __shared__ uint32_t lds[16];
    const int64_t gc = (cols + 127) / 128;
    const int64_t G = rows * gc;
    const int slot = threadIdx.x >> 4, j = threadIdx.x & 15;
    const int64_t stride = (int64_t)gridDim.x * 16;
    Counters cnt;
    for (int64_t g0 = (int64_t)blockIdx.x * 16 + slot; g0 - slot < G; g0 += stride * kUnroll) {
        Pack<InT> p[kUnroll];
        uint32_t m[kUnroll];
        int nv[kUnroll];
        int64_t xo[kUnroll], qo[kUnroll];
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int64_t g = g0 + i * stride;
            m[i] = 0; nv[i] = 0; xo[i] = 0; qo[i] = 0;
            if (g < G) {
                const int64_t r = g / gc, kb = g - r * gc;
                const int64_t c = kb * 128 + j * 8;
                nv[i] = cols - c >= 8 ? 8 : (cols - c > 0 ? (int)(cols - c) : 0);
                xo[i] = r * ld + c;
                qo[i] = r * ldq + c;
                if (nv[i] > 0) {
                    p[i] = load_unit<InT, true>(x, xo[i], nv[i], vec_in);
                    m[i] = p[i].abs_max();
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const uint32_t gm = group_max_u32<16>(m[i]);
            const int64_t g = g0 + i * stride;
            if (g < G) {
                const float s = scale_from_amax_bits<FMT>(gm, pow2);
                if (j == 0) {
                    amax_out[g] = __uint_as_float(gm);
                    if (WRITE_Q) scale_inv_out[g] = recip_rn(s);
                }
                if constexpr (WRITE_Q) {
                    if (nv[i] > 0) store_unit(q, qo[i], nv[i], vec_out, encode_unit<FMT, DIAG>(p[i], s, cnt));
                }
            }
        }
    }
    if constexpr (DIAG) block_add_diag(cnt, lds, diag);
}

// 128x128 blocks: one workgroup per block, 8 units per thread held in
// registers.  amax/scale arrays are [ceil(rows/128) x ceil(cols/128)].
template <typename InT, int FMT, bool DIAG, bool WRITE_Q>
__global__ __launch_bounds__(kThreads) void k_cast_128x128(
    const InT* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, bool vec_in,
    uint8_t* __restrict__ q, int64_t ldq, bool vec_out, bool pow2,
    float* __restrict__ scale_inv_out, float* __restrict__ amax_out, fp8_diag* diag) {
    __shared__ uint32_t lds[16];
    const int t = threadIdx.x;
    const int cu = t & 15, rr = t >> 4;
    const int64_t r0 = (int64_t)blockIdx.y * 128;
    const int64_t c = (int64_t)blockIdx.x * 128 + cu * 8;
    const int nvc = (int)(cols - c >= 8 ? 8 : (cols - c > 0 ? cols - c : 0));
    Pack<InT> p[8];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = r0 + rr + 16 * i;
        if (r < rows && nvc > 0) {
            p[i] = load_unit<InT, true>(x, r * ld + c, nvc, vec_in);
            m = max(m, p[i].abs_max());
        }
    }
    const uint32_t bm0 = block_max(m, lds);
    __shared__ uint32_t bcast;
    if (t == 0) bcast = bm0;
    __syncthreads();
    const uint32_t bm = bcast;
    const float s = scale_from_amax_bits<FMT>(bm, pow2);
    const int64_t g = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    if (t == 0) {
        amax_out[g] = __uint_as_float(bm);
        if (WRITE_Q) scale_inv_out[g] = recip_rn(s);
    }
    Counters cnt;
    if constexpr (WRITE_Q) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = r0 + rr + 16 * i;
            if (r < rows && nvc > 0)
                store_unit(q, r * ldq + c, nvc, vec_out, encode_unit<FMT, DIAG>(p[i], s, cnt));
        }
    }
    if constexpr (DIAG) block_add_diag(cnt, lds, diag);
}

// ---------------------------------------------------------------- host side --
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Scratch layout (uint32 words of the per-stream scratch, kScratchWords).
constexpr int kScratchCastPartials = 0;      // <= kMaxCastBlocks partials of a delayed cast
constexpr int kScratchAmaxPartials = 4096;   // <= kMaxAmaxBlocks partials of pass 1
constexpr int kScratchDiag = 8192;           // fp8_diag of a guarded delayed cast (zero between calls)
constexpr int64_t kMaxCastBlocks = 4096;
constexpr int64_t kMaxAmaxBlocks = 1024;   // a stream needs about 4 workgroups per CU (measured)
static_assert(kScratchAmaxPartials + kMaxAmaxBlocks <= kScratchDiag, "scratch layout");
static_assert(kScratchDiag + 4 <= kScratchGroupTable, "scratch layout: the grouped GEMM's table follows");

constexpr int64_t kTBlocksPerCU = 4;     // transposed cast: tiles per block = tiles / (CUs * this)
constexpr int64_t kRowBlocksPerCU = 3;   // measured: 2, 3 and 4 per CU, 3 fastest

inline unsigned grid_for(int64_t work_items, int64_t per_block, int64_t cap) {
    int64_t b = (work_items + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (unsigned)b;
}

template <typename InT, int FMT>
hipError_t quantize_geom(const QuantArgs& a, const InT* x, int esz);

template <typename InT, int FMT>
hipError_t quantize_typed(const QuantArgs& a) {
    const InT* x = static_cast<const InT*>(a.x);
    const int esz = (int)sizeof(InT);
    // an empty tensor still yields its scale (1) and amax (0) through the flat path
    QuantArgs a_eff = a;
    if (a.rows == 0 || a.cols == 0) a_eff.transpose = false;
    return quantize_geom<InT, FMT>(a_eff, x, esz);
}

template <typename InT, int FMT>
hipError_t quantize_geom(const QuantArgs& a, const InT* x, int esz) {
    const bool diag = a.diag != nullptr;
    const bool contiguous_in = a.ld == a.cols;
    const bool contiguous_out = !a.write_q || a.transpose || a.ldq == a.cols;
    // 2-D geometry, or the flat view of a contiguous matrix
    UnitGeom g;
    if (contiguous_in && contiguous_out && !a.transpose) {
        g.rows = 1; g.cols = a.rows * a.cols; g.ld = g.cols; g.ldq = g.cols;
    } else {
        g.rows = a.rows; g.cols = a.cols; g.ld = a.ld; g.ldq = a.ldq;
    }
    g.upr = (uint32_t)((g.cols + 7) / 8);
    g.units = (uint32_t)(g.rows * (int64_t)g.upr);
    const bool vec_in = aligned(x, 16) && (g.rows == 1 || (g.ld * esz) % 16 == 0);
    const bool vec_out = a.q != nullptr && aligned(a.q, 8) && (g.rows == 1 || g.ldq % 8 == 0);
    const unsigned cap = (unsigned)(a.num_cus * 8);
    hipStream_t st = a.stream;

    if (a.gran == FP8_GRAN_TENSOR) {
        uint32_t* cast_partials = a.scratch + kScratchCastPartials;
        uint32_t* amax_partials = a.scratch + kScratchAmaxPartials;
        const bool delayed = a.hist != nullptr;
        const unsigned agrid = grid_for(g.units, (int64_t)kThreads * kUnroll, kMaxAmaxBlocks);
        const unsigned cgrid = grid_for(g.units, (int64_t)kThreads * kUnroll, cap);
        const int64_t tiles = ((a.rows + 127) / 128) * ((a.cols + 127) / 128);
        const unsigned tgrid = grid_for(tiles, 1, std::min<int64_t>(kMaxCastBlocks, (int64_t)a.num_cus * kTBlocksPerCU));
        const bool v16 = a.q != nullptr && aligned(a.q, 16) && a.ldq % 16 == 0;
        const bool v2 = a.q2 != nullptr && aligned(a.q2, 8) && a.ldq2 % 8 == 0;
        // contiguous, aligned input (and codes): the kernels' plain-indexed fast path
        const bool flat_in = g.rows == 1 && vec_in;
        const bool flat = flat_in && vec_out;
        // pass 1: amax partials (JIT), or the bootstrap partials of an empty history
        if (flat_in)
            hipLaunchKernelGGL((k_amax_partials<InT, true>), dim3(agrid), dim3(kThreads), 0, st, x, g, vec_in,
                               amax_partials, (const fp8_amax_history*)a.hist);
        else
            hipLaunchKernelGGL((k_amax_partials<InT, false>), dim3(agrid), dim3(kThreads), 0, st, x, g, vec_in,
                               amax_partials, (const fp8_amax_history*)a.hist);
        if (!a.write_q) {
            hipLaunchKernelGGL(k_reduce_amax, dim3(1), dim3(kThreads), 0, st, (const uint32_t*)amax_partials,
                               (int)agrid, a.amax);
            return hipGetLastError();
        }
#define FP8MI_TENSOR_CAST(MODE, DG, DIAGP)                                                                  \
    do {                                                                                                  \
        if (a.transpose)                                                                                  \
            hipLaunchKernelGGL((k_cast_tensor_t<InT, FMT, MODE, DG>), dim3(tgrid), dim3(kThreads), 0, st, x,    \
                               a.rows, a.cols, a.ld, vec_in, a.q, a.ldq, v16,                             \
                               (const uint32_t*)amax_partials, (int)agrid,                                \
                               (const fp8_amax_history*)a.hist, a.pow2, a.scale_inv, a.amax, DIAGP,       \
                               cast_partials, a.q2, a.ldq2, v2);                                          \
        else if (flat)                                                                                    \
            hipLaunchKernelGGL((k_cast_tensor<InT, FMT, MODE, DG, true>), dim3(cgrid), dim3(kThreads), 0, st, x,\
                               g, vec_in, a.q, vec_out, (const uint32_t*)amax_partials, (int)agrid,       \
                               (const fp8_amax_history*)a.hist, a.pow2, a.scale_inv, a.amax, DIAGP,       \
                               cast_partials);                                                            \
        else                                                                                              \
            hipLaunchKernelGGL((k_cast_tensor<InT, FMT, MODE, DG, false>), dim3(cgrid), dim3(kThreads), 0, st,  \
                               x, g, vec_in, a.q, vec_out, (const uint32_t*)amax_partials, (int)agrid,    \
                               (const fp8_amax_history*)a.hist, a.pow2, a.scale_inv, a.amax, DIAGP,       \
                               cast_partials);                                                            \
    } while (0)
        if (delayed) {
            // with the guard, the first cast's diagnostics wait in scratch
            fp8_diag* diag_tmp = a.guard ? reinterpret_cast<fp8_diag*>(a.scratch + kScratchDiag) : nullptr;
            fp8_diag* d1 = a.guard ? diag_tmp : a.diag;
            if (diag) FP8MI_TENSOR_CAST(kModeDelayed, true, d1);
            else FP8MI_TENSOR_CAST(kModeDelayed, false, d1);
            const int nparts = (int)(a.transpose ? tgrid : cgrid);
            if (a.guard) {
                hipLaunchKernelGGL((k_delayed_finish<FMT, true>), dim3(1), dim3(kThreads), 0, st, a.hist,
                                   (const uint32_t*)cast_partials, nparts, a.pow2, a.amax, a.scale_inv, a.diag,
                                   diag ? diag_tmp : nullptr);
                if (diag) FP8MI_TENSOR_CAST(kModeRecast, true, a.diag);
                else FP8MI_TENSOR_CAST(kModeRecast, false, a.diag);
            } else {
                hipLaunchKernelGGL((k_delayed_finish<FMT, false>), dim3(1), dim3(kThreads), 0, st, a.hist,
                                   (const uint32_t*)cast_partials, nparts, a.pow2, a.amax, a.scale_inv, a.diag,
                                   (fp8_diag*)nullptr);
            }
        } else {
            if (diag) FP8MI_TENSOR_CAST(kModeJit, true, a.diag);
            else FP8MI_TENSOR_CAST(kModeJit, false, a.diag);
        }
#undef FP8MI_TENSOR_CAST
        return hipGetLastError();
    }

    // group granularities: the 2-D geometry always
    const bool gvec_in = aligned(x, 16) && (a.ld * esz) % 16 == 0;
    const bool gvec_out = a.q != nullptr && aligned(a.q, 8) && a.ldq % 8 == 0;
#define FP8MI_GROUP_LAUNCH(KERNEL, GRID)                                                          \
    do {                                                                                          \
        if (!a.write_q)                                                                           \
            hipLaunchKernelGGL((KERNEL<InT, FMT, false, false>), GRID, dim3(kThreads), 0, st, x,  \
                               a.rows, a.cols, a.ld, gvec_in, a.q, a.ldq, gvec_out, a.pow2,       \
                               a.scale_inv, a.amax, a.diag);                                      \
        else if (diag)                                                                            \
            hipLaunchKernelGGL((KERNEL<InT, FMT, true, true>), GRID, dim3(kThreads), 0, st, x,    \
                               a.rows, a.cols, a.ld, gvec_in, a.q, a.ldq, gvec_out, a.pow2,       \
                               a.scale_inv, a.amax, a.diag);                                      \
        else                                                                                      \
            hipLaunchKernelGGL((KERNEL<InT, FMT, false, true>), GRID, dim3(kThreads), 0, st, x,   \
                               a.rows, a.cols, a.ld, gvec_in, a.q, a.ldq, gvec_out, a.pow2,       \
                               a.scale_inv, a.amax, a.diag);                                      \
    } while (0)

    if (a.gran == FP8_GRAN_ROW) {
        // a persistent grid of kRowBlocksPerCU blocks (4 waves each) per CU
        const dim3 grid(grid_for(a.rows, 4, (int64_t)a.num_cus * kRowBlocksPerCU));
        FP8MI_GROUP_LAUNCH(k_cast_rows, grid);
    } else if (a.gran == FP8_GRAN_BLOCK_1x128) {
        const int64_t G = a.rows * ((a.cols + 127) / 128);
        const dim3 grid(grid_for(G, 16 * kUnroll, (int64_t)a.num_cus * 8));
        FP8MI_GROUP_LAUNCH(k_cast_1x128, grid);
    } else {
        const dim3 grid((unsigned)((a.cols + 127) / 128), (unsigned)((a.rows + 127) / 128));
        FP8MI_GROUP_LAUNCH(k_cast_128x128, grid);
    }
#undef FP8MI_GROUP_LAUNCH
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a) {
    if (a.in_bf16) {
        return a.fmt == 0 ? quantize_typed<uint16_t, kE4M3>(a) : quantize_typed<uint16_t, kE5M2>(a);
    }
    return a.fmt == 0 ? quantize_typed<float, kE4M3>(a) : quantize_typed<float, kE5M2>(a);
}

hipError_t launch_history_init(fp8_amax_history* h, int32_t len, hipStream_t stream) {
    hipLaunchKernelGGL(k_history_init, dim3(1), dim3(64), 0, stream, h, len);
    return hipGetLastError();
}

hipError_t launch_history_set_guard(fp8_amax_history* h, float threshold, hipStream_t stream) {
    hipLaunchKernelGGL(k_history_set_guard, dim3(1), dim3(64), 0, stream, h, threshold);
    return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t* w, int n, hipStream_t stream) {
    hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(256), 0, stream, w, n);
    return hipGetLastError();
}

}  // namespace fp8mi
