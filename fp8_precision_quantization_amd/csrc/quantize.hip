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
#include <cstddef>
#include <mutex>

#include "cast_unit.hpp"
#include "device_common.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

constexpr int kThreads = 256;
constexpr int kMultiMax = FP8_MAX_TENSORS;
// Transposed cast: workgroups per CU (a workgroup's 4 waves take one SIMD
// each, so also the waves per SIMD its registers must allow).
constexpr int kTBlocksPerCU = 4;
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

// Block-wide max, returned to every thread.
__device__ __forceinline__ uint32_t block_max_all(uint32_t v, uint32_t* lds) {
    v = wave_max_u32(v);
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) lds[w] = v;
    __syncthreads();
    v = max(max(lds[0], lds[1]), max(lds[2], lds[3]));
    __syncthreads();
    return v;
}

// One block's max |x| over units [beg, end) of a [rows x cols] (ld) tensor
// (units of 8 elements in row-major order), to every thread: a piece of the
// just-in-time amax that the first delayed call needs while its history is
// still empty.
template <typename InT>
__device__ __forceinline__ uint32_t units_amax(const InT* __restrict__ x, int64_t rows, int64_t cols,
                                               int64_t ld, bool vec_in, int64_t beg, int64_t end, uint32_t* lds) {
    constexpr int U = 8;
    const int64_t upr = (cols + 7) / 8;
    uint32_t m = 0;
    for (int64_t u0 = beg + threadIdx.x; u0 < end; u0 += (int64_t)kThreads * U) {
        Pack<InT> p[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t u = u0 + (int64_t)i * kThreads;
            if (u < end) {
                const int64_t r = u / upr, c = (u - r * upr) * 8;
                p[i] = load_unit<InT>(x, r * ld + c, cols - c >= 8 ? 8 : (int)(cols - c), vec_in);
            } else {
                p[i] = Pack<InT>{};
            }
        }
#pragma unroll
        for (int i = 0; i < U; ++i) m = max(m, p[i].abs_max());
    }
    return block_max_all(m, lds);
}

// Delayed scaling ([DeepL bets on FP8] 2.3: the factor comes from earlier
// steps' statistics).  The history's sync words are zero between calls
// (fp8_history_init zeroes them, and so does the finish kernel of every
// call).  While the history is empty the call needs this step's just-in-time
// amax first: the tensor is cut into as many slices as the grid has
// workgroups, each arriving workgroup claims slices from sync[2] until none
// is left, folds each slice's max into sync[1] and counts it done in
// sync[0].  A workgroup then waits until every slice is done.  It waits only
// for slices already claimed, i.e. for running workgroups, so the scheme
// assumes nothing about which workgroups are resident.  The words are
// exchanged only through atomic read-modify-writes, each waited for before
// the next: no fence, so no workgroup writes back or invalidates its XCD's
// L2.
__device__ __forceinline__ uint32_t sync_read(uint32_t* w) { return atomicOr(w, 0u); }

// Wait until this thread's memory operations, atomics included, are done.
__device__ __forceinline__ void wait_memory() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The wait for the slices is bounded: should they never all be counted (a
// history whose sync words were not zero), a workgroup reads the whole
// tensor itself after about a quarter of a second.
constexpr uint32_t kBootSpins = 1u << 20;

// Start of a call: the scale from the window's max; with an empty history,
// from this step's just-in-time amax over the tensor's `units` units
// (slice_amax(beg, end) gives one block's max over units [beg, end)).
template <int FMT, typename SliceAmax>
__device__ __forceinline__ float delayed_begin(fp8_amax_history* h, bool pow2, uint32_t* lds, int64_t units,
                                               SliceAmax slice_amax) {
    const int32_t count = h->count;
    uint32_t basis = 0;
    if (count > 0) {
        const int n = count > 16 ? 16 : count;
        for (int i = 0; i < n; ++i) basis = max(basis, __float_as_uint(h->amax[i]) & 0x7FFFFFFFu);
        return scale_from_amax_bits<FMT>(basis, pow2);
    }
    const uint32_t slices = gridDim.x;
    const int64_t per = (units + slices - 1) / slices;
    for (;;) {
        __syncthreads();
        if (threadIdx.x == 0) lds[8] = atomicAdd(&h->sync[2], 1u);
        __syncthreads();
        const uint32_t sl = lds[8];
        if (sl >= slices) break;
        const int64_t beg = (int64_t)sl * per;
        const int64_t end = beg + per < units ? beg + per : units;
        const uint32_t m = beg < end ? slice_amax(beg, end) : 0u;
        if (threadIdx.x == 0) {
            atomicMax(&h->sync[1], m);
            wait_memory();                       // the max is in place before the slice counts as done
            atomicAdd(&h->sync[0], 1u);
        }
    }
    if (threadIdx.x == 0) {
        uint32_t got = 0;
        for (uint32_t i = 0; i < kBootSpins; ++i) {
            if (sync_read(&h->sync[0]) >= slices) {
                got = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(8);
        }
        lds[9] = got ? sync_read(&h->sync[1]) : 0u;
        lds[10] = got;
    }
    __syncthreads();
    basis = lds[9];
    if (lds[10] == 0u) basis = slice_amax(0, units);
    __syncthreads();
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

// The whole units [beg, end) of a flat tensor that block b streams: one
// contiguous run per block, `chunk` units long (a multiple of the kThreads *
// kUnroll units one iteration covers).  Per-block runs keep each block's
// consecutive loads in the same DRAM pages; measured on 1 GiB, contiguous
// runs read at about 7.0 TB/s for 2 to 16 blocks per CU, where a
// grid-stride loop over the same units falls to 5.2-5.9 TB/s at 4 to 8.
__device__ __forceinline__ void flat_run_of(uint32_t blk, uint32_t whole, uint32_t chunk, uint32_t& beg,
                                            uint32_t& end) {
    const uint64_t b = (uint64_t)blk * chunk, e = b + chunk;
    beg = (uint32_t)(b < whole ? b : whole);
    end = (uint32_t)(e < whole ? e : whole);
}
__device__ __forceinline__ void flat_run(uint32_t whole, uint32_t chunk, uint32_t& beg, uint32_t& end) {
    flat_run_of(blockIdx.x, whole, chunk, beg, end);
}

// The units [it + t, it + t + kThreads, ...) of one loop iteration of a flat
// run ending at `end` (t = threadIdx.x).  A whole iteration, the usual case,
// issues all kUnroll loads with no per-unit test, so they are in flight
// together; with a test per load the compiler waits for each load before
// the next one's branch.  Units past `end` read as zeros.
template <typename InT>
__device__ __forceinline__ void load_iteration(const InT* __restrict__ x, uint32_t it, uint32_t end,
                                               Pack<InT> (&p)[kUnroll]) {
    const uint32_t u0 = it + threadIdx.x;
    if (it + kThreads * kUnroll <= end) {
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) p[i] = load_flat<InT>(x, u0 + i * kThreads);
    } else {
#pragma unroll
        for (int i = 0; i < kUnroll; ++i)
            p[i] = u0 + i * kThreads < end ? load_flat<InT>(x, u0 + i * kThreads) : Pack<InT>{};
    }
}

// Per-tensor amax, pass 1: one partial per block.  FLAT: the tensor is one
// contiguous, 16-byte aligned run of g.cols elements (g.rows == 1, vec_in),
// so every unit but a ragged last one is whole and loads with plain
// indexing, each block streaming its own run of `chunk` units; block 0's
// thread 0 takes the ragged last unit.  Otherwise a grid-stride loop over
// the 2-D geometry.
template <typename InT, bool FLAT>
__global__ __launch_bounds__(kThreads) void k_amax_partials(const InT* __restrict__ x, UnitGeom g,
                                                            uint32_t chunk, bool vec_in,
                                                            uint32_t* __restrict__ partials) {
    __shared__ uint32_t lds[16];
    const uint32_t stride = gridDim.x * kThreads;
    uint32_t m = 0;
    if constexpr (FLAT) {
        const uint32_t whole = (uint32_t)(g.cols / 8);
        uint32_t beg, end;
        flat_run(whole, chunk, beg, end);
        for (uint32_t it = beg; it < end; it += kThreads * kUnroll) {
            Pack<InT> p[kUnroll];
            load_iteration(x, it, end, p);
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
    // The history as it stands before this call's update, one word per
    // thread, read beside the partials' reduction: the ring update then
    // waits for no load of its own (one round trip to memory instead of a
    // chain of them).
    constexpr int kWords = (int)(sizeof(fp8_amax_history) / 4);
    constexpr int kLen = (int)(offsetof(fp8_amax_history, len) / 4);
    constexpr int kPos = (int)(offsetof(fp8_amax_history, pos) / 4);
    constexpr int kCount = (int)(offsetof(fp8_amax_history, count) / 4);
    constexpr int kSteps = (int)(offsetof(fp8_amax_history, steps) / 4);
    constexpr int kThr = (int)(offsetof(fp8_amax_history, spike_threshold) / 4);
    constexpr int kSpikes = (int)(offsetof(fp8_amax_history, spikes) / 4);
    static_assert(kWords <= kThreads && offsetof(fp8_amax_history, amax) == 0, "history layout");
    __shared__ uint32_t hw[kWords];
    uint32_t word = 0;
    if (threadIdx.x < kWords) word = reinterpret_cast<const uint32_t*>(h)[threadIdx.x];
    const uint32_t cur = reduce_partials(partials, n, lds);
    if (threadIdx.x < kWords) hw[threadIdx.x] = word;
    __syncthreads();
    if (threadIdx.x != 0) return;
    const float amax_now = __uint_as_float(cur);
    amax_out[0] = amax_now;
    int32_t len = (int32_t)hw[kLen];
    len = len < 1 ? 1 : (len > 16 ? 16 : len);
    int32_t pos = (int32_t)hw[kPos];
    pos = (pos < 0 || pos >= len) ? 0 : pos;
    const int32_t count_in = (int32_t)hw[kCount];
    if constexpr (GUARD) {
        const int32_t count0 = count_in < 0 ? 0 : (count_in > len ? len : count_in);
        uint32_t wbits = 0;
        for (int i = 0; i < count0; ++i) wbits = max(wbits, hw[i] & 0x7FFFFFFFu);
        const float thr = __uint_as_float(hw[kThr]);
        const bool spiked = count0 > 0 && thr > 0.0f && amax_now > thr * __uint_as_float(wbits);
        h->internal[0] = spiked ? 1u : 0u;
        if (spiked) {
            const float sj = scale_from_amax_bits<FMT>(cur, pow2);
            h->internal[1] = __float_as_uint(sj);
            scale_inv_out[0] = recip_rn(sj);
            h->spikes = hw[kSpikes] + 1u;
        }
        if (diag_tmp != nullptr && !spiked && diag != nullptr) {
            diag->sat_count += diag_tmp->sat_count;
            diag->nonfinite_count += diag_tmp->nonfinite_count;
            diag->underflow_count += diag_tmp->underflow_count;
        }
    }
    h->amax[pos] = amax_now;
    h->pos = (pos + 1) % len;
    const int32_t count = count_in < len ? count_in + 1 : len;
    h->count = count;
    // the window after this step's entry: slot pos now holds amax_now
    uint32_t basis = 0;
    for (int i = 0; i < count; ++i) basis = max(basis, (i == pos ? cur : hw[i]) & 0x7FFFFFFFu);
    const float s = scale_from_amax_bits<FMT>(basis, pow2);
    h->scale = s;
    h->scale_inv = 1.0f / s;
    h->steps = hw[kSteps] + 1u;
    for (int i = 0; i < 3; ++i) h->sync[i] = 0u;
}

// Per-tensor cast.  JIT: s from the amax partials of pass 1 (block 0 also
// writes amax_out).  DELAYED: s from the history (delayed_begin); each
// block stores its own amax partial for the finish kernel.  RECAST: s
// recorded by a guarded finish kernel, or nothing to do.
template <typename InT, int FMT, int MODE, bool DIAG, bool FLAT>
__global__ __launch_bounds__(kThreads) void k_cast_tensor(
    const InT* __restrict__ x, UnitGeom g, uint32_t chunk, bool vec_in, uint8_t* __restrict__ q, bool vec_out,
    const uint32_t* __restrict__ partials_in, int n_in, fp8_amax_history* hist, bool pow2,
    float* __restrict__ scale_inv_out, float* __restrict__ amax_out, fp8_diag* diag,
    uint32_t* __restrict__ partials_out) {
    __shared__ uint32_t lds[16];
    constexpr bool DELAYED = MODE == kModeDelayed;
    float s;
    if constexpr (MODE == kModeRecast) {
        if (hist->internal[0] == 0u) return;
        s = __uint_as_float(hist->internal[1]);
    } else if constexpr (DELAYED) {
        s = delayed_begin<FMT>(hist, pow2, lds, (int64_t)g.units, [&](int64_t b, int64_t e) {
            return units_amax<InT>(x, g.rows, g.cols, g.ld, vec_in, b, e, lds);
        });
    } else {
        const uint32_t am = reduce_partials(partials_in, n_in, lds);
        s = scale_from_amax_bits<FMT>(am, pow2);
        if (blockIdx.x == 0 && threadIdx.x == 0) amax_out[0] = __uint_as_float(am);
    }
    if (MODE != kModeRecast && blockIdx.x == 0 && threadIdx.x == 0) scale_inv_out[0] = recip_rn(s);

    const uint32_t stride = gridDim.x * kThreads;
    uint32_t m = 0;
    Counters cnt;
    if constexpr (FLAT) {     // contiguous input and codes: this block's run of whole units, then the ragged last one
        const uint32_t whole = (uint32_t)(g.cols / 8);
        uint32_t beg, end;
        flat_run(whole, chunk, beg, end);
        for (uint32_t it = beg; it < end; it += kThreads * kUnroll) {
            Pack<InT> p[kUnroll];
            load_iteration(x, it, end, p);
#pragma unroll
            for (int i = 0; i < kUnroll; ++i) {
                const uint32_t u = it + threadIdx.x + i * kThreads;
                if (u < end) {
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

// Several contiguous tensors quantized just in time, each with its own
// per-tensor scale, in one amax launch and one cast launch.  Each tensor
// owns a run of consecutive blocks in both grids (first[t] .. first[t+1]),
// at least one even when empty, and each of its blocks streams `chunk`
// whole units of it exactly as the single-tensor flat kernels do; the
// tensor's first block takes its ragged last unit.  The amax pass leaves
// one partial per block; a cast block reduces its own tensor's partials.
struct MultiSet {
    const void* x[kMultiMax];
    uint8_t* q[kMultiMax];
    float* scale_inv[kMultiMax];
    float* amax[kMultiMax];
    fp8_diag* diag[kMultiMax];
    uint32_t whole[kMultiMax];          // whole 8-element units
    uint32_t tail[kMultiMax];           // elements of a ragged last unit, 0..7
    uint32_t afirst[kMultiMax + 1];     // first amax-pass block of each tensor; afirst[n] = grid
    uint32_t cfirst[kMultiMax + 1];     // first cast-pass block of each tensor; cfirst[n] = grid
    uint32_t achunk, cchunk;
    int n;
};

// The tensor whose block run holds block b (runs are non-empty and in order).
__device__ __forceinline__ int multi_tensor_of(const uint32_t* first, int n, uint32_t b) {
    int t = 0;
    for (int i = 1; i < n; ++i) t += b >= first[i] ? 1 : 0;
    return t;
}

template <typename InT>
__global__ __launch_bounds__(kThreads) void k_amax_multi(MultiSet ms, uint32_t* __restrict__ partials) {
    __shared__ uint32_t lds[16];
    const int t = multi_tensor_of(ms.afirst, ms.n, blockIdx.x);
    const uint32_t blk = blockIdx.x - ms.afirst[t];
    const InT* __restrict__ x = static_cast<const InT*>(ms.x[t]);
    const uint32_t whole = ms.whole[t];
    uint32_t beg, end;
    flat_run_of(blk, whole, ms.achunk, beg, end);
    uint32_t m = 0;
    for (uint32_t it = beg; it < end; it += kThreads * kUnroll) {
        Pack<InT> p[kUnroll];
        load_iteration(x, it, end, p);
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) m = max(m, p[i].abs_max());
    }
    if (blk == 0 && threadIdx.x == 0 && ms.tail[t] != 0)
        m = max(m, load_unit<InT>(x, (int64_t)whole * 8, (int)ms.tail[t], false).abs_max());
    const uint32_t bm = block_max(m, lds);
    if (threadIdx.x == 0) partials[blockIdx.x] = bm;
}

template <typename InT, int FMT, bool DIAG>
__global__ __launch_bounds__(kThreads) void k_cast_multi(MultiSet ms, const uint32_t* __restrict__ partials,
                                                         bool pow2) {
    __shared__ uint32_t lds[16];
    const int t = multi_tensor_of(ms.cfirst, ms.n, blockIdx.x);
    const uint32_t blk = blockIdx.x - ms.cfirst[t];
    const uint32_t am = reduce_partials(partials + ms.afirst[t], (int)(ms.afirst[t + 1] - ms.afirst[t]), lds);
    const float s = scale_from_amax_bits<FMT>(am, pow2);
    if (blk == 0 && threadIdx.x == 0) {
        ms.amax[t][0] = __uint_as_float(am);
        ms.scale_inv[t][0] = recip_rn(s);
    }
    const InT* __restrict__ x = static_cast<const InT*>(ms.x[t]);
    uint8_t* __restrict__ q = ms.q[t];
    const uint32_t whole = ms.whole[t];
    uint32_t beg, end;
    flat_run_of(blk, whole, ms.cchunk, beg, end);
    Counters cnt;
    for (uint32_t it = beg; it < end; it += kThreads * kUnroll) {
        Pack<InT> p[kUnroll];
        load_iteration(x, it, end, p);
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const uint32_t u = it + threadIdx.x + i * kThreads;
            if (u < end) store_flat(q, u, encode_unit<FMT, DIAG>(p[i], s, cnt));
        }
    }
    if (blk == 0 && threadIdx.x == 0 && ms.tail[t] != 0) {
        const int64_t off = (int64_t)whole * 8;
        const int nv = (int)ms.tail[t];
        store_unit(q, off, nv, false, encode_unit<FMT, DIAG>(load_unit<InT>(x, off, nv, false), s, cnt));
    }
    if constexpr (DIAG) {
        if (ms.diag[t] != nullptr) block_add_diag(cnt, lds, ms.diag[t]);
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
__global__ __launch_bounds__(kThreads, kTBlocksPerCU) void k_cast_tensor_t(
    const InT* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, bool vec_in,
    uint8_t* __restrict__ q, int64_t ldq, bool vec_out16, const uint32_t* __restrict__ partials_in,
    int n_in, fp8_amax_history* hist, bool pow2, float* __restrict__ scale_inv_out,
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
        s = delayed_begin<FMT>(hist, pow2, lds, rows * ((cols + 7) / 8), [&](int64_t b, int64_t e) {
            return units_amax<InT>(x, rows, cols, ld, vec_in, b, e, lds);
        });
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
    // this thread's 8 units of tile tl (zeros past the matrix).  An interior
    // tile of an aligned matrix issues its 8 loads with no per-unit test, so
    // they are in flight together (the ragged path's 2-byte loads would
    // otherwise make the compiler wait before each vector load).
    Pack<InT> p[8];
    auto load_tile = [&](int64_t tl) {
        const int64_t r0 = (tl / tiles_c) * 128, c = (tl % tiles_c) * 128 + cu * 8;
        if (vec_in && r0 + 128 <= rows && (tl % tiles_c) * 128 + 128 <= cols) {
#pragma unroll
            for (int i = 0; i < 8; ++i) p[i] = load_unit<InT, true>(x, (r0 + rr + 16 * i) * ld + c, 8, true);
            return;
        }
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
            if constexpr (DELAYED) {
                m = max(m, p[i].abs_max());
                // keep the running max (and counters) here: left free, the
                // compiler sinks these reductions past the next tile's loads
                // and holds two tiles of input (158 VGPRs instead of 94)
                asm volatile("" : "+v"(m));
            }
            const uint2 codes = encode_unit<FMT, DIAG>(p[i], s, cnt);
            if constexpr (DIAG) asm volatile("" : "+v"(cnt.sat), "+v"(cnt.nonfinite), "+v"(cnt.under));
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
// (Contiguous row ranges per wave measured slower: qkv 0.048 against 0.044
// ms, moe 0.026 against 0.023.)
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

// 1x128 blocks: 16 lanes per block of 128 elements, kUnroll blocks per lane
// in flight.  Workgroup b takes the contiguous run of groups [b * C,
// (b + 1) * C) (row-major group order, C a multiple of the 64 groups one
// iteration covers), so that it streams one run of memory.  amax/scale
// arrays are [rows x ceil(cols/128)].
template <typename InT, int FMT, bool DIAG, bool WRITE_Q>
__global__ __launch_bounds__(kThreads) void k_cast_1x128(
    const InT* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, bool vec_in,
    uint8_t* __restrict__ q, int64_t ldq, bool vec_out, bool pow2,
    float* __restrict__ scale_inv_out, float* __restrict__ amax_out, fp8_diag* diag) {
    __shared__ uint32_t lds[16];
    const int64_t gc = (cols + 127) / 128;
    const int64_t G = rows * gc;
    const int slot = threadIdx.x >> 4, j = threadIdx.x & 15;
    constexpr int64_t kStep = 16 * kUnroll;
    const int64_t C = ((G + gridDim.x - 1) / gridDim.x + kStep - 1) / kStep * kStep;
    const int64_t beg = (int64_t)blockIdx.x * C;
    const int64_t end = beg + C < G ? beg + C : G;
    Counters cnt;
    for (int64_t base = beg; base < end; base += kStep) {
        Pack<InT> p[kUnroll];
        uint32_t m[kUnroll];
        int nv[kUnroll];
        int64_t xo[kUnroll], qo[kUnroll];
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int64_t g = base + i * 16 + slot;
            m[i] = 0; nv[i] = 0; xo[i] = 0; qo[i] = 0;
            if (g < end) {
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
            const int64_t g = base + i * 16 + slot;
            if (g < end) {
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

// 1x128 blocks of a contiguous, aligned tensor whose rows are whole blocks
// (cols % 128 == 0, codes contiguous too): unit u (8 elements) lies in block
// u / 16, so the flat unit order is the block order and no row arithmetic
// is needed.  Each workgroup streams one contiguous run of whole blocks
// (kThreads * kUnroll units per iteration); 16 consecutive lanes hold one
// block, whose max is a DPP reduction inside their 16-lane row.
template <typename InT, int FMT, bool DIAG, bool WRITE_Q>
__global__ __launch_bounds__(kThreads) void k_cast_1x128_flat(
    const InT* __restrict__ x, uint32_t units, uint32_t chunk, uint8_t* __restrict__ q, bool pow2,
    float* __restrict__ scale_inv_out, float* __restrict__ amax_out, fp8_diag* diag) {
    __shared__ uint32_t lds[16];
    uint32_t beg, end;
    flat_run(units, chunk, beg, end);
    Counters cnt;
    // runs, ends and iterations are multiples of 16 units, so the 16 lanes of
    // a block are active or idle together
    for (uint32_t it = beg; it < end; it += kThreads * kUnroll) {
        const uint32_t u0 = it + threadIdx.x;
        Pack<InT> p[kUnroll];
        load_iteration(x, it, end, p);
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const uint32_t u = u0 + i * kThreads;
            const uint32_t gm = group_max_u32<16>(p[i].abs_max());
            const float s = scale_from_amax_bits<FMT>(gm, pow2);
            const float si = recip_rn(s);
            if (u < end) {
                if ((threadIdx.x & 15) == 0) {
                    amax_out[u >> 4] = __uint_as_float(gm);
                    if (WRITE_Q) scale_inv_out[u >> 4] = si;
                }
                if constexpr (WRITE_Q) store_flat(q, u, encode_unit<FMT, DIAG>(p[i], s, cnt));
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

// Workspace layout (uint32 words of the caller's workspace, kScratchWords).
constexpr int kScratchCastPartials = 0;      // <= kMaxCastBlocks partials of a delayed cast
constexpr int kScratchAmaxPartials = 4096;   // <= kMaxAmaxBlocks partials of pass 1
constexpr int kScratchDiag = 8192;           // fp8_diag of a guarded delayed cast's first pass
constexpr int64_t kMaxCastBlocks = 4096;
constexpr int64_t kMaxAmaxBlocks = 1024;   // a stream needs about 4 workgroups per CU (measured)
static_assert(kScratchAmaxPartials + kMaxAmaxBlocks <= kScratchDiag, "scratch layout");
static_assert(kScratchDiag + 4 <= kScratchGroupTable, "scratch layout: the grouped GEMM's table follows");

constexpr int64_t kRowBlocksPerCU = 3;   // measured: 2, 3 and 4 per CU, 3 fastest

inline unsigned grid_for(int64_t work_items, int64_t per_block, int64_t cap) {
    int64_t b = (work_items + per_block - 1) / per_block;
    if (b < 1) b = 1;
    if (b > cap) b = cap;
    return (unsigned)b;
}

// Blocks for a flat pass over `whole` units with at most `cap` blocks: each
// block's run (*chunk units) is a whole number of loop iterations, so the
// runs start on 16 KiB boundaries (bf16) of a 16-byte aligned tensor.
inline unsigned flat_grid(int64_t whole, int64_t cap, uint32_t* chunk) {
    const int64_t step = (int64_t)kThreads * kUnroll;
    int64_t per = (whole + cap - 1) / cap;
    per = std::max<int64_t>(step, (per + step - 1) / step * step);
    *chunk = (uint32_t)per;
    return (unsigned)std::max<int64_t>(1, (whole + per - 1) / per);
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
    // delayed casts keep one partial per block in the workspace: at most kMaxCastBlocks
    const unsigned cap = (unsigned)std::min<int64_t>((int64_t)a.num_cus * 8, kMaxCastBlocks);
    hipStream_t st = a.stream;

    if (a.gran == FP8_GRAN_TENSOR) {
        uint32_t* amax_partials = a.scratch + kScratchAmaxPartials;
        uint32_t* cast_partials = a.scratch + kScratchCastPartials;
        const bool delayed = a.hist != nullptr;
        // contiguous, aligned input (and codes): the kernels' plain-indexed fast path
        const bool flat_in = g.rows == 1 && vec_in;
        const bool flat = flat_in && vec_out;
        // flat passes: each block streams one run of whole units
        uint32_t achunk = 0, cchunk = 0;
        const unsigned agrid = flat_in ? flat_grid(g.cols / 8, kMaxAmaxBlocks, &achunk)
                                       : grid_for(g.units, (int64_t)kThreads * kUnroll, kMaxAmaxBlocks);
        const unsigned cgrid = flat ? flat_grid(g.cols / 8, cap, &cchunk)
                                    : grid_for(g.units, (int64_t)kThreads * kUnroll, cap);
        const int64_t tiles = ((a.rows + 127) / 128) * ((a.cols + 127) / 128);
        const unsigned tgrid =
            grid_for(tiles, 1, std::min<int64_t>(kMaxCastBlocks, (int64_t)a.num_cus * kTBlocksPerCU));
        const bool v16 = a.q != nullptr && aligned(a.q, 16) && a.ldq % 16 == 0;
        const bool v2 = a.q2 != nullptr && aligned(a.q2, 8) && a.ldq2 % 8 == 0;
#define FP8MI_TENSOR_CAST(MODE, DG, DIAGP)                                                                  \
    do {                                                                                                  \
        if (a.transpose)                                                                                  \
            hipLaunchKernelGGL((k_cast_tensor_t<InT, FMT, MODE, DG>), dim3(tgrid), dim3(kThreads), 0, st, x,    \
                               a.rows, a.cols, a.ld, vec_in, a.q, a.ldq, v16,                             \
                               (const uint32_t*)amax_partials, (int)agrid, a.hist, a.pow2, a.scale_inv,   \
                               a.amax, DIAGP, cast_partials, a.q2, a.ldq2, v2);                           \
        else if (flat)                                                                                    \
            hipLaunchKernelGGL((k_cast_tensor<InT, FMT, MODE, DG, true>), dim3(cgrid), dim3(kThreads), 0, st, x,\
                               g, cchunk, vec_in, a.q, vec_out, (const uint32_t*)amax_partials, (int)agrid,\
                               a.hist, a.pow2, a.scale_inv, a.amax, DIAGP, cast_partials);               \
        else                                                                                              \
            hipLaunchKernelGGL((k_cast_tensor<InT, FMT, MODE, DG, false>), dim3(cgrid), dim3(kThreads), 0, st,  \
                               x, g, 0u, vec_in, a.q, vec_out, (const uint32_t*)amax_partials, (int)agrid,\
                               a.hist, a.pow2, a.scale_inv, a.amax, DIAGP, cast_partials);               \
    } while (0)
        if (delayed) {
            // the cast (its scale from the history, or from its own
            // bootstrap while the history is empty), then the one-block
            // finish that pushes the ring.  With the guard, the cast's
            // diagnostics wait in the workspace (cleared first: its contents
            // are arbitrary), and a re-cast follows that does nothing unless
            // the finish saw a spike.
            fp8_diag* diag_tmp = a.guard ? reinterpret_cast<fp8_diag*>(a.scratch + kScratchDiag) : nullptr;
            fp8_diag* d1 = a.guard ? diag_tmp : a.diag;
            if (a.guard && diag)
                hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(64), 0, st, a.scratch + kScratchDiag, 4);
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
            return hipGetLastError();
        }
        // just in time: pass 1, the amax partials
        if (flat_in)
            hipLaunchKernelGGL((k_amax_partials<InT, true>), dim3(agrid), dim3(kThreads), 0, st, x, g, achunk,
                               vec_in, amax_partials);
        else
            hipLaunchKernelGGL((k_amax_partials<InT, false>), dim3(agrid), dim3(kThreads), 0, st, x, g, 0u,
                               vec_in, amax_partials);
        if (!a.write_q) {
            hipLaunchKernelGGL(k_reduce_amax, dim3(1), dim3(kThreads), 0, st, (const uint32_t*)amax_partials,
                               (int)agrid, a.amax);
            return hipGetLastError();
        }
        if (diag) FP8MI_TENSOR_CAST(kModeJit, true, a.diag);
        else FP8MI_TENSOR_CAST(kModeJit, false, a.diag);
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
        const int64_t units = a.rows * a.cols / 8;
        const bool flat = a.cols % 128 == 0 && a.ld == a.cols && (!a.write_q || a.ldq == a.cols) && gvec_in &&
                          (!a.write_q || aligned(a.q, 8)) && units < ((int64_t)1 << 31);
        if (flat) {
            uint32_t chunk = 0;
            const dim3 grid(flat_grid(units, (int64_t)a.num_cus * 8, &chunk));
#define FP8MI_1x128_FLAT(DG, WQ)                                                                          \
    hipLaunchKernelGGL((k_cast_1x128_flat<InT, FMT, DG, WQ>), grid, dim3(kThreads), 0, st, x, (uint32_t)units, \
                       chunk, a.q, a.pow2, a.scale_inv, a.amax, a.diag)
            if (!a.write_q) FP8MI_1x128_FLAT(false, false);
            else if (diag) FP8MI_1x128_FLAT(true, true);
            else FP8MI_1x128_FLAT(false, true);
#undef FP8MI_1x128_FLAT
        } else {
            const dim3 grid(grid_for(G, 16 * kUnroll, (int64_t)a.num_cus * 8));
            FP8MI_GROUP_LAUNCH(k_cast_1x128, grid);
        }
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

// Grids of fp8_quantize_tensors: one chunk length per pass for all tensors
// (the single-tensor flat grid's, taken over the tensors' total units), so
// every block but a tensor's last streams the same number of units, and
// each tensor gets the blocks its units need (at least one).
template <typename InT, int FMT>
hipError_t quantize_multi_typed(const MultiQuantArgs& a) {
    MultiSet ms = {};
    ms.n = a.n;
    int64_t total = 0;
    for (int t = 0; t < a.n; ++t) {
        ms.x[t] = a.x[t];
        ms.q[t] = a.q[t];
        ms.scale_inv[t] = a.scale_inv[t];
        ms.amax[t] = a.amax[t];
        ms.diag[t] = a.diag[t];
        ms.whole[t] = (uint32_t)(a.elems[t] / 8);
        ms.tail[t] = (uint32_t)(a.elems[t] % 8);
        total += a.elems[t] / 8;
    }
    const unsigned cap = (unsigned)std::min<int64_t>((int64_t)a.num_cus * 8, kMaxCastBlocks);
    flat_grid(total, kMaxAmaxBlocks, &ms.achunk);
    flat_grid(total, cap, &ms.cchunk);
    ms.afirst[0] = ms.cfirst[0] = 0;
    for (int t = 0; t < a.n; ++t) {
        const uint32_t w = ms.whole[t];
        ms.afirst[t + 1] = ms.afirst[t] + std::max<uint32_t>(1u, (w + ms.achunk - 1) / ms.achunk);
        ms.cfirst[t + 1] = ms.cfirst[t] + std::max<uint32_t>(1u, (w + ms.cchunk - 1) / ms.cchunk);
    }
    // at most kMaxAmaxBlocks + kMultiMax partials: inside the workspace's partials region
    static_assert(kMaxAmaxBlocks + kMultiMax <= kScratchDiag - kScratchAmaxPartials, "scratch layout");
    uint32_t* partials = a.scratch + kScratchAmaxPartials;
    hipStream_t st = a.stream;
    hipLaunchKernelGGL((k_amax_multi<InT>), dim3(ms.afirst[a.n]), dim3(kThreads), 0, st, ms, partials);
    bool diag = false;
    for (int t = 0; t < a.n; ++t) diag = diag || a.diag[t] != nullptr;
    if (diag)
        hipLaunchKernelGGL((k_cast_multi<InT, FMT, true>), dim3(ms.cfirst[a.n]), dim3(kThreads), 0, st, ms,
                           (const uint32_t*)partials, a.pow2);
    else
        hipLaunchKernelGGL((k_cast_multi<InT, FMT, false>), dim3(ms.cfirst[a.n]), dim3(kThreads), 0, st, ms,
                           (const uint32_t*)partials, a.pow2);
    return hipGetLastError();
}

hipError_t launch_quantize_multi(const MultiQuantArgs& a) {
    if (a.in_bf16) {
        return a.fmt == 0 ? quantize_multi_typed<uint16_t, kE4M3>(a) : quantize_multi_typed<uint16_t, kE5M2>(a);
    }
    return a.fmt == 0 ? quantize_multi_typed<float, kE4M3>(a) : quantize_multi_typed<float, kE5M2>(a);
}

// The workspace of fp8_quantize_noalloc: 64 KiB of device memory in the
// library's own code object, one copy per device, held until the process
// ends.  Every call on a device shares that device's copy.  In host code the
// array's name is not a device address; its address on the current device
// comes from hipGetSymbolAddress, taken once per device.
static __device__ __align__(256) uint32_t scratch[kScratchWords];

hipError_t static_workspace(uint32_t** out) {
    constexpr int kDevices = 64;
    static std::once_flag once[kDevices];
    static uint32_t* ptr[kDevices] = {};
    static hipError_t err[kDevices] = {};
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
    std::call_once(once[dev], [&] {
        void* p = nullptr;
        err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err[dev] == hipSuccess && p == nullptr) err[dev] = hipErrorInvalidSymbol;
        ptr[dev] = static_cast<uint32_t*>(p);
    });
    *out = ptr[dev];
    return err[dev];
}

hipError_t launch_history_init(fp8_amax_history* h, int32_t len, hipStream_t stream) {
    hipLaunchKernelGGL(k_history_init, dim3(1), dim3(64), 0, stream, h, len);
    return hipGetLastError();
}

hipError_t launch_history_set_guard(fp8_amax_history* h, float threshold, hipStream_t stream) {
    hipLaunchKernelGGL(k_history_set_guard, dim3(1), dim3(64), 0, stream, h, threshold);
    return hipGetLastError();
}

}  // namespace fp8mi
