// gemm.hip -- scaled FP8 x FP8 GEMM on gfx950 matrix cores (MFMA), fp32
// accumulation, dequantizing fp32/bf16 epilogue; and the block-scaled
// variant that promotes each 128-wide K block's partial sum with its scale.
//
// Method: [H100 FP8 acceleration, measured, scrxy.com] FP8 matrix
// multiply-add directly in hardware; [Soup, lbrq.cn] tensorwise (one scale
// per operand) and rowwise GEMMs; [DeepL bets on FP8, hmyw.cn] 2.3 per-block
// scaling, 2.2 the result returns to high precision, 5.3 results are not
// bit-identical across tilings (this kernel is bit-reproducible run to run:
// no split-K, no atomics).
//
// Computes C[m,n] = (sum_k dec(A[m,k]) dec(B[n,k])) * fl32(sa(m) sb(n)) with
// A [M x K] and B [N x K] both K-contiguous (Y = X W^T).
//
// Design for CDNA4 (gfx950):
//   * v_mfma_f32_32x32x64_f8f6f4 (E4M3/E5M2 chosen per operand).  Four waves
//     as a 2x2 grid over a BM x BN block tile; each wave owns (BM/2) x (BN/2)
//     in 32x32 MFMA blocks.  B is the instruction's first operand, so a lane
//     ends up holding 4 consecutive output columns of one output row (one
//     row scale per lane).  The epilogue stages the scaled, converted tile
//     in LDS and stores full 256-byte row segments, 16 bytes per lane.
//   * Operands reach LDS by buffer-load-to-LDS DMA (no staging registers)
//     issued from inline asm (it has no register results), so the compiler
//     neither tracks nor waits for it: explicit s_waitcnt vmcnt(N) plus
//     s_barrier is the only ordering, and the asm's memory clobber keeps
//     every LDS read below it.  Operand fragments are double-buffered in
//     registers so the LDS reads of the next step overlap the MFMAs.
//   * The scaled GEMM (k_gemm_p, 256 x 256 tiles) moves K in stages of 128
//     bytes, so that 8 lanes of a DMA instruction read one whole 128-byte
//     line per row (measured: 64-byte row pieces cost about twice the
//     vector-memory time), through a ring of five 32 KiB slots: A two stages
//     ahead, B one stage ahead, one barrier per stage.  It is persistent
//     (one block per CU when tiles outnumber CUs): the next tile's first
//     stages stream in during the current tile's last ones, and the
//     epilogue's stores overlap the next tile's first stage.
//   * A round of tiles that would leave CUs idle (a persistent launch's
//     last round, a small problem, a grouped GEMM's leftover tiles) runs on
//     128- or 64-row tiles of the same MFMA program, so every output is the
//     same chain of MFMAs whatever tile computes it.
//   * The block-scaled GEMM (k_gemm_bq, 256 x 256 tiles, eight waves) moves
//     K in stages of 128 bytes, one stage per 128-wide scale block, through
//     two buffers that carry the block's A-row scales too; the promotion of
//     a block's partial sum by one wave runs beside the MFMAs of the other
//     wave on its SIMD.
//   * LDS rows carry an XOR swizzle of their 16-byte chunks that makes the
//     32-rows-by-16-bytes fragment reads conflict free.  The swizzle is
//     applied by choosing which global chunk each DMA lane fetches.
//   * Ragged M/N and a K tail are zero-filled by the buffer unit itself: the
//     lanes that fall outside get an out-of-range offset and return zeros.
//   * blockIdx -> tile mapping keeps each XCD (blocks are dealt round robin
//     over 8 XCDs) on a contiguous, M-grouped range of tiles so that
//     concurrently running tiles share A and B panels in that XCD's L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kGemmThreads = 256;
constexpr uint32_t kOOB = 0x80000000u; // offset past every descriptor's range

extern __shared__ __attribute__((aligned(1024))) uint8_t g_ring[];

struct GemmParams {
    const uint8_t* A;
    const uint8_t* B;
    int64_t lda, ldb;
    int M, N, K;
    const float* sa;
    const float* sb;
    int sa_row, sb_row;
    void* C;
    int64_t ldc;
    int tiles_m, tiles_n;
    int group_m;
    int vec_out;          // C rows allow 16-byte vector stores
    // grouped GEMM: tile table (header, then one entry per 256-row tile of a
    // group: expert, first row, end row of the group) and expert stride of B
    const int4* gtab;
    int64_t b_gstride;
    int main_grid;        // grouped: the persistent grid, when k_gemm_h takes a last round split off (else 0)
    // plain persistent launch: the problem's full N when columns [N, tail_N)
    // run as 128-row half tiles after the whole rounds of columns [0, N)
    // (else 0)
    int tail_N;
};

template <int FX, int FY>
__device__ __forceinline__ v16f mfma32(const v8i& x, const v8i& y, const v16f& c) {
    // cbsz / blgp select the operand formats: 0 = E4M3, 1 = E5M2.  Zero scale
    // operands select the unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, FX, FY, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const LDS_AS void*)p;
}

// Buffer descriptor over `bytes` bytes from `base` (raw, gfx9 data format),
// made wave-uniform so that it lives in SGPRs.
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// 64 lanes x 16 bytes from rsrc + voff[lane] + soff into LDS [lds, lds + 1024).
// No register result: nothing in flight targets a VGPR.  A lane whose voff
// is past the descriptor's range reads zeros whatever soff is.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, v4i rsrc, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                    "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}

// 64 lanes x 4 bytes into LDS [lds, lds + 256).
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, v4i rsrc) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc) : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are in
// flight, then meet the other waves; also a compiler barrier for memory.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// blockIdx -> (tile_m, tile_n)
__device__ __forceinline__ void tile_coords(const GemmParams& p, int& tm, int& tn) {
    int bid = blockIdx.x;
    const int nb = gridDim.x;
    if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);   // XCD-contiguous ranges
    const int per_group = p.group_m * p.tiles_n;
    const int group = bid / per_group;
    const int first_m = group * p.group_m;
    const int gsize = min(p.tiles_m - first_m, p.group_m);
    const int in_group = bid - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

template <int BM, int BN>
struct Frags {
    v8i a[BM / 64];
    v8i b[BN / 64];
};

__device__ __forceinline__ void set_half(v8i& f, int h, uint4 v) {
    f[4 * h + 0] = (int)v.x; f[4 * h + 1] = (int)v.y; f[4 * h + 2] = (int)v.z; f[4 * h + 3] = (int)v.w;
}

// ------------------------------------------------------------------------
// Scaled GEMM with 128-byte K stages (256 x 256 tiles).
//
// A stage holds K = 128 bytes of every A and B row of the tile, so each DMA
// lane group reads whole 128-byte lines (8 lanes per row).  The A rows of
// stage s live in ring slot (2s) mod 5 and the B rows in slot (2s+1) mod 5
// (slots of 32 KiB).  A stage is consumed in two MFMA steps of K = 64:
//   even step 2s:   MFMAs of step 2s; LDS reads of step 2s+1 (stage s,
//                   second half); DMA of A(s+2) into B(s-1)'s slot;
//   odd step 2s+1:  after the first MFMA, s_waitcnt for A(s+1), B(s+1)
//                   (only A(s+2) may still be in flight) and for this wave's
//                   LDS reads, then s_barrier: stage s+1 is in LDS and every
//                   wave is done reading stage s; then the LDS reads of step
//                   2s+2 (stage s+1, first half) and the DMA of B(s+2) into
//                   A(s)'s slot.
// So A runs two stages ahead and B one, with one barrier per 128 K.
// ------------------------------------------------------------------------
constexpr int kBK2 = 128;                 // K bytes per stage
constexpr int kSlot2 = 256 * kBK2;        // one operand of one stage: 32 KiB

// 16-byte chunk swizzle of 128-byte LDS rows.  A ds_read_b128 serves 16
// lanes per LDS cycle; lanes 0-15 read 16 consecutive rows at one logical
// chunk, whose 16 bank quads (8 * (row & 1) + physical chunk) are distinct
// under this XOR.
__device__ __forceinline__ int swz2(int row) { return (row >> 1) & 7; }

// DMA plan of one operand for one stage (ROWS rows x 128 bytes) filled by
// WAVES waves: wave w fills rows [w*ROWS/WAVES, (w+1)*ROWS/WAVES) with
// ROWS/(8*WAVES) instructions of 8 rows; lane l of instruction i lands at
// LDS row (w*ROWS/WAVES + 8i + l/8), physical chunk l%8, and fetches the
// logical chunk (l%8) ^ swz2(row).  The swizzle depends on the row only
// through (8i + l/8) bits 1..3 (ROWS/WAVES is a multiple of 16), i.e. on
// the parity of i, so the per-lane offset of instruction i is
// base[i & 1] + 8i * ld.  The descriptor covers exactly the tile's valid
// rows, so a row past them is out of range and reads zeros.
template <int ROWS, int WAVES = 4>
struct DmaL {
    static constexpr int kWaveRows = ROWS / WAVES;
    static constexpr int kInst = kWaveRows / 8;
    static_assert(kWaveRows % 16 == 0, "a wave's rows keep the swizzle's parity rule");
    v4i rsrc;
    uint32_t base[2];      // byte offset of instruction 0 / 1 at k = 0, minus 8 * ld for 1
    uint32_t ld8;          // 8 * ld (wave-uniform)
    uint32_t lds0;         // LDS offset of this wave's first row within a slot

    // logical byte column of this lane's chunk in instruction i
    __device__ __forceinline__ static int col_of(int i) {
        const int lane = threadIdx.x & 63;
        return ((lane & 7) ^ (((8 * i + (lane >> 3)) >> 1) & 7)) * 16;
    }
    __device__ __forceinline__ uint32_t off(int i) const { return base[i & 1] + (uint32_t)i * ld8; }

    __device__ __forceinline__ void init(const uint8_t* base_ptr, int64_t ld, int row0, int rows_valid, int wave) {
        const int lane = threadIdx.x & 63;
        const int rows_here = max(0, min(ROWS, rows_valid - row0));
        rsrc = make_rsrc(base_ptr + (int64_t)row0 * ld, (uint32_t)((int64_t)rows_here * ld));
        lds0 = (uint32_t)(wave * kWaveRows * kBK2);
        ld8 = (uint32_t)(8 * ld);
        const uint32_t r0 = (uint32_t)((wave * kWaveRows + (lane >> 3)) * ld);
        base[0] = r0 + (uint32_t)col_of(0);
        base[1] = r0 + (uint32_t)col_of(1);
    }
    __device__ __forceinline__ void issue_full(uint32_t slot, int k0, int i) const {
        dma16(slot + lds0 + (uint32_t)(8 * i * kBK2), off(i), rsrc, (uint32_t)k0);
    }
    // issue_full with the lane's offset formed here from an opaque copy of
    // its base, so that the compiler keeps two base registers live instead of
    // one precomputed offset per instruction.  Every DMA of the GEMM kernels
    // goes through it: precomputed offsets are spilled across the epilogue,
    // and each reload's wait (vector-memory operations complete in issue
    // order) would also wait for the tile's stores of C and the DMA in flight.
    __device__ __forceinline__ void issue_full_lean(uint32_t slot, int k0, int i) const {
        uint32_t b = base[i & 1];
        asm volatile("" : "+v"(b));
        dma16(slot + lds0 + (uint32_t)(8 * i * kBK2), b + (uint32_t)i * ld8, rsrc, (uint32_t)k0);
    }
    __device__ __forceinline__ void issue_checked(uint32_t slot, int k0, int K, int i) const {
        uint32_t b = base[i & 1];
        asm volatile("" : "+v"(b));
        const uint32_t o = (k0 + col_of(i) < K) ? b + (uint32_t)i * ld8 + (uint32_t)k0 : kOOB;
        dma16(slot + lds0 + (uint32_t)(8 * i * kBK2), o, rsrc, 0u);
    }
    __device__ __forceinline__ void issue(uint32_t slot, int k0, int K) const {
        if (k0 + kBK2 <= K) {
#pragma unroll
            for (int i = 0; i < kInst; ++i) issue_full_lean(slot, k0, i);
        } else {
#pragma unroll
            for (int i = 0; i < kInst; ++i) issue_checked(slot, k0, K, i);
        }
    }
};
using Dma2 = DmaL<256>;

// The DMA instructions of one operand of one full stage, as a functor.
template <typename D>
struct FullDma {
    static constexpr int kCount = D::kInst;
    const D* d;
    uint32_t slot;
    int k0;
    __device__ __forceinline__ void operator()(int i) const { d->issue_full_lean(slot, k0, i); }
};

// The same for the last stages: `on` and `full` are wave-uniform.
template <typename D>
struct TailDma {
    static constexpr int kCount = D::kInst;
    const D* d;
    uint32_t slot;
    int k0, K;
    bool on, full;
    __device__ __forceinline__ void operator()(int i) const {
        if (on) {
            if (full) d->issue_full_lean(slot, k0, i);
            else d->issue_checked(slot, k0, K, i);
        }
    }
};

// Half e of the 32-byte K piece of step h for the 32-row block at `row`.
__device__ __forceinline__ uint4 read_half2(const uint8_t* slot, int row, int h, int e) {
    const int lane = threadIdx.x & 63;
    const int c = 4 * h + 2 * (lane >> 5) + e;
    return *reinterpret_cast<const uint4*>(slot + row * kBK2 + ((c ^ swz2(row)) << 4));
}

// All fragments of step h of a stage, in the order mma_step reads them
// (BM-row tile: a wave covers BM/2 rows, BM/64 blocks of 32).
template <int BM>
__device__ __forceinline__ void load_frags2(Frags<BM, 256>& f, const uint8_t* As, const uint8_t* Bs, int h,
                                            int wm, int wn) {
    constexpr int TI = BM / 64;
    const int lane = threadIdx.x & 63;
    set_half(f.a[0], 0, read_half2(As, wm * (BM / 2) + (lane & 31), h, 0));
    set_half(f.a[0], 1, read_half2(As, wm * (BM / 2) + (lane & 31), h, 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        set_half(f.b[j], 0, read_half2(Bs, wn * 128 + j * 32 + (lane & 31), h, 0));
        set_half(f.b[j], 1, read_half2(Bs, wn * 128 + j * 32 + (lane & 31), h, 1));
    }
#pragma unroll
    for (int i = 1; i < TI; ++i) {
        set_half(f.a[i], 0, read_half2(As, wm * (BM / 2) + i * 32 + (lane & 31), h, 0));
        set_half(f.a[i], 1, read_half2(As, wm * (BM / 2) + i * 32 + (lane & 31), h, 1));
    }
}

// The 4 * BM/64 MFMAs of one K = 64 step from `cur`, as an explicit
// program.  BAR: after the first MFMA, s_waitcnt vmcnt(N) lgkmcnt(0) and
// s_barrier, with N = 0, VM1 or VM2 for vmsel = 0, 1, 2.  The LDS reads of
// the next step's fragments (step h of the stage in As/Bs) are spread over
// the MFMAs after the barrier, and so are the DMA functor's kCount
// instructions.
template <int FA, int FB, bool BAR, int VM1, int VM2, typename DMA, int BM>
__device__ __forceinline__ void mma_step(v16f (&acc)[4][BM / 64], const Frags<BM, 256>& cur, Frags<BM, 256>& nxt,
                                         const uint8_t* As, const uint8_t* Bs, int h, int wm, int wn,
                                         const DMA& dma, int vmsel) {
    constexpr int TI = BM / 64;
    constexpr int kReads = 2 * (TI + 4), kMfma = 4 * TI;
    constexpr int q0 = BAR ? 1 : 0;             // first MFMA followed by reads / DMA
    constexpr int kSlots = kMfma - q0;
    const int lane = threadIdx.x & 63;
    auto one_read = [&](int r) {
        const int f = r >> 1, e = r & 1;
        if (f == 0) {
            set_half(nxt.a[0], e, read_half2(As, wm * (BM / 2) + (lane & 31), h, e));
        } else if (f <= 4) {
            const int j = f - 1;
            set_half(nxt.b[j], e, read_half2(Bs, wn * 128 + j * 32 + (lane & 31), h, e));
        } else {
            const int i = f - 4;
            set_half(nxt.a[i], e, read_half2(As, wm * (BM / 2) + i * 32 + (lane & 31), h, e));
        }
    };
#pragma unroll
    for (int q = 0; q < kMfma; ++q) {
        const int i = q / 4, j = q % 4;
        acc[j][i] = mfma32<FB, FA>(cur.b[j], cur.a[i], acc[j][i]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (BAR) {
            if (q == 0) {
                if (vmsel == 1) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM1) : "memory");
                else if (vmsel == 2) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(VM2) : "memory");
                else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
            }
        }
        if (q >= q0) {
            const int t = q - q0;
            {
                const int lo = (t * kReads) / kSlots, hi = ((t + 1) * kReads) / kSlots;
#pragma unroll
                for (int r = 0; r < kReads; ++r)
                    if (r >= lo && r < hi) one_read(r);
            }
            const int d0 = (t * DMA::kCount) / kSlots, d1 = ((t + 1) * DMA::kCount) / kSlots;
#pragma unroll
            for (int d = 0; d < DMA::kCount; ++d)
                if (d >= d0 && d < d1) dma(d);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Epilogue of one BM x 256 tile staged through 32 KiB of LDS: each wave
// owns 8 KiB = 32 rows x 256 bytes of it, so it writes its (BM/2) x 128
// tile in passes of one 32-row MFMA block (BM = 256, bf16: all 128 columns,
// 4 passes; fp32: 64 columns, 8 passes; BM = 128: half as many).  A pass
// writes the scaled, converted values (row r's 16-byte chunk c at physical
// chunk c ^ (r & 15)), reads them back as 16-byte row chunks (16 lanes per
// 256-byte row segment) and stores them.
// An interior tile with 16-byte aligned rows issues exactly kStores vector
// stores per wave, unconditionally (the persistent loop's vmcnt accounting
// relies on it).
template <bool OUT_BF16, int BM>
struct Epi2 {
    static constexpr int kEsz = OUT_BF16 ? 2 : 4;
    static constexpr int kCols = 256 / kEsz;            // columns per pass
    static constexpr int kJ = kCols / 32;               // MFMA column blocks per pass
    static constexpr int kPasses = (BM / 64) * (4 / kJ);
    static constexpr int kStores = kPasses * 8;         // 8 KiB per pass, 1 KiB per store
};

// Scale of an epilogue: SMODE bit 0 = one A scale per row (else sa0), bit 1
// = one B scale per column (else sb0); every mode multiplies the fp32 sum by
// fl32(sa * sb).  SMODE 4 stores the sums as they are (the block-scaled
// GEMM has applied its scales already).  The per-row and per-column scales a lane needs (4 rows, 64
// columns) are loaded once at the start of the epilogue, so the only wait
// for them is the one before the first pass; the scalar scales come in
// through scalar loads, which never wait for the vector-memory DMA.
template <bool OUT_BF16, int SMODE, int BM>
__device__ __forceinline__ void epilogue_body(const GemmParams& p, const float* __restrict__ sbp, float sa0,
                                              float sb0, const v16f (&acc)[4][BM / 64], int m0, int n0, int wm,
                                              int wn, int wave, int lane, uint8_t* slot, bool interior) {
    using E = Epi2<OUT_BF16, BM>;
    constexpr int TI = BM / 64;
    constexpr int kEsz = E::kEsz, kJ = E::kJ;
    uint8_t* stage = slot + wave * 8192;
    const int mw = m0 + wm * (BM / 2), nw = n0 + wn * 128; // wave tile origin
    const int r_w = lane & 31;                              // row of this lane in a 32-row block
    float sar[TI];
    float sbc[4][4][4];
    if constexpr (SMODE & 1) {
#pragma unroll
        for (int i = 0; i < TI; ++i) sar[i] = p.sa[min(mw + i * 32 + r_w, p.M - 1)];
    }
    if constexpr (SMODE & 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sbc[j][g][e] = sbp[min(nw + j * 32 + g * 8 + (lane >> 5) * 4 + e, p.N - 1)];
    }
    const float s00 = sa0 * sb0;
#pragma unroll
    for (int pass = 0; pass < E::kPasses; ++pass) {
        const int i = pass / (4 / kJ);                      // 32-row block
        const int jb = (pass % (4 / kJ)) * kJ;              // first MFMA column block
        float srow = s00;
        if constexpr (SMODE == 1) srow = sar[i] * sb0;
        // 1. registers -> LDS: lane holds columns j*32 + g*8 + (lane/32)*4 + 0..3
#pragma unroll
        for (int jj = 0; jj < kJ; ++jj) {
            const int j = jb + jj;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = jj * 32 + g * 8 + (lane >> 5) * 4;     // within the pass
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float sc;
                    if constexpr (SMODE == 3) sc = sar[i] * sbc[j][g][e];
                    else if constexpr (SMODE == 2) sc = sa0 * sbc[j][g][e];
                    else sc = srow;
                    if constexpr (SMODE == 4) v[e] = acc[j][i][4 * g + e];
                    else v[e] = acc[j][i][4 * g + e] * sc;
                }
                const int byte = col * kEsz;                           // logical byte in the 256-byte row
                uint8_t* dst = stage + r_w * 256 + ((((byte >> 4) ^ (r_w & 15)) << 4) | (byte & 15));
                if constexpr (OUT_BF16) {
                    typedef float f2 __attribute__((ext_vector_type(2)));
                    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
                    const f2 lo = {v[0], v[1]}, hi = {v[2], v[3]};
                    const b2 blo = __builtin_convertvector(lo, b2), bhi = __builtin_convertvector(hi, b2);
                    uint2 w;
                    w.x = __builtin_bit_cast(uint32_t, blo);
                    w.y = __builtin_bit_cast(uint32_t, bhi);
                    *reinterpret_cast<uint2*>(dst) = w;
                } else {
                    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
        __builtin_amdgcn_wave_barrier();
        // 2. LDS -> global: store t covers rows 4t .. 4t+3, lane -> row 4t + lane/16, chunk lane%16
        const int ncol0 = nw + jb * 32;
        const int ch = lane & 15;
        uint4 w[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int row = 4 * t + (lane >> 4);
            w[t] = *reinterpret_cast<const uint4*>(stage + row * 256 + ((ch ^ (row & 15)) << 4));
        }
        const int n = ncol0 + ch * (16 / kEsz);
        if (interior) {
            // exactly 8 vector stores per pass
            uint8_t* dst0 = reinterpret_cast<uint8_t*>(p.C) +
                            ((int64_t)(mw + i * 32 + (lane >> 4)) * p.ldc + n) * kEsz;
            const int64_t step = (int64_t)4 * p.ldc * kEsz;
#pragma unroll
            for (int t = 0; t < 8; ++t) *reinterpret_cast<uint4*>(dst0 + t * step) = w[t];
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int m = mw + i * 32 + 4 * t + (lane >> 4);
                uint8_t* dstg = reinterpret_cast<uint8_t*>(p.C) + ((int64_t)m * p.ldc + n) * kEsz;
                if (m < p.M && p.vec_out && n + 16 / kEsz <= p.N) {
                    *reinterpret_cast<uint4*>(dstg) = w[t];
                } else if (m < p.M && n < p.N) {
                    const uint32_t ww[4] = {w[t].x, w[t].y, w[t].z, w[t].w};
                    for (int e = 0; e < 16 / kEsz && n + e < p.N; ++e) {
                        if constexpr (OUT_BF16)
                            reinterpret_cast<uint16_t*>(dstg)[e] = (uint16_t)(ww[e >> 1] >> (16 * (e & 1)));
                        else
                            reinterpret_cast<uint32_t*>(dstg)[e] = ww[e];
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);   // the reads of this pass are done before the next writes
        __builtin_amdgcn_wave_barrier();
    }
}

// Epilogue of one BM x 256 tile: the scale mode is uniform, so one of the
// four bodies runs.  p.sb (per-column mode) and sb0 are the tile's B scales.
template <bool OUT_BF16, int BM>
__device__ __forceinline__ void epilogue_slot(const GemmParams& p, float sa0, float sb0,
                                              const v16f (&acc)[4][BM / 64], int m0, int n0, int wm, int wn, int wave,
                                              int lane_in, uint8_t* slot, bool interior) {
    // the lane id formed here from the execution mask (every lane is
    // active), opaquely: the per-lane address arithmetic stays here instead
    // of being hoisted out of the tile loop, and no register keeps the id
    // live across the K loop (a spilled id would come back through a
    // scratch load, whose wait also waits for every DMA and store in flight)
    (void)lane_in;
    int lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    const int mode = (p.sa_row ? 1 : 0) | (p.sb_row ? 2 : 0);
    if (mode == 0)
        epilogue_body<OUT_BF16, 0, BM>(p, p.sb, sa0, sb0, acc, m0, n0, wm, wn, wave, lane, slot, interior);
    else if (mode == 1)
        epilogue_body<OUT_BF16, 1, BM>(p, p.sb, sa0, sb0, acc, m0, n0, wm, wn, wave, lane, slot, interior);
    else if (mode == 2)
        epilogue_body<OUT_BF16, 2, BM>(p, p.sb, sa0, sb0, acc, m0, n0, wm, wn, wave, lane, slot, interior);
    else
        epilogue_body<OUT_BF16, 3, BM>(p, p.sb, sa0, sb0, acc, m0, n0, wm, wn, wave, lane, slot, interior);
}

// A uniform fp32 load through the scalar cache (the address is wave-uniform
// and the kernel never writes the data).
__device__ __forceinline__ float load_uniform(const float* ptr) {
    return *reinterpret_cast<const __attribute__((address_space(4))) float*>(reinterpret_cast<uintptr_t>(ptr));
}

// Linear tile of block b in round r (persistent grid of G blocks): the
// blocks of one round take G consecutive tiles, each XCD a contiguous range
// of them; the linear index is then grouped along M as in tile_coords.
__device__ __forceinline__ void tile_of_linear(const GemmParams& p, int tiles_m, int group_m, int t, int& tm,
                                               int& tn) {
    const int per_group = group_m * p.tiles_n;
    const int group = t / per_group;
    const int first_m = group * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int in_group = t - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// Grouped: the linear tiles [0, T) of a persistent grid of G blocks whose
// last round is at most half full end at the last whole round; k_gemm_h
// takes the rest as 128-row halves.
__device__ __forceinline__ int grouped_main_tiles(int T, int G) {
    const int rem = T % G;
    return (T > G && rem != 0 && 2 * rem <= G) ? T - rem : T;
}

__device__ __forceinline__ bool tile_of_round(const GemmParams& p, int tiles_m, int group_m, int limit, int r,
                                              int& tm, int& tn) {
    const int G = gridDim.x;
    int b = blockIdx.x;
    if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
    const int t = r * G + b;
    if (t >= limit) return false;
    const int per_group = group_m * p.tiles_n;
    const int group = t / per_group;
    const int first_m = group * group_m;
    const int gsize = min(tiles_m - first_m, group_m);
    const int in_group = t - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
    return true;
}

// Where the rows, the B operand and the B scales of M-tile tm come from.
// Plain: rows [256 tm, M) of A, B and sb as given.  Grouped: the table entry
// of tm names its expert g and its rows [m0, m_end) (at most 256 of them,
// m_end the end of the group), B is expert g's matrix and sb its scale (one
// per expert, or the expert's N row scales).
template <bool GROUPED, int BM>
struct TileRef {                  // plain: nothing to carry
    __device__ __forceinline__ void load(const GemmParams&, int) {}
    __device__ __forceinline__ int m0(const GemmParams&, int tm) const { return tm * BM; }
    __device__ __forceinline__ int m_end(const GemmParams& p) const { return p.M; }
    __device__ __forceinline__ const uint8_t* B(const GemmParams& p) const { return p.B; }
};

template <>
struct TileRef<true, 256> {
    int row0, end;
    const uint8_t* b;
    const float* sb;
    float sb0;
    __device__ __forceinline__ void load(const GemmParams& p, int tm) {
        const int4 e = p.gtab[1 + tm];
        row0 = e.y;
        end = e.z;
        b = p.B + (int64_t)e.x * p.b_gstride;
        sb = p.sb + (p.sb_row ? (int64_t)e.x * p.N : (int64_t)e.x);
        sb0 = load_uniform(sb);
    }
    __device__ __forceinline__ int m0(const GemmParams&, int) const { return row0; }
    __device__ __forceinline__ int m_end(const GemmParams&) const { return end; }
    __device__ __forceinline__ const uint8_t* B(const GemmParams&) const { return b; }
};

// Persistent scaled GEMM over 256 x 256 tiles with 128-byte K stages.
// Stages are numbered globally over this block's tiles; the ring schedule
// of each stage is the one described above, so the first two stages of the
// next tile stream in during the last two stages of the current one.  The
// epilogue stages through B(last)'s slot, which the schedule leaves free
// until the next tile's first even step, and its stores overlap the next
// tile's first stage: the first odd-step wait of a tile counts them as in
// flight (vector-memory operations complete in issue order).
// Needs K > 256 (three stages) when a block runs more than one tile.
// GROUPED: the M-tiles are those of the grouped GEMM's table, whose size
// only the device knows.
template <int FA, int FB, bool OUT_BF16, bool RAGGED, bool GROUPED>
__device__ __forceinline__ void p_rounds(const GemmParams& p) {
    constexpr int BM = 256, TI = BM / 64;        // tile rows; 32-row MFMA blocks per wave
    int tiles_m = p.tiles_m, group_m = p.group_m;
    // scalar scales (per-tensor modes; the grouped B scale is the tile's)
    const float sa0 = load_uniform(p.sa);
    const float sb0 = GROUPED ? 0.0f : load_uniform(p.sb);
    if constexpr (GROUPED) {     // the table's size, within the host's bound (p.tiles_m)
        tiles_m = min(p.gtab[0].x, p.tiles_m);
        group_m = tiles_m < 4 ? tiles_m : 4;
    }
    using E = Epi2<OUT_BF16, BM>;
    using DA = DmaL<BM>;
    constexpr int kVm1 = DA::kInst;              // the A DMA of the even step may still fly
    constexpr int kVm2 = kVm1 + E::kStores < 63 ? kVm1 + E::kStores : 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int K = p.K;
    const int nsteps = (K + 63) / 64;            // K = 64 MFMA steps
    const int nks = (nsteps + 1) / 2;            // K = 128 stages per tile
    const uint32_t ring = lds_addr(g_ring);
    auto wrap = [](int x) { return x >= 5 ? x - 5 : x; };
    auto addr = [&](int slot) { return ring + (uint32_t)(slot * kSlot2); };
    auto ptr = [&](int slot) { return g_ring + slot * kSlot2; };

    int tm, tn;
    int limit = tiles_m * p.tiles_n;
    if constexpr (GROUPED) {
        if (p.main_grid) limit = grouped_main_tiles(limit, (int)gridDim.x);
    }
    if (!tile_of_round(p, tiles_m, group_m, limit, 0, tm, tn)) return;
    int tm_n = 0, tn_n = 0;
    bool has_next = tile_of_round(p, tiles_m, group_m, limit, 1, tm_n, tn_n);
    TileRef<GROUPED, BM> cur, nxt;
    cur.load(p, tm);
    if (has_next) nxt.load(p, tm_n);

    DA da;
    Dma2 db;
    da.init(p.A, p.lda, cur.m0(p, tm), cur.m_end(p), wave);
    db.init(cur.B(p), p.ldb, tn * 256, p.N, wave);

    v16f acc[4][TI];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

    Frags<BM, 256> f0, f1;
    if (nks > 0) {
        da.issue(addr(0), 0, K);
        db.issue(addr(1), 0, K);
        if (nks > 1) {
            da.issue(addr(2), kBK2, K);
            db.issue(addr(3), kBK2, K);
            wait_and_barrier<DA::kInst + Dma2::kInst>();
        } else {
            wait_and_barrier<0>();
        }
        load_frags2(f0, ptr(0), ptr(1), 0, wm, wn);
    }
    // settle the prologue's LDS / scalar loads so that the loop head waits
    // only for the reads of the previous step
    __builtin_amdgcn_s_waitcnt(0xC07F);

    int sl = 0;        // 2g mod 5 for the global stage g: A(g) in slot sl, B(g) in sl+1,
                       // A(g+1) in sl+2, B(g+1) in sl+3, A(g+2) in sl+4, B(g+2) in sl
    int first_vm = 1;  // the first odd-step wait of a tile: 8, or 8 + the previous epilogue's stores
    for (int r = 0;; ++r) {
        const int m0 = cur.m0(p, tm), n0 = tn * 256;
        int s = 0;
        // stages whose DMA target (s + 2) is in this tile
        for (; s + 2 < nks; ++s) {
            const int s1 = wrap(sl + 1), s2 = wrap(sl + 2), s3 = wrap(sl + 3), s4 = wrap(sl + 4);
            const int vmsel = s == 0 ? first_vm : 1;
            if constexpr (RAGGED) {
                const bool full = (s + 3) * kBK2 <= K;
                const TailDma<DA> dA{&da, addr(s4), (s + 2) * kBK2, K, true, full};
                mma_step<FA, FB, false, kVm1, kVm2>(acc, f0, f1, ptr(sl), ptr(s1), 1, wm, wn, dA, 0);
                const TailDma<Dma2> dB{&db, addr(sl), (s + 2) * kBK2, K, true, full};
                mma_step<FA, FB, true, kVm1, kVm2>(acc, f1, f0, ptr(s2), ptr(s3), 0, wm, wn, dB, vmsel);
            } else {
                const FullDma<DA> dA{&da, addr(s4), (s + 2) * kBK2};
                mma_step<FA, FB, false, kVm1, kVm2>(acc, f0, f1, ptr(sl), ptr(s1), 1, wm, wn, dA, 0);
                const FullDma<Dma2> dB{&db, addr(sl), (s + 2) * kBK2};
                mma_step<FA, FB, true, kVm1, kVm2>(acc, f1, f0, ptr(s2), ptr(s3), 0, wm, wn, dB, vmsel);
            }
            sl = s2;
        }
        // every DMA of this tile is issued: point the descriptors at the next
        // tile, whose stages 0 and 1 are issued by this tile's last two stages
        if (has_next) {
            da.init(p.A, p.lda, nxt.m0(p, tm_n), nxt.m_end(p), wave);
            db.init(nxt.B(p), p.ldb, tn_n * 256, p.N, wave);
        }
        for (; s < nks; ++s) {
            const int s1 = wrap(sl + 1), s2 = wrap(sl + 2), s3 = wrap(sl + 3), s4 = wrap(sl + 4);
            // odd-step wait: stage s+1 (this tile's, or the next tile's stage 0)
            // must be in; only the A issued in this even step may still fly
            const int vmsel = has_next ? 1 : 0;
            const TailDma<DA> dA{&da, addr(s4), (s + 2 - nks) * kBK2, K, has_next, true};
            mma_step<FA, FB, false, kVm1, kVm2>(acc, f0, f1, ptr(sl), ptr(s1), 1, wm, wn, dA, 0);
            const TailDma<Dma2> dB{&db, addr(sl), (s + 2 - nks) * kBK2, K, has_next, true};
            mma_step<FA, FB, true, kVm1, kVm2>(acc, f1, f0, ptr(s2), ptr(s3), 0, wm, wn, dB, vmsel);
            sl = s2;
        }
        // B(last)'s slot is free until the next tile's first even step
        const bool interior = p.vec_out && m0 + BM <= cur.m_end(p) && n0 + 256 <= p.N;
        if constexpr (GROUPED) {
            GemmParams pt = p;           // the tile's rows end at its group's end
            pt.M = cur.end;
            pt.sb = cur.sb;
            epilogue_slot<OUT_BF16, BM>(pt, sa0, cur.sb0, acc, m0, n0, wm, wn, wave, lane, ptr(wrap(sl + 4)), interior);
        } else {
            epilogue_slot<OUT_BF16, BM>(p, sa0, sb0, acc, m0, n0, wm, wn, wave, lane, ptr(wrap(sl + 4)), interior);
        }
        if (!has_next) break;
        first_vm = interior ? 2 : 1;
        tm = tm_n; tn = tn_n;
        if constexpr (GROUPED) cur = nxt;
        has_next = tile_of_round(p, tiles_m, group_m, limit, r + 2, tm_n, tn_n);
        if (has_next) nxt.load(p, tm_n);
        __syncthreads();   // every wave is done with the staging slot
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < TI; ++i)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[j][i][q] = 0.0f;
    }
}

// ------------------------------------------------------------------------
// Scaled GEMM over 128 x 256 tiles, one tile per block, for the launches
// whose tiles would otherwise leave half the CUs idle.  A whole stage (A
// 128 x 128 B, B 256 x 128 B: 48 KiB) fits three times in LDS: stage s
// lives in slot s mod 3.  The odd step of stage s waits for stage s+1 (only
// A(s+2) and B(s+2) may still fly), meets the other waves (every wave is
// done reading stage s), then issues B(s+3) into stage s's slot; the next
// even step issues A(s+3) there.  So B streams three stages ahead (less
// the odd step) and A two, against one and two in k_gemm_p.  The MFMA
// program, its fragment reads and the epilogue are those of k_gemm_p with
// 128-row tiles, so every output's K sum is the same chain of MFMAs.
// ------------------------------------------------------------------------
// One stage of a BM x 256 tile: A (BM x 128 B), then B (256 x 128 B).
template <int BM>
constexpr int h_stage() { return BM * kBK2 + 256 * kBK2; }
constexpr int kHStage = h_stage<128>();               // 48 KiB
constexpr int kHRing = 3 * kHStage;                   // the ring of the largest tile

// One BM x 256 tile (BM = 128, or 64 for the quarter tiles of a grouped
// GEMM's last round) at rows [m0, m_end) and columns n0.. (m_end: the
// problem's M, or the end of the tile's group), with B operand Bp and the
// tile's B scales sbp (per column) or sb0.  BM = 64: each wave covers 32
// rows, one row block of the same MFMA program.
template <int FA, int FB, bool OUT_BF16, bool GROUPED, int BM = 128>
__device__ __forceinline__ void h_tile(const GemmParams& p, int m0, int m_end, int n0, const uint8_t* Bp,
                                       const float* sbp, float sa0, float sb0) {
    constexpr int kStage = h_stage<BM>();
    using DA = DmaL<BM>;
    constexpr int kVm1 = DA::kInst + Dma2::kInst;  // A(s+2) and B(s+2) may still fly
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int K = p.K;
    const int nks = (K + kBK2 - 1) / kBK2;
    const uint32_t ring = lds_addr(g_ring);
    auto addr = [&](int slot) { return ring + (uint32_t)(slot * kStage); };
    auto aptr = [&](int slot) { return g_ring + slot * kStage; };
    auto bptr = [&](int slot) { return g_ring + slot * kStage + BM * kBK2; };

    DA da;
    Dma2 db;
    da.init(p.A, p.lda, m0, m_end, wave);
    db.init(Bp, p.ldb, n0, p.N, wave);

    v16f acc[4][BM / 64];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < BM / 64; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.0f;

    Frags<BM, 256> f0, f1;
    if (nks > 0) {
        // A(0), B(0), A(1), B(1), B(2); A(2) comes with the first even step
        for (int i = 0; i < 2 && i < nks; ++i) {
            da.issue(addr(i), i * kBK2, K);
            db.issue(addr(i) + (uint32_t)(BM * kBK2), i * kBK2, K);
        }
        if (nks > 2) db.issue(addr(2) + (uint32_t)(BM * kBK2), 2 * kBK2, K);
        if (nks > 2) wait_and_barrier<DA::kInst + 2 * Dma2::kInst>();
        else if (nks == 2) wait_and_barrier<kVm1>();
        else wait_and_barrier<0>();
        load_frags2(f0, aptr(0), bptr(0), 0, wm, wn);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);

    int cs = 0;                                    // slot of stage s
    int s = 0;
    // even step: the MFMAs of stage s's first half, the reads of its second;
    // A(s+2) into stage s-1's slot (free since the last barrier).  Odd step:
    // stage s+1 in (only A(s+2), B(s+2) may fly; nothing past the last
    // stage), every wave done with stage s; reads of stage s+1's first half
    // and B(s+3) into stage s's slot.  While both DMAs are whole stages the
    // loop carries no branch around them.
    for (; s + 3 < nks && (s + 4) * kBK2 <= K; ++s) {
        const int ns = cs == 2 ? 0 : cs + 1;       // slot of stage s+1
        const int ps = ns == 2 ? 0 : ns + 1;       // slot of stage s+2 (stage s-1's)
        const FullDma<DA> dA{&da, addr(ps), (s + 2) * kBK2};
        mma_step<FA, FB, false, kVm1, kVm1>(acc, f0, f1, aptr(cs), bptr(cs), 1, wm, wn, dA, 0);
        const FullDma<Dma2> dB{&db, addr(cs) + (uint32_t)(BM * kBK2), (s + 3) * kBK2};
        mma_step<FA, FB, true, kVm1, kVm1>(acc, f1, f0, aptr(ns), bptr(ns), 0, wm, wn, dB, 1);
        cs = ns;
    }
    for (; s < nks; ++s) {
        const int ns = cs == 2 ? 0 : cs + 1;
        const int ps = ns == 2 ? 0 : ns + 1;
        const TailDma<DA> dA{&da, addr(ps), (s + 2) * kBK2, K, s + 2 < nks, (s + 3) * kBK2 <= K};
        mma_step<FA, FB, false, kVm1, kVm1>(acc, f0, f1, aptr(cs), bptr(cs), 1, wm, wn, dA, 0);
        const TailDma<Dma2> dB{&db, addr(cs) + (uint32_t)(BM * kBK2), (s + 3) * kBK2, K, s + 3 < nks,
                               (s + 4) * kBK2 <= K};
        mma_step<FA, FB, true, kVm1, kVm1>(acc, f1, f0, aptr(ns), bptr(ns), 0, wm, wn, dB, s + 2 < nks ? 1 : 0);
        cs = ns;
    }
    // the last odd step's fragment reads (of no stage) are done before the
    // epilogue stages its values through the ring
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __syncthreads();
    const bool interior = p.vec_out && m0 + BM <= m_end && n0 + 256 <= p.N;
    if constexpr (GROUPED) {
        GemmParams pt = p;           // the tile's rows end at its group's end
        pt.M = m_end;
        pt.sb = sbp;
        epilogue_slot<OUT_BF16, BM>(pt, sa0, sb0, acc, m0, n0, wm, wn, wave, lane, g_ring, interior);
    } else {
        epilogue_slot<OUT_BF16, BM>(p, sa0, sb0, acc, m0, n0, wm, wn, wave, lane, g_ring, interior);
    }
}

// k_gemm_h: one BM-row tile per block, over p's tiles (problems with at
// most half as many 256-row tiles as CUs, or at most 128 rows; BM = 64 when
// one round of 64-row tiles fits the grid).  GROUPED:
// the blocks take the R grouped-GEMM tiles that the persistent kernel left
// (its last round, when at most half full: grouped_main_tiles with the grid
// p.main_grid), as 4 R quarters of 64 rows when they fit the grid, else as
// 2 R halves of 128 rows: a quarter has a quarter of a tile's K loop, so
// the round ends sooner while most CUs would idle anyway.  Pieces are dealt
// so that every XCD takes an equal run of whole tiles (a tile's pieces
// share its B panel in that XCD's L2); piece j of tile t covers rows
// j * BM.. of the tile.  Pieces past their group's end, and blocks past the
// pieces, exit.
template <int FA, int FB, bool OUT_BF16, bool GROUPED, int BM = 128>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_h(GemmParams p) {
    int tm, tn;
    if constexpr (GROUPED) {
        const int tiles_m = min(p.gtab[0].x, p.tiles_m);
        const int T = tiles_m * p.tiles_n;
        const int main = grouped_main_tiles(T, p.main_grid);
        const int G = gridDim.x;
        const bool quarters = 4 * (T - main) <= G;
        const int sh = quarters ? 2 : 1;             // log2 of pieces per tile
        const int np = (T - main) << sh;
        int b = blockIdx.x;
        if ((G & 7) == 0) {
            const int c = ((np + (8 << sh) - 1) >> (3 + sh)) << sh;   // pieces per XCD, whole tiles
            if (c <= (G >> 3)) b = (b >> 3) < c ? (b & 7) * c + (b >> 3) : np;
        }
        if (b >= np) return;
        const int t = main + (b >> sh);
        tile_of_linear(p, tiles_m, tiles_m < 4 ? tiles_m : 4, t, tm, tn);
        const int4 e = p.gtab[1 + tm];
        const int m0 = e.y + (quarters ? 64 : 128) * (b & ((1 << sh) - 1));
        if (m0 >= e.z) return;
        const uint8_t* Bp = p.B + (int64_t)e.x * p.b_gstride;
        const float* sbp = p.sb + (p.sb_row ? (int64_t)e.x * p.N : (int64_t)e.x);
        if (quarters)
            h_tile<FA, FB, OUT_BF16, true, 64>(p, m0, e.z, tn * 256, Bp, sbp, load_uniform(p.sa), load_uniform(sbp));
        else
            h_tile<FA, FB, OUT_BF16, true>(p, m0, e.z, tn * 256, Bp, sbp, load_uniform(p.sa), load_uniform(sbp));
    } else {
        tile_coords(p, tm, tn);
        h_tile<FA, FB, OUT_BF16, false, BM>(p, tm * BM, p.M, tn * 256, p.B, p.sb, load_uniform(p.sa),
                                            load_uniform(p.sb));
    }
}

// Which of T half tiles (T <= the grid) this block runs after its whole
// rounds: every XCD (blocks are dealt to the 8 XCDs round robin) takes a
// contiguous run of ceil(T / 8) of them, so that a tail smaller than the
// grid still spreads over every XCD and neighbouring tiles share an XCD's
// L2.  A result >= T: none.
__device__ __forceinline__ int tail_slot(int T) {
    const int G = gridDim.x, b = blockIdx.x;
    if ((G & 7) != 0) return b;
    const int c = (T + 7) >> 3;            // <= G / 8 since T <= G
    return (b >> 3) < c ? (b & 7) * c + (b >> 3) : T;
}

// The half tiles of a plain persistent launch (p.tail_N > p.N): columns
// [p.N, p.tail_N) as 128 x 256 tiles, at most one per block, which a block
// runs once its whole rounds are done, in the order of tile_coords.
template <int FA, int FB, bool OUT_BF16>
__device__ __forceinline__ void p_tail(const GemmParams& p) {
    constexpr int kEsz = OUT_BF16 ? 2 : 4;
    const int n0 = p.N;
    GemmParams t = p;
    t.B = p.B + (int64_t)n0 * p.ldb;
    t.C = reinterpret_cast<uint8_t*>(p.C) + (int64_t)n0 * kEsz;
    if (p.sb_row) t.sb = p.sb + n0;
    t.N = p.tail_N - n0;
    t.tiles_m = (p.M + 127) / 128;
    t.tiles_n = (t.N + 255) / 256;
    t.group_m = t.tiles_m < 4 ? t.tiles_m : 4;
    const int T = t.tiles_m * t.tiles_n;
    const int b = tail_slot(T);
    if (b >= T) return;
    int tm, tn;
    tile_of_linear(t, t.tiles_m, t.group_m, b, tm, tn);
    h_tile<FA, FB, OUT_BF16, false>(t, tm * 128, t.M, tn * 256, t.B, t.sb, load_uniform(t.sa),
                                    load_uniform(t.sb));
}

// Persistent scaled GEMM (p_rounds), then a plain launch's half tiles, if
// any: each block takes its half tile once its whole rounds are done.  (The
// grouped GEMM leaves its half tiles to a k_gemm_h launch: in the grouped
// kernel, the tail's code raised the register spills of the main loop from
// 4 to 22 and made the moe GEMM 2 % slower.)
template <int FA, int FB, bool OUT_BF16, bool RAGGED, bool GROUPED>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_p(GemmParams p) {
    p_rounds<FA, FB, OUT_BF16, RAGGED, GROUPED>(p);
    if constexpr (!GROUPED) {
        if (p.tail_N > p.N) {
            __syncthreads();     // every wave is done with the last epilogue's staging slot
            p_tail<FA, FB, OUT_BF16>(p);
        }
    }
}

// ------------------------------------------------------------------------
// Block-scaled GEMM over 256 x 256 tiles with eight waves (two per SIMD),
// persistent ([DeepL bets on FP8] 2.3, per-block scaling).
//
// Wave w owns rows 64 (w >> 1) .. +64 and columns 128 (w & 1) .. +128 of the
// tile (2 x 4 MFMA blocks of 32 x 32); the two waves that share a SIMD own
// the same columns and different rows.  A stage is one 128-wide K block:
// A and B (32 KiB each) and the block's 256 A-row scales land in one of two
// LDS buffers by DMA (per wave: four A and four B instructions of 8 rows
// and one 4-byte load of 32 row scales).  A wave holds the stage's A
// fragments (both 64-wide halves of its two row blocks) for the whole stage
// and streams B one column block at a time (double-buffered).  Each output
// block takes its two MFMAs back to back into a fresh partial sum, which
// the wave then promotes into the accumulator,
// acc += part * fl32(sa[m, kb] * sb[n/128, kb]), one FMA per element in
// architectural registers; while one wave waits for its MFMAs and promotes,
// the other wave of the SIMD issues its own MFMAs, so the promotion runs
// beside the matrix instructions.  Two barriers per stage: at column block
// 1 every wave holds its A fragments and scales of the stage, so A and the
// scales of stage s+2 may replace them in this buffer; at column block 3
// stage s+1 has landed and every wave is done reading this buffer's B,
// which then receives B of stage s+2.  Per output, the arithmetic is the
// same two MFMAs per K block from zero and the same FMA per K block in K
// order as the definition above the public entry point states.
// ------------------------------------------------------------------------
constexpr int kBQThreads = 512;
constexpr int kBQSlot = 256 * kBK2;              // one operand of one stage: 32 KiB
constexpr int kBQB = 2 * kBQSlot;                // LDS: A0 | A1 | B0 | B1 | scales 0 | scales 1
constexpr int kBQScale = 8 * 256;                // 8 waves x 64 lanes x 4 bytes (32 rows used per wave)
constexpr int kBQS = 4 * kBQSlot;
constexpr int kBQLds = kBQS + 2 * kBQScale;

// One LDS fragment read at a per-lane address plus a constant offset.
__device__ __forceinline__ uint4 lds_read16(uint32_t addr, int imm) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    const u4 v = *reinterpret_cast<const LDS_AS u4*>((uintptr_t)(addr + (uint32_t)imm));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// One stage of k_gemm_bq from buffer Q (the K loop is unrolled by two, so
// every LDS offset is a constant): column blocks 0-2 with the next column
// block's B streaming in, then the barrier, then column block 3 with the
// DMA of stage s+2 into this buffer and the reads of stage s+1.  RB: 32-row
// blocks per wave (2 in a 256-row tile, 1 in a 128-row tile).
template <int RB>
struct BQState {
    v16f acc[4][RB];    // [column block j][row block i]
    v16f part;          // partial sum of the latest output block
    v8i a[RB][2];       // A fragments of the stage: [row block][64-wide half]
    v8i bc[2], bn[2];   // B fragments of the current / next column block: [half]
    float sc[RB];       // promotion scales of this stage, per row block
};

// DMA instructions per wave per stage of a (128 RB)-row tile: A rows, B
// rows, then one for the A-row scales.
template <int RB>
struct BQDma {
    using DA = DmaL<128 * RB, 8>;
    using DB = DmaL<256, 8>;
    static constexpr int kA = DA::kInst, kB = DB::kInst, kPer = kA + kB + 1;
};

template <int Q, int RB, typename ISSUE>
__device__ __forceinline__ void bq_stage(BQState<RB>& t, const uint32_t (&la)[2][2], const uint32_t (&lb)[2][2],
                                         uint32_t lsc, bool more, bool fill, float sbn,
                                         const ISSUE& issue) {
    constexpr int kA = BQDma<RB>::kA, kB = BQDma<RB>::kB, kS = kA + kB;   // kS: the scale DMA
    auto read_b = [&](v8i (&b)[2], int q, int j) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e) set_half(b[h], e, lds_read16(lb[h][e], q * kBQSlot + j * 32 * kBK2));
    };
    auto read_a = [&](int q, int i) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e) set_half(t.a[i][h], e, lds_read16(la[h][e], q * kBQSlot + i * 32 * kBK2));
    };
    // The empty asm takes the sums as operands, so the FMAs stay here instead
    // of sinking towards the epilogue (which would keep every block's
    // partial sum alive).
    auto promote = [&](int j, int i, float f) {
#pragma unroll
        for (int q = 0; q < 16; ++q) t.acc[j][i][q] = __builtin_fmaf(t.part[q], f, t.acc[j][i][q]);
        asm volatile("" : "+v"(t.acc[j][i]));
    };
    auto block_mma = [&](int i) {
        const v16f z = {};
        t.part = mfma32<0, 0>(t.bc[0], t.a[i][0], z);
        __builtin_amdgcn_sched_barrier(0);
        t.part = mfma32<0, 0>(t.bc[1], t.a[i][1], t.part);
        __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) {
        if (jj == 1) {
            // every wave has its A fragments and scales of this stage (read at
            // the end of the previous one): A and the scales of stage s+2 may
            // replace them
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        read_b(t.bn, Q, jj + 1);
        block_mma(0);
        if (jj == 1 && fill) {
#pragma unroll
            for (int d = 0; d < (RB == 2 ? kA - 1 : kA); ++d) issue(d);
            if constexpr (RB == 1) issue(kS);
        }
        promote(jj, 0, t.sc[0]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (RB == 2) {
            block_mma(1);
            if (jj == 1 && fill) {
                issue(kA - 1);
                issue(kS);
            }
            promote(jj, 1, t.sc[1]);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) t.bc[h] = t.bn[h];
    }
    // column block 3: stage s+1 has landed (only this stage's A and scale
    // DMA may still fly) and every wave is done reading this buffer's B
    // (the last B reads were waited for here)
    if (fill) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kA + 1) : "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    asm volatile("" : "+s"(sbn));
    block_mma(0);
    if (fill) {
#pragma unroll
        for (int d = kA; d < kA + kB / 2; ++d) issue(d);
    }
    promote(3, 0, t.sc[0]);
    __builtin_amdgcn_sched_barrier(0);
    float san[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) san[i] = 0.0f;
    if (more) {
        read_b(t.bn, Q ^ 1, 0);
        read_a(Q ^ 1, 0);
#pragma unroll
        for (int i = 0; i < RB; ++i)
            san[i] = *reinterpret_cast<const LDS_AS float*>(
                (uintptr_t)(lsc + (uint32_t)((Q ^ 1) * kBQScale + i * 256)));
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (RB == 2) {
        block_mma(1);
        if (fill) {
#pragma unroll
            for (int d = kA + kB / 2; d < kS; ++d) issue(d);
        }
        promote(3, 1, t.sc[1]);
        __builtin_amdgcn_sched_barrier(0);
        if (more) read_a(Q ^ 1, 1);
    } else {
        if (fill) {
#pragma unroll
            for (int d = kA + kB / 2; d < kS; ++d) issue(d);
        }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) t.bc[h] = t.bn[h];
#pragma unroll
    for (int i = 0; i < RB; ++i) t.sc[i] = san[i] * sbn;
}

// One (128 RB) x 256 tile of k_gemm_bq at rows m0, columns n0: eight waves
// as 4 x 2, each (32 RB) rows x 128 columns.  RB = 1 serves the last round
// of a grid whose remaining tiles fill at most half of it, as half tiles:
// every output's K sum is the same chain of MFMAs and promotions as in a
// whole tile.
template <int RB, bool OUT_BF16>
__device__ __forceinline__ void bq_tile(const GemmParams& p, int m0, int n0, int wave, int wm, int wn) {
    using Dm = BQDma<RB>;
    typename Dm::DA da;
    typename Dm::DB db;
    const int lane = threadIdx.x & 63;
    const int K = p.K;
    const int nks = K / kBK2;                    // stages (128-wide K blocks) per tile
    const int nbn = p.N / 128;                   // 128-row blocks of B
    const uint32_t ring = lds_addr(g_ring);
    // Per-lane LDS addresses of the fragment reads in buffer 0, [half h][piece
    // e]: row r of the wave's first 32-row block, 16-byte chunk
    // 4h + 2 (lane / 32) + e under the row's swizzle (which depends on r only
    // through bits 1-3, so a row block's and buffer 1's offsets are constants
    // that fit a read's 16-bit immediate).
    uint32_t la[2][2], lb[2][2];
    {
        const int r32 = lane & 31;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int ra = wm * (32 * RB) + r32, rb = wn * 128 + r32;
                const int c = 4 * h + 2 * (lane >> 5) + e;
                la[h][e] = ring + (uint32_t)(ra * kBK2 + ((c ^ swz2(ra)) << 4));
                lb[h][e] = ring + (uint32_t)(kBQB + rb * kBK2 + ((c ^ swz2(rb)) << 4));
                asm volatile("" : "+v"(la[h][e]), "+v"(lb[h][e]));
            }
    }
    // this lane's A-row scale of row block 0 in buffer 0 (row block 1: +256
    // bytes): wave w's scale DMA fills rows 32 w .. 32 w + 31
    uint32_t lsc = ring + (uint32_t)(kBQS + (wm * RB) * 256 + (lane & 31) * 4);
    asm volatile("" : "+v"(lsc));

    da.init(p.A, p.lda, m0, p.M, wave);
    db.init(p.B, p.ldb, n0, p.N, wave);
    // this wave's DMA of A-row scales: rows 32 w + lane (lanes 0-31)
    const int rows_here = max(0, min(128 * RB, p.M - m0));
    const v4i sa_rsrc = make_rsrc(p.sa + (int64_t)m0 * nks, (uint32_t)((int64_t)rows_here * nks * 4));
    const int srow = wave * 32 + lane;
    const uint32_t sa_off0 = (lane < 32 && srow < rows_here) ? (uint32_t)(srow * nks * 4) : kOOB;
    // the B scales of this wave's 128 columns (a block past N is never stored)
    const float* sbw = p.sb + (int64_t)min((n0 + wn * 128) / 128, nbn - 1) * nks;
    auto issue_one = [&](int st, int q, int d) {
        if (d < Dm::kA) da.issue_full_lean(ring + (uint32_t)(q * kBQSlot), st * kBK2, d);
        else if (d < Dm::kA + Dm::kB)
            db.issue_full_lean(ring + (uint32_t)(kBQB + q * kBQSlot), st * kBK2, d - Dm::kA);
        else dma4(ring + (uint32_t)(kBQS + q * kBQScale + wave * 256),
                  sa_off0 == kOOB ? kOOB : sa_off0 + (uint32_t)(st * 4), sa_rsrc);
    };

    // prologue: stages 0 and 1 in flight, wait for stage 0
    BQState<RB> t;
    const float sb0 = load_uniform(sbw);
#pragma unroll
    for (int d = 0; d < Dm::kPer; ++d) issue_one(0, 0, d);
    if (nks > 1) {
#pragma unroll
        for (int d = 0; d < Dm::kPer; ++d) issue_one(1, 1, d);
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(Dm::kPer) : "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
#pragma unroll
    for (int i = 0; i < RB; ++i)
        t.sc[i] = *reinterpret_cast<const LDS_AS float*>((uintptr_t)(lsc + (uint32_t)(i * 256))) * sb0;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 2; ++e) set_half(t.a[i][h], e, lds_read16(la[h][e], i * 32 * kBK2));
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 2; ++e) set_half(t.bc[h], e, lds_read16(lb[h][e], 0));
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < RB; ++i)
#pragma unroll
            for (int q = 0; q < 16; ++q) t.acc[j][i][q] = 0.0f;

    for (int s = 0; s < nks; s += 2) {
        {
            const float sbn = s + 1 < nks ? load_uniform(sbw + s + 1) : 0.0f;
            auto iss = [&](int d) { issue_one(s + 2, 0, d); };
            bq_stage<0, RB>(t, la, lb, lsc, s + 1 < nks, s + 2 < nks, sbn, iss);
        }
        if (s + 1 < nks) {
            const float sbn = s + 2 < nks ? load_uniform(sbw + s + 2) : 0.0f;
            auto iss = [&](int d) { issue_one(s + 3, 1, d); };
            bq_stage<1, RB>(t, la, lb, lsc, s + 2 < nks, s + 3 < nks, sbn, iss);
        }
    }
    __syncthreads();
    // an opaque copy of the lane id: the epilogue's per-lane address
    // arithmetic stays here instead of being hoisted out of the tile loop
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const bool interior = p.vec_out && m0 + 128 * RB <= p.M && n0 + 256 <= p.N;
    epilogue_body<OUT_BF16, 4, 64 * RB>(p, p.sb, 1.0f, 1.0f, t.acc, m0, n0, wm, wn, wave, lane_e, g_ring,
                                        interior);
    __syncthreads();          // every wave is done with the staging area
}

// Persistent block-scaled GEMM over 256 x 256 tiles.  When the tiles leave
// a last round that fills at most half of the grid, that round runs as
// 128 x 256 halves over the whole grid (both halves of a tile on one XCD);
// a problem with at most half as many tiles as the grid runs all of them
// so (a half past M has nothing to do).
template <bool OUT_BF16>
__global__ __launch_bounds__(kBQThreads, 1) void k_gemm_bq(GemmParams p) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int G = gridDim.x;
    const int T = p.tiles_m * p.tiles_n;
    const int full = T / G, rem = T % G;
    const bool halves = rem != 0 && 2 * rem <= G;    // (full == 0: a small problem, all halves)
    const int limit = halves ? full * G : T;
    int tm, tn;
    for (int r = 0; tile_of_round(p, p.tiles_m, p.group_m, limit, r, tm, tn); ++r)
        bq_tile<2, OUT_BF16>(p, tm * 256, tn * 256, wave, wm, wn);
    if (halves) {
        int b = blockIdx.x;
        if ((G & 7) == 0) b = (b & 7) * (G >> 3) + (b >> 3);
        if (b < 2 * rem) {
            tile_of_linear(p, p.tiles_m, p.group_m, full * G + (b >> 1), tm, tn);
            const int m0 = tm * 256 + (b & 1) * 128;
            if (m0 < p.M) bq_tile<1, OUT_BF16>(p, m0, tn * 256, wave, wm, wn);
        }
    }
}

// ---------------------------------------------------------------- host side --
// Dynamic LDS of each kernel: its ring, or the epilogue staging if larger.
template <bool OUT_BF16>
constexpr size_t lds_scaled() { return (size_t)5 * kSlot2; }          // the epilogue uses one slot
static_assert(lds_scaled<true>() <= 160 * 1024 && kBQLds <= 160 * 1024 && kHRing <= 160 * 1024,
              "LDS budget of one CU");

template <typename KERN>
hipError_t set_lds(KERN kern, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

// One-time set-up of a launch site (its kernels' LDS attribute) on each
// device a call runs on: the attribute is set with the device current, so a
// process that drives several GPUs sets it on every one of them.
struct PerDeviceOnce {
    static constexpr int kDevices = 64;
    std::once_flag flag[kDevices];
    hipError_t err[kDevices] = {};
    template <typename F>
    hipError_t run(F&& f) {
        int dev = 0;
        const hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
        std::call_once(flag[dev], [&] { err[dev] = f(); });
        return err[dev];
    }
};

GemmParams make_params(const GemmArgs& a, int bm, int bn) {
    GemmParams p;
    p.A = a.A; p.B = a.B; p.lda = a.lda; p.ldb = a.ldb;
    p.M = (int)a.M; p.N = (int)a.N; p.K = (int)a.K;
    p.sa = a.sa; p.sb = a.sb; p.sa_row = a.sa_per_row; p.sb_row = a.sb_per_row;
    p.C = a.C; p.ldc = a.ldc;
    p.tiles_m = (int)((a.M + bm - 1) / bm);
    p.tiles_n = (int)((a.N + bn - 1) / bn);
    p.group_m = p.tiles_m < 4 ? p.tiles_m : 4;
    const int esz = a.out_bf16 ? 2 : 4;
    p.vec_out = ((a.ldc * esz) % 16 == 0) && ((uintptr_t)a.C % 16 == 0);   // 16-byte row chunks
    p.gtab = nullptr;
    p.b_gstride = 0;
    p.main_grid = 0;
    p.tail_N = 0;
    return p;
}

// One launch of k_gemm_p over p: a persistent grid of one block per CU when
// there are more tiles than CUs and K has at least three stages, or when
// asked for (a launch with half tiles after its rounds), else one block per
// tile.
template <int FA, int FB, bool OUT_BF16>
hipError_t launch_tiles(const GemmParams& p, int num_cus, hipStream_t stream, bool persistent = false) {
    static PerDeviceOnce once;
    const hipError_t attr_err = once.run([] {
        const hipError_t e = set_lds(k_gemm_p<FA, FB, OUT_BF16, false, false>, lds_scaled<OUT_BF16>());
        return e != hipSuccess ? e : set_lds(k_gemm_p<FA, FB, OUT_BF16, true, false>, lds_scaled<OUT_BF16>());
    });
    if (attr_err != hipSuccess) return attr_err;
    unsigned grid = (unsigned)(p.tiles_m * p.tiles_n);
    if ((grid > (unsigned)num_cus && p.K > 2 * kBK2) || persistent) grid = (unsigned)num_cus;
    if (grid == 0) return hipSuccess;
    if (p.K % kBK2 != 0)
        hipLaunchKernelGGL((k_gemm_p<FA, FB, OUT_BF16, true, false>), dim3(grid), dim3(kGemmThreads),
                           lds_scaled<OUT_BF16>(), stream, p);
    else
        hipLaunchKernelGGL((k_gemm_p<FA, FB, OUT_BF16, false, false>), dim3(grid), dim3(kGemmThreads),
                           lds_scaled<OUT_BF16>(), stream, p);
    return hipGetLastError();
}

// One launch of k_gemm_h: over p's tiles (BM-row tiles, one block each),
// or GROUPED over the grouped GEMM's split-off last round (`grid` blocks).
template <int FA, int FB, bool OUT_BF16, bool GROUPED = false, int BM = 128>
hipError_t launch_half(const GemmParams& p, hipStream_t stream, unsigned grid_grouped = 0) {
    static PerDeviceOnce once;
    const hipError_t attr_err =
        once.run([] { return set_lds(k_gemm_h<FA, FB, OUT_BF16, GROUPED, BM>, (size_t)kHRing); });
    if (attr_err != hipSuccess) return attr_err;
    const unsigned grid = GROUPED ? grid_grouped : (unsigned)(p.tiles_m * p.tiles_n);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((k_gemm_h<FA, FB, OUT_BF16, GROUPED, BM>), dim3(grid), dim3(kGemmThreads), (size_t)kHRing,
                       stream, p);
    return hipGetLastError();
}

// Scaled GEMM.  A single tile takes about the same time whether one CU or
// all of them are busy (its K loop), so a round of tiles that fills at most
// half the CUs costs nearly a full round.  Such a round runs as 128 x 256
// tiles instead, which halves each CU's share of it: a problem with at most
// half as many 256 x 256 tiles as CUs, or with at most 128 rows, runs
// entirely on them (k_gemm_h), or on 64 x 256 tiles when one round of
// those fits the grid; a persistent problem whose last round is at
// most half full runs its last columns (enough 256-wide column tiles to
// hold that round's tiles) as one round of 128-row tiles that each block of
// the persistent launch takes once its whole rounds of the other columns
// are done.  Every output's K sum is the same chain of MFMAs in both tile
// heights, so the result is bit-identical to the 256-row tiling.
template <int FA, int FB, bool OUT_BF16>
hipError_t launch_scaled_typed(const GemmArgs& a) {
    const GemmParams p = make_params(a, 256, 256);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n, cus = a.num_cus;
    if (tiles == 0) return hipSuccess;
    if (2 * tiles <= cus || a.M <= 128) {
        // 64-row tiles when one round of them fits the grid (each has a
        // quarter of a 256-row tile's K loop, so more CUs share the work)
        const GemmParams q = make_params(a, 64, 256);
        if ((int64_t)q.tiles_m * q.tiles_n <= cus) return launch_half<FA, FB, OUT_BF16, false, 64>(q, a.stream);
        return launch_half<FA, FB, OUT_BF16>(make_params(a, 128, 256), a.stream);
    }
    const int64_t last = tiles % cus;
    if (tiles > cus && a.K > 2 * kBK2 && last != 0 && 2 * last <= cus) {
        const int tail_n = (int)((last + p.tiles_m - 1) / p.tiles_m);            // column tiles of the tail
        const int64_t half_tiles = (int64_t)((p.M + 127) / 128) * tail_n;
        if (tail_n < p.tiles_n && half_tiles <= cus) {
            GemmParams head = p;
            head.N = (p.tiles_n - tail_n) * 256;
            head.tiles_n = p.tiles_n - tail_n;
            head.tail_N = p.N;
            return launch_tiles<FA, FB, OUT_BF16>(head, a.num_cus, a.stream, true);
        }
    }
    return launch_tiles<FA, FB, OUT_BF16>(p, a.num_cus, a.stream);
}

// Grouped GEMM ([DeepL bets on FP8] 3.2, MoE): one block builds the table of
// 256-row tiles of every group from the device offsets (clamped to [0, M];
// an end below its start makes the group empty; tiles past the table's
// capacity are dropped, which only offsets that are not non-decreasing can
// cause); the persistent GEMM then walks the table.
__global__ __launch_bounds__(256) void k_group_table(const int32_t* __restrict__ offsets, int groups, int M,
                                                     int* __restrict__ tab) {
    __shared__ int part[256];
    const int t = threadIdx.x;
    const int per = (groups + 255) / 256;
    const int g0 = min(groups, t * per), g1 = min(groups, g0 + per);
    auto bounds = [&](int g, int& lo, int& hi) {
        lo = min(max(offsets[g], 0), M);
        hi = max(min(max(offsets[g + 1], 0), M), lo);
    };
    int cnt = 0;
    for (int g = g0; g < g1; ++g) {
        int lo, hi;
        bounds(g, lo, hi);
        cnt += (hi - lo + 255) / 256;
    }
    part[t] = cnt;
    __syncthreads();
    if (t == 0) {                     // exclusive prefix over 256 partial counts
        int run = 0;
        for (int i = 0; i < 256; ++i) {
            const int c = part[i];
            part[i] = run;
            run += c;
        }
        tab[0] = min(run, kGroupTableTiles);
        tab[1] = tab[2] = tab[3] = 0;
    }
    __syncthreads();
    int e = part[t];
    for (int g = g0; g < g1; ++g) {
        int lo, hi;
        bounds(g, lo, hi);
        for (int m = lo; m < hi; m += 256, ++e) {
            if (e < kGroupTableTiles) {
                int* w = tab + 4 + 4 * e;
                w[0] = g; w[1] = m; w[2] = hi; w[3] = 0;
            }
        }
    }
}

template <int FA, int FB, bool OUT_BF16>
hipError_t launch_grouped_typed(const GemmArgs& a) {
    static PerDeviceOnce once;
    const hipError_t attr_err = once.run([] {
        const hipError_t e = set_lds(k_gemm_p<FA, FB, OUT_BF16, false, true>, lds_scaled<OUT_BF16>());
        return e != hipSuccess ? e : set_lds(k_gemm_p<FA, FB, OUT_BF16, true, true>, lds_scaled<OUT_BF16>());
    });
    if (attr_err != hipSuccess) return attr_err;
    int* tab = reinterpret_cast<int*>(a.scratch + kScratchGroupTable);
    hipLaunchKernelGGL(k_group_table, dim3(1), dim3(256), 0, a.stream, a.group_offsets, a.groups, (int)a.M, tab);
    GemmParams p = make_params(a, 256, 256);
    p.gtab = reinterpret_cast<const int4*>(tab);
    p.b_gstride = a.b_group_stride;
    // at most ceil(M / 256) + groups M-tiles (non-decreasing offsets), never
    // more than the table holds; the kernel takes no more than this many, so
    // that with K <= 256 (no persistent loop) every block runs one tile
    const int64_t mt = std::min<int64_t>((a.M + 255) / 256 + a.groups, kGroupTableTiles);
    p.tiles_m = (int)mt;
    int64_t grid = mt * p.tiles_n;
    // persistent: a last round of tiles at most half full (the count is
    // known on the device only) is split off to k_gemm_h as 128-row halves
    const bool split = grid > a.num_cus && a.K > 2 * kBK2;
    if (split) grid = a.num_cus;
    if (grid == 0) return hipGetLastError();
    p.main_grid = split ? (int)grid : 0;
    if (a.K % kBK2 != 0)
        hipLaunchKernelGGL((k_gemm_p<FA, FB, OUT_BF16, true, true>), dim3((unsigned)grid), dim3(kGemmThreads),
                           lds_scaled<OUT_BF16>(), a.stream, p);
    else
        hipLaunchKernelGGL((k_gemm_p<FA, FB, OUT_BF16, false, true>), dim3((unsigned)grid), dim3(kGemmThreads),
                           lds_scaled<OUT_BF16>(), a.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !split) return e;
    return launch_half<FA, FB, OUT_BF16, true>(p, a.stream, (unsigned)grid);
}

// Block-scaled GEMM (E4M3 x E4M3): 256 x 256 tiles, a persistent grid of
// at most one block per CU.  Tiles are grouped 8 along M: the 32 tiles an
// XCD runs at once then span up to 2048 rows of A and only four 256-row
// panels of B, so a large B streams from HBM about once per 2048 rows
// (grouped by 4, twice; measured on the 70B MLP shape: 13 % faster).
template <bool OUT_BF16>
hipError_t launch_block_typed(const GemmArgs& a) {
    static PerDeviceOnce once;
    const hipError_t attr_err = once.run([] { return set_lds(k_gemm_bq<OUT_BF16>, (size_t)kBQLds); });
    if (attr_err != hipSuccess) return attr_err;
    GemmParams p = make_params(a, 256, 256);
    p.group_m = p.tiles_m < 8 ? p.tiles_m : 8;
    unsigned grid = (unsigned)(p.tiles_m * p.tiles_n);
    // at most half as many tiles as CUs: one block per CU, the tiles as halves
    if (grid > (unsigned)a.num_cus || 2 * grid <= (unsigned)a.num_cus) grid = (unsigned)a.num_cus;
    if (p.tiles_m * p.tiles_n > 0)
        hipLaunchKernelGGL((k_gemm_bq<OUT_BF16>), dim3(grid), dim3(kBQThreads), (size_t)kBQLds, a.stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scaled_gemm(const GemmArgs& a) {
#define FP8MI_FMT_CASE(FA, FB)                                                              \
    if (a.fa == FA && a.fb == FB)                                                           \
        return a.out_bf16 ? launch_scaled_typed<FA, FB, true>(a) : launch_scaled_typed<FA, FB, false>(a);
    FP8MI_FMT_CASE(0, 0)
    FP8MI_FMT_CASE(1, 0)
    FP8MI_FMT_CASE(0, 1)
    FP8MI_FMT_CASE(1, 1)
#undef FP8MI_FMT_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_grouped_gemm(const GemmArgs& a) {
#define FP8MI_FMT_CASE(FA, FB)                                                              \
    if (a.fa == FA && a.fb == FB)                                                           \
        return a.out_bf16 ? launch_grouped_typed<FA, FB, true>(a) : launch_grouped_typed<FA, FB, false>(a);
    FP8MI_FMT_CASE(0, 0)
    FP8MI_FMT_CASE(1, 0)
    FP8MI_FMT_CASE(0, 1)
    FP8MI_FMT_CASE(1, 1)
#undef FP8MI_FMT_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_blockscaled_gemm(const GemmArgs& a) {
    if (a.fa != 0 || a.fb != 0) return hipErrorInvalidValue;
    return a.out_bf16 ? launch_block_typed<true>(a) : launch_block_typed<false>(a);
}

}  // namespace fp8mi
