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
//   * v_mfma_f32_32x32x64_f8f6f4 (E4M3/E5M2 per operand), 4 waves of 64 as a
//     2x2 grid, each wave a (BM/2) x (BN/2) tile of 32x32 MFMA blocks;
//   * K tiles of 128 bytes staged global -> registers -> LDS, two LDS stages
//     so the next tile's loads are in flight during the current MFMAs; one
//     barrier per K tile;
//   * LDS rows of 128 B with the 16-byte chunk index XORed by (row & 7) so
//     that the MFMA operand reads (8 rows at the same chunk per LDS cycle)
//     hit distinct banks;
//   * blockIdx -> tile mapping that keeps each XCD (blocks are dealt round
//     robin over 8 XCDs) on a contiguous, M-grouped range of tiles so that
//     concurrently running tiles share A and B panels in that XCD's L2.
#include <hip/hip_runtime.h>

#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"

namespace fp8mi {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;          // K bytes per tile
constexpr int kGemmThreads = 256;

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
};

template <int FA, int FB>
__device__ __forceinline__ v16f mfma32(const v8i& a, const v8i& b, const v16f& c) {
    // cbsz / blgp select the operand formats: 0 = E4M3, 1 = E5M2.  Zero scale
    // operands select the unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 4); }

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

template <int ROWS>
struct TileLoader {
    static constexpr int kChunks = ROWS * (kBK / 16) / kGemmThreads;   // 16-byte chunks per thread
    uint4 r[kChunks];

    __device__ __forceinline__ void load(const uint8_t* __restrict__ base, int64_t ld, int row0, int rows_valid,
                                         int k0, int K) {
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = threadIdx.x + kGemmThreads * i;
            const int row = c >> 3, cc = c & 7;
            const int k = k0 + cc * 16;
            if (row0 + row < rows_valid && k < K)
                r[i] = *reinterpret_cast<const uint4*>(base + (int64_t)(row0 + row) * ld + k);
            else
                r[i] = make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __device__ __forceinline__ void store(uint8_t* lds) const {
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
            const int c = threadIdx.x + kGemmThreads * i;
            const int row = c >> 3, cc = c & 7;
            *reinterpret_cast<uint4*>(lds + swz(row, cc)) = r[i];
        }
    }
};

// Operand fragment of one 32-row block for K step ks (64 bytes): lane l
// takes row (l & 31) and 32 bytes at K offset ks*64 + (l >> 5)*32.  A and B
// use the same lane->K assignment, so the K order inside an MFMA cannot
// change the dot product.
__device__ __forceinline__ v8i read_frag(const uint8_t* lds, int row, int ks) {
    const int lane = threadIdx.x & 63;
    const int c0 = ks * 4 + (lane >> 5) * 2;
    const uint4 lo = *reinterpret_cast<const uint4*>(lds + swz(row, c0));
    const uint4 hi = *reinterpret_cast<const uint4*>(lds + swz(row, c0 + 1));
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
    const uint32_t b = __float_as_uint(v);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x0040u);   // quiet NaN
    const uint32_t rounded = b + 0x7FFFu + ((b >> 16) & 1u);
    return (uint16_t)(rounded >> 16);
}

// BLOCK: sa is [M x K/128], sb is [N/128 x K/128]; each K tile is one scale
// block whose MFMA partial sum is promoted into acc with fl32(sa*sb).
template <int BM, int BN, int FA, int FB, bool OUT_BF16, bool BLOCK>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm(GemmParams p) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int kStageBytes = (BM + BN) * kBK;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    float* sa_lds = reinterpret_cast<float*>(smem + 2 * kStageBytes);   // BLOCK: [2][BM]

    int tile_m, tile_n;
    tile_coords(p, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int nk = (p.K + kBK - 1) / kBK;
    const int nkb = p.K / kBK;   // BLOCK only (K % 128 == 0)

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    TileLoader<BM> la;
    TileLoader<BN> lb;
    float sa_reg = 0.0f;
    la.load(p.A, p.lda, m0, p.M, 0, p.K);
    lb.load(p.B, p.ldb, n0, p.N, 0, p.K);
    if constexpr (BLOCK) {
        if (threadIdx.x < BM && m0 + (int)threadIdx.x < p.M)
            sa_reg = p.sa[(int64_t)(m0 + threadIdx.x) * nkb];
    }
    la.store(smem);
    lb.store(smem + BM * kBK);
    if constexpr (BLOCK) {
        if (threadIdx.x < BM) sa_lds[threadIdx.x] = sa_reg;
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        const uint8_t* As = smem + st * kStageBytes;
        const uint8_t* Bs = As + BM * kBK;
        const bool more = kt + 1 < nk;
        if (more) {
            la.load(p.A, p.lda, m0, p.M, (kt + 1) * kBK, p.K);
            lb.load(p.B, p.ldb, n0, p.N, (kt + 1) * kBK, p.K);
            if constexpr (BLOCK) {
                if (threadIdx.x < BM && m0 + (int)threadIdx.x < p.M)
                    sa_reg = p.sa[(int64_t)(m0 + threadIdx.x) * nkb + kt + 1];
            }
        }
        if constexpr (!BLOCK) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                v8i af[TM], bf[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) af[i] = read_frag(As, wm * WM + i * 32 + (lane & 31), ks);
#pragma unroll
                for (int j = 0; j < TN; ++j) bf[j] = read_frag(Bs, wn * WN + j * 32 + (lane & 31), ks);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc[i][j] = mfma32<FA, FB>(af[i], bf[j], acc[i][j]);
            }
        } else {
            v16f part[TM][TN];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                v8i af[TM], bf[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) af[i] = read_frag(As, wm * WM + i * 32 + (lane & 31), ks);
#pragma unroll
                for (int j = 0; j < TN; ++j) bf[j] = read_frag(Bs, wn * WN + j * 32 + (lane & 31), ks);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        if (ks == 0) {
                            const v16f z = {};
                            part[i][j] = mfma32<FA, FB>(af[i], bf[j], z);
                        } else {
                            part[i][j] = mfma32<FA, FB>(af[i], bf[j], part[i][j]);
                        }
                    }
            }
            // promotion: acc += part * fl32(sa[row] * sb[col block])
            const float sbv = p.sb[(int64_t)((n0 + wn * WN) / 128) * nkb + kt];
            const float* sa_st = sa_lds + st * BM;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                float sc[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 s4 = *reinterpret_cast<const float4*>(
                        sa_st + wm * WM + i * 32 + g * 8 + (lane >> 5) * 4);
                    sc[4 * g + 0] = s4.x * sbv;
                    sc[4 * g + 1] = s4.y * sbv;
                    sc[4 * g + 2] = s4.z * sbv;
                    sc[4 * g + 3] = s4.w * sbv;
                }
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][j][r] = __builtin_fmaf(part[i][j][r], sc[r], acc[i][j][r]);
            }
        }
        if (more) {
            uint8_t* nxt = smem + (st ^ 1) * kStageBytes;
            la.store(nxt);
            lb.store(nxt + BM * kBK);
            if constexpr (BLOCK) {
                if (threadIdx.x < BM) sa_lds[(st ^ 1) * BM + threadIdx.x] = sa_reg;
            }
        }
        __syncthreads();
    }

    // epilogue: lane holds column (lane & 31) and rows (r/4)*8 + (lane>>5)*4 + r%4
    float sa_t = 1.0f, sb_t = 1.0f;
    if constexpr (!BLOCK) {
        if (!p.sa_row) sa_t = p.sa[0];
        if (!p.sb_row) sb_t = p.sb[0];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 32 + (lane & 31);
        if (n >= p.N) continue;
        float sbn = sb_t;
        if constexpr (!BLOCK) {
            if (p.sb_row) sbn = p.sb[n];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (m >= p.M) continue;
                float v = acc[i][j][r];
                if constexpr (!BLOCK) {
                    const float sam = p.sa_row ? p.sa[m] : sa_t;
                    v = v * (sam * sbn);
                }
                if constexpr (OUT_BF16) {
                    reinterpret_cast<uint16_t*>(p.C)[(int64_t)m * p.ldc + n] = f32_to_bf16_rne(v);
                } else {
                    reinterpret_cast<float*>(p.C)[(int64_t)m * p.ldc + n] = v;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- host side --
template <int BM, int BN, int FA, int FB, bool OUT_BF16, bool BLOCK>
hipError_t launch_tile(const GemmArgs& a) {
    constexpr size_t smem = 2 * (size_t)(BM + BN) * kBK + (BLOCK ? 2 * BM * sizeof(float) : 0);
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    auto kern = k_gemm<BM, BN, FA, FB, OUT_BF16, BLOCK>;
    std::call_once(once, [&] {
        attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    });
    if (attr_err != hipSuccess) return attr_err;
    GemmParams p;
    p.A = a.A; p.B = a.B; p.lda = a.lda; p.ldb = a.ldb;
    p.M = (int)a.M; p.N = (int)a.N; p.K = (int)a.K;
    p.sa = a.sa; p.sb = a.sb; p.sa_row = a.sa_per_row; p.sb_row = a.sb_per_row;
    p.C = a.C; p.ldc = a.ldc;
    p.tiles_m = (int)((a.M + BM - 1) / BM);
    p.tiles_n = (int)((a.N + BN - 1) / BN);
    p.group_m = p.tiles_m < 4 ? p.tiles_m : 4;
    const unsigned grid = (unsigned)(p.tiles_m * p.tiles_n);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kGemmThreads), smem, a.stream, p);
    return hipGetLastError();
}

template <int BM, int BN, bool BLOCK>
hipError_t dispatch_formats(const GemmArgs& a) {
#define FP8MI_FMT_CASE(FA, FB)                                                  \
    if (a.fa == FA && a.fb == FB)                                               \
        return a.out_bf16 ? launch_tile<BM, BN, FA, FB, true, BLOCK>(a)        \
                          : launch_tile<BM, BN, FA, FB, false, BLOCK>(a);
    FP8MI_FMT_CASE(0, 0)
    if constexpr (!BLOCK) {
        FP8MI_FMT_CASE(1, 0)
        FP8MI_FMT_CASE(0, 1)
        FP8MI_FMT_CASE(1, 1)
    }
#undef FP8MI_FMT_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scaled_gemm(const GemmArgs& a) {
    return dispatch_formats<256, 256, false>(a);
}

hipError_t launch_blockscaled_gemm(const GemmArgs& a) {
    return dispatch_formats<256, 128, true>(a);
}

}  // namespace fp8mi
