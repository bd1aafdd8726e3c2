/*
 * fp8mi.h -- C ABI of the MI355X (gfx950) FP8 scaled-quantization and
 * scaled-GEMM library (libfp8mi.so).
 *
 * The operations follow these web pages (cited by title, site and section):
 *   [DeepL] "DeepL bets on FP8: unified-precision training and inference"
 *           (hmyw.cn/news/121341): 2.1 format roles and bit splits, 2.2 cast of
 *           the high-precision master weights to FP8 before every GEMM, 2.3
 *           scaling factors at tensor / row / block granularity and delayed
 *           scaling from previous steps' statistics, 4.2 per-layer max-abs and
 *           scale diagnostics, 5.1 E5M2 gradient overflow, 5.3 FP8 GEMMs not
 *           bit-identical across tilings.
 *   [H100]  "H100 FP8 acceleration, measured" (scrxy.com/news/908489):
 *           paragraph on the FP8 formats (jointly defined formats, E5M2 range
 *           +-57344) and on FP8 matrix multiply-add in hardware.
 *   [Soup]  "FP8 training and QAT ... with Soup on Hopper GPUs"
 *           (lbrq.cn/news/198264): table of the tensorwise / rowwise (power-of-
 *           two scales) recipes; configuration errors rejected up front with
 *           an explicit message.
 *   [Swift] "FP8 quantization support in ms-swift" (maplevalley.com.cn/news/
 *           598486): E4M3 / E5M2 and the dynamic per-tensor method.
 *   [DeepL] 3.1 also: the FP8 KV cache (half of BF16's memory) and the one
 *           layer whose K cache stayed in BF16; 3.2: MoE's grouped GEMM.
 *
 * Conventions for every entry point:
 *   - All pointers except the ones documented as host pointers are DEVICE
 *     pointers on the current HIP device.  The caller owns every buffer:
 *     inputs, outputs, scale arrays, histories, counters and the workspace
 *     of the calls that need one.  The library never allocates, frees or
 *     synchronizes.
 *   - Workspace: the per-tensor reductions of fp8_amax / fp8_quantize /
 *     fp8_quantize_dual (FP8_GRAN_TENSOR) / fp8_quantize_tensors and the
 *     grouped GEMM's tile table need `workspace`, device memory of at least
 *     fp8_workspace_size() bytes, 16-byte aligned (else FP8_ERR_INVALID_ARG
 *     / FP8_ERR_MISALIGNED).  It needs no initialization and holds nothing
 *     the caller reads; a call owns it from launch until its kernels
 *     finish, so calls in flight at the same time (different streams) need
 *     different workspaces, while calls ordered on one stream can share one.
 *     Calls that do not need it accept NULL.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call is asynchronous: it returns after host-side validation and
 *     the kernel launches.  A fault inside a kernel surfaces at the caller's
 *     next synchronization.
 *   - Validation runs before any launch.  On any error nothing is launched
 *     and no output is touched; fp8_last_error() returns a message that names
 *     the offending argument (thread-local, valid until the next call).
 *   - Only gfx950 is supported; any other device gives
 *     FP8_ERR_UNSUPPORTED_DEVICE.
 *   - Matrices are row-major with an explicit leading dimension (elements
 *     between consecutive rows, >= the number of columns).
 *   - Scale convention: dequantized value = decode(q) * scale_inv.
 *   - Reentrant; the only global state is a per-device architecture cache
 *     and the kernels' per-device launch attributes.
 */
#ifndef FP8MI_H
#define FP8MI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8MI_ABI_VERSION 7

typedef enum {
    FP8_OK = 0,
    FP8_ERR_INVALID_ARG = 1,        /* bad enum, NULL pointer, size <= 0, ld < cols, bad flags */
    FP8_ERR_UNSUPPORTED_SHAPE = 2,  /* shape the operation does not support (e.g. K % 16 != 0) */
    FP8_ERR_MISALIGNED = 3,         /* pointer or leading dimension misaligned */
    FP8_ERR_UNSUPPORTED_DEVICE = 4, /* current device is not gfx950 */
    FP8_ERR_HIP = 5                 /* a HIP runtime call or launch failed */
} fp8_status;

/* [DeepL] 2.1: E4M3 (1/4/3 bits) for forward weights and activations, E5M2
 * (1/5/2 bits) for gradients.  Both are the OCP formats ([H100], formats
 * paragraph): E4M3 has no infinities, max finite 448, NaN = S.1111.111;
 * E5M2 has IEEE-style Inf/NaN, max finite 57344. */
typedef enum { FP8_E4M3 = 0, FP8_E5M2 = 1 } fp8_format;

typedef enum { FP8_IN_F32 = 0, FP8_IN_BF16 = 1 } fp8_in_dtype;
typedef enum { FP8_OUT_F32 = 0, FP8_OUT_BF16 = 1 } fp8_out_dtype;

/* [DeepL] 2.3: one factor per tensor, per row, or per block.  Blocks are
 * 1x128 (one row, 128 consecutive columns) or 128x128, aligned at (0,0); a
 * final partial block covers the remainder.  Group grids (row-major):
 *   TENSOR: 1;  ROW: rows;  BLOCK_1x128: rows x ceil(cols/128);
 *   BLOCK_128x128: ceil(rows/128) x ceil(cols/128). */
typedef enum {
    FP8_GRAN_TENSOR = 0,
    FP8_GRAN_ROW = 1,
    FP8_GRAN_BLOCK_1x128 = 2,
    FP8_GRAN_BLOCK_128x128 = 3
} fp8_granularity;

/* [Soup] rowwise recipe: round every scale down to a power of two
 * (s = 2^floor(log2(448/amax)), so scale_inv is exact). */
#define FP8_SCALE_POW2 1u
/* Write q transposed: q is [cols x rows] with leading dimension ldq >= rows.
 * Only with FP8_GRAN_TENSOR (the wgrad operands X^T and dY^T). */
#define FP8_TRANSPOSE_OUT 2u
/* Spike guard for delayed scaling ([DeepL] 2.3: the delayed scale lags a
 * sudden change of the distribution; compare the current statistic with the
 * history and recompute the scale past a threshold).  Needs hist.  When this
 * step's amax exceeds hist->spike_threshold x the window max (an fp32
 * product; never with an empty window or a threshold <= 0), the tensor is
 * cast again just in time, with s = fmax / amax (FP8_SCALE_POW2 applies),
 * scale_inv_out holds that scale's inverse, diag counts that cast only and
 * hist->spikes grows by one.  The ring is updated as without the guard. */
#define FP8_SPIKE_GUARD 4u

/* Data-dependent conditions are counted on the device, never returned as a
 * status ([DeepL] 4.2 and 6.2: watch max-abs, scale and overflow).  Device
 * memory; the library ADDS to the counters, so the caller zeroes them.
 *   sat_count:        non-NaN products |x*s| > max finite (saturated, Inf incl.)
 *   nonfinite_count:  NaN or Inf inputs
 *   underflow_count:  nonzero, non-NaN inputs whose code is +-0 */
typedef struct fp8_diag {
    uint32_t sat_count;
    uint32_t nonfinite_count;
    uint32_t underflow_count;
    uint32_t reserved;
} fp8_diag;

/* Delayed scaling ([DeepL] 2.3): this step's scale comes from the raw amax of
 * the previous min(count, len) steps: s = fmax / max(history).  The current
 * step is excluded; with an empty history the call scales just in time from
 * the current amax.  After the cast the current amax enters the ring.
 * Device memory, 128 bytes, caller-owned; initialize with
 * fp8_history_init().  Saving and restoring the 128 bytes (a device copy)
 * checkpoints the state.  `scale`/`scale_inv` hold the scale the NEXT call
 * will use (for inspection).  Calls sharing one history must be ordered on
 * one stream.  A delayed call is the cast and a one-workgroup finish that
 * pushes the ring; on an empty history the cast's workgroups share the
 * just-in-time amax through `sync`, which the finish clears (a call cut
 * short by a device fault can leave it non-zero: fp8_history_init, or
 * restoring a checkpoint taken between calls, clears it). */
typedef struct fp8_amax_history {
    float amax[16];         /* raw amax of past steps; slot `pos` is written next */
    int32_t len;            /* window length, 1..16 */
    int32_t pos;            /* next slot to write */
    int32_t count;          /* valid entries, 0..len */
    uint32_t internal[2];   /* last guarded call: 1 if it cast again, and that scale's bits */
    float scale;            /* scale the next call will use (count > 0) */
    float scale_inv;
    uint32_t steps;         /* calls completed */
    float spike_threshold;  /* FP8_SPIKE_GUARD threshold, 0 after fp8_history_init (off) */
    uint32_t spikes;        /* guarded calls that cast again */
    uint32_t sync[3];       /* used by the kernels during a call; zero between calls */
    uint32_t reserved[3];
} fp8_amax_history;

/* Library version of this header (FP8MI_ABI_VERSION). */
int fp8_abi_version(void);

/* Static description of a status code. */
const char* fp8_status_string(fp8_status status);

/* Thread-local message for the last error returned on this thread ("" after
 * a successful call). */
const char* fp8_last_error(void);

/* Bytes of the workspace the per-tensor quantize / amax calls and the
 * grouped GEMM take (FP8_WORKSPACE_BYTES: 64 KiB).  Words of it carry one
 * partial maximum per workgroup of a reduction pass (combined by the next
 * kernel instead of by same-address atomics), the first pass's counters of
 * a guarded delayed cast, and the grouped GEMM's table of row tiles. */
#define FP8_WORKSPACE_BYTES 65536
int64_t fp8_workspace_size(void);

/* Zero a history and set its window length (1..16) on `stream`. */
fp8_status fp8_history_init(fp8_amax_history* hist, int32_t len, void* stream);

/* Set the spike threshold of a history on `stream` (see FP8_SPIKE_GUARD;
 * the pages give no value: a ratio such as 10 is the caller's choice). */
fp8_status fp8_history_set_guard(fp8_amax_history* hist, float threshold, void* stream);

/* amax = max |x| per group ([DeepL] 4.2: the per-layer maximum absolute value
 * behind the scale).  x: [rows x cols], element type in_dtype, leading
 * dimension ld.  amax_out: fp32 array of the group grid (see
 * fp8_granularity).  A NaN anywhere in a group gives NaN, else an Inf gives
 * Inf.  Any pointer alignment is accepted; 16-byte-aligned rows are fastest. */
fp8_status fp8_amax(const void* x, fp8_in_dtype in_dtype, int64_t rows, int64_t cols, int64_t ld,
                    fp8_granularity gran, float* amax_out, void* workspace, int64_t workspace_bytes,
                    void* stream);

/* Scaled quantization ([DeepL] 2.1, 2.3; [Soup] recipes; [Swift] dynamic
 * per-tensor):
 *   per group:  amax, s = fl32(fmax / amax) (amax = 0 or non-finite -> 1,
 *               overflow -> FLT_MAX; FP8_SCALE_POW2 truncates s to a power
 *               of two), s_inv = fl32(1 / s);
 *   per element: q = saturating round-to-nearest-even of fl32(x * s) into
 *               `fmt`; NaN -> 0x7F|sign; the sign survives underflow.
 * x: [rows x cols] (ld).  q: uint8 codes [rows x cols] (ldq >= cols), or
 * [cols x rows] (ldq >= rows) with FP8_TRANSPOSE_OUT.
 * scale_inv_out, amax_out: fp32 arrays of the group grid, both required.
 * hist: NULL = just in time; non-NULL = delayed scaling (FP8_GRAN_TENSOR
 * only); amax_out then receives the current step's amax and scale_inv_out
 * the inverse of the scale actually used.
 * diag: optional counters (NULL to skip the counting).
 * workspace: needed with FP8_GRAN_TENSOR (see the conventions above). */
fp8_status fp8_quantize(const void* x, fp8_in_dtype in_dtype, int64_t rows, int64_t cols,
                        int64_t ld, fp8_format fmt, fp8_granularity gran, uint32_t flags,
                        fp8_amax_history* hist, uint8_t* q, int64_t ldq, float* scale_inv_out,
                        float* amax_out, fp8_diag* diag, void* workspace, int64_t workspace_bytes,
                        void* stream);

/* fp8_quantize for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments and results without the workspace, which is a 64 KiB array in
 * device memory that the library holds, one per device, from the first call
 * on that device until the process ends (that first call looks up its
 * address).  The call itself allocates nothing.  Every call on a device
 * shares that device's array, so calls that can overlap on one device (on
 * different streams, or from different threads) race and must not be
 * issued; calls ordered on one stream are fine.  The array's use does not
 * grow with the tensor (per-workgroup partial maxima of at most 4096 + 1024
 * workgroups and 4 counter words, all below word 8196 of its 16384), so
 * every size fp8_quantize accepts is accepted here, every other is rejected
 * by the same checks with the same messages, and nothing of it needs
 * clearing by the caller. */
fp8_status fp8_quantize_noalloc(const void* x, fp8_in_dtype in_dtype, int64_t rows, int64_t cols,
                                int64_t ld, fp8_format fmt, fp8_granularity gran, uint32_t flags,
                                fp8_amax_history* hist, uint8_t* q, int64_t ldq, float* scale_inv_out,
                                float* amax_out, fp8_diag* diag, void* stream);

/* Per-tensor quantization with both layouts from one pass over x: q
 * [rows x cols] (ldq >= cols) and qt [cols x rows] (ldqt >= rows), the same
 * codes.  A gradient feeds the data-gradient GEMM as dY and the weight-
 * gradient GEMM as dY^T, both in E5M2 ([DeepL] 2.1), so one read of dY gives
 * both operands.  Arguments and rules as fp8_quantize with FP8_GRAN_TENSOR;
 * flags: FP8_SCALE_POW2, FP8_SPIKE_GUARD.  workspace: required. */
fp8_status fp8_quantize_dual(const void* x, fp8_in_dtype in_dtype, int64_t rows, int64_t cols, int64_t ld,
                             fp8_format fmt, uint32_t flags, fp8_amax_history* hist, uint8_t* q, int64_t ldq,
                             uint8_t* qt, int64_t ldqt, float* scale_inv_out, float* amax_out, fp8_diag* diag,
                             void* workspace, int64_t workspace_bytes, void* stream);

/* One tensor of fp8_quantize_tensors (a host-side descriptor; its pointers
 * are device pointers).  x: [rows x cols] contiguous (no leading dimension),
 * 16-byte aligned.  q: [rows x cols] uint8 codes, contiguous, 8-byte
 * aligned.  scale_inv, amax: one fp32 each (4-byte aligned).  diag: optional
 * counters (NULL to skip), as fp8_quantize. */
typedef struct fp8_tensor {
    const void* x;
    int64_t rows;
    int64_t cols;
    uint8_t* q;
    float* scale_inv;
    float* amax;
    fp8_diag* diag;
} fp8_tensor;

#define FP8_MAX_TENSORS 8

/* Just-in-time per-tensor quantization of up to FP8_MAX_TENSORS tensors in
 * two launches, whatever their number: one amax pass over all of them, then
 * one cast pass.  A GEMM's operands are cast to FP8 together before it
 * ([DeepL] 2.2; [Swift] dynamic per-tensor), each with its own factor
 * ([DeepL] 2.3, tensor granularity), so the activation and the weight of a
 * layer can share the launches.  Each tensor's amax, scale_inv and codes
 * are those fp8_quantize gives it with FP8_GRAN_TENSOR and no history, bit
 * for bit.
 * tensors: HOST array of `count` descriptors (1..FP8_MAX_TENSORS), read
 * during the call only.  All tensors share in_dtype and fmt; flags:
 * FP8_SCALE_POW2 only.  Tensors may be empty (amax 0, scale_inv 1).  Each
 * tensor's outputs must not overlap any input or another tensor's outputs.
 * workspace: required (see the conventions above).  Errors name the tensor
 * by its index. */
fp8_status fp8_quantize_tensors(const fp8_tensor* tensors, int32_t count, fp8_in_dtype in_dtype, fp8_format fmt,
                                uint32_t flags, void* workspace, int64_t workspace_bytes, void* stream);

/* Scaled FP8 GEMM ([H100] FP8 matrix multiply-add in hardware; [Soup]
 * tensorwise and rowwise GEMMs; [DeepL] 2.2 results return to high
 * precision):
 *   C[m,n] = (sum_k decode(A[m,k]) * decode(B[n,k])) * fl32(sa(m) * sb(n))
 * accumulated in fp32 on the FP8 matrix cores, i.e. C = A_hat . B_hat^T with
 * both operands K-contiguous (Y = X W^T; the wgrad dW = dY^T X takes the
 * transposed casts of dY and X).  A: uint8 [M x K] codes of format fa (lda);
 * B: uint8 [N x K] codes of format fb (ldb).  sa = a_scale_inv[0] if
 * a_per_row == 0, else a_scale_inv[m] ([M]); likewise sb with [N].
 * C: [M x N] fp32 or bf16 (round-to-nearest-even), leading dimension ldc.
 * Requirements: K % 16 == 0; A, B 16-byte aligned; lda, ldb multiples of 16
 * and <= 2^23; C aligned to its element size.  Results are bit-reproducible run to run
 * (no split-K, no atomics).  Every output's K sum is the same sequence of
 * matrix-core operations whatever M and N are and however the call splits
 * into launches (256- or 128-row tiles), so an output's bits do not depend
 * on the rest of the problem; they may differ from another library's
 * tiling in the last bits of the fp32 sum ([DeepL] 5.3). */
fp8_status fp8_scaled_gemm(const uint8_t* A, fp8_format fa, int64_t lda,
                           const uint8_t* B, fp8_format fb, int64_t ldb,
                           int64_t M, int64_t N, int64_t K,
                           const float* a_scale_inv, int a_per_row,
                           const float* b_scale_inv, int b_per_row,
                           void* C, fp8_out_dtype out_dtype, int64_t ldc, void* stream);

/* Block-scaled FP8 GEMM ([DeepL] 2.3, per-block scaling): E4M3 operands,
 * A with one scale per (row, 128-wide K block), B with one per (128x128
 * block):
 *   C[m,n] = sum_kb  fl32(a_scale_inv[m, kb] * b_scale_inv[n/128, kb])
 *                    * (sum_{k in kb} decode(A[m,k]) * decode(B[n,k]))
 * Each K block's partial sum is formed in fp32 on the matrix cores and then
 * promoted into the fp32 accumulator with its scale product.
 * a_scale_inv: [M x K/128] row-major; b_scale_inv: [N/128 x K/128].
 * Requirements: K % 128 == 0 and N % 128 == 0 (else
 * FP8_ERR_UNSUPPORTED_SHAPE); alignment as fp8_scaled_gemm. */
fp8_status fp8_blockscaled_gemm(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb,
                                int64_t M, int64_t N, int64_t K,
                                const float* a_scale_inv, const float* b_scale_inv,
                                void* C, fp8_out_dtype out_dtype, int64_t ldc, void* stream);

/* Grouped scaled FP8 GEMM for mixture-of-experts layers ([DeepL] 3.2: each
 * token activates a few experts, so the batch's tokens are grouped by their
 * routing and every group is multiplied with its own expert's weight; FP8
 * halves the expert weights).  For every row m of group g, i.e.
 * group_offsets[g] <= m < group_offsets[g+1]:
 *   C[m,n] = (sum_k decode(A[m,k]) * decode(B_g[n,k])) * fl32(sa(m) * sb_g(n))
 * with the arithmetic of fp8_scaled_gemm.  A: uint8 [M x K] codes of format
 * fa (lda), the tokens sorted by group.  B: `groups` expert matrices, each
 * uint8 [N x K] of format fb with row stride ldb, expert g at
 * B + g * b_group_stride (b_group_stride >= (N-1)*ldb + K, a multiple of 16).
 * group_offsets: DEVICE int32 [groups + 1], non-decreasing, within [0, M]
 * (read on the device: out-of-range offsets are clamped, and decreasing ones
 * leave the overlapping rows' values unspecified, never an out-of-range
 * access).  Rows in no group are not written.  sa = a_scale_inv[0]
 * (a_per_row == 0) or a_scale_inv[m] ([M]); sb_g(n) = b_scale_inv[g]
 * (b_per_row == 0, one scale per expert, [groups]) or b_scale_inv[g*N + n]
 * ([groups x N]).  C: [M x N] fp32 or bf16, leading dimension ldc.
 * Requirements as fp8_scaled_gemm, plus groups >= 1 and
 * ceil(M / 256) + groups <= FP8_GROUPED_MAX_TILES (the size of the table of
 * 256-row tiles the call builds in the workspace, which is required), else
 * FP8_ERR_UNSUPPORTED_SHAPE. */
#define FP8_GROUPED_MAX_TILES 1983
fp8_status fp8_grouped_gemm(const uint8_t* A, fp8_format fa, int64_t lda,
                            const uint8_t* B, fp8_format fb, int64_t ldb, int64_t b_group_stride,
                            int64_t M, int64_t N, int64_t K, int32_t groups, const int32_t* group_offsets,
                            const float* a_scale_inv, int a_per_row,
                            const float* b_scale_inv, int b_per_row,
                            void* C, fp8_out_dtype out_dtype, int64_t ldc,
                            void* workspace, int64_t workspace_bytes, void* stream);

/* FP8 KV cache ([DeepL] 3.1: K and V caches held in FP8 take half of BF16's
 * memory; K's precision drives the attention scores, V's the mixed output;
 * keeping one layer's K cache in BF16 removed a long-sequence error, so the
 * storage is chosen per layer and per tensor).
 *
 * One layer's K (or V) cache: `cache` [capacity x heads x head_dim], head_dim
 * contiguous -- uint8 codes (FP8_KV_E4M3 / FP8_KV_E5M2) or bf16 values
 * (FP8_KV_BF16, the fallback).  Scales (FP8 storage only), dequantized value
 * = decode(q) * scale_inv:
 *   FP8_KV_PER_TOKEN_HEAD: scale_inv [capacity x heads] fp32, written by
 *     fp8_kv_store: each (token, head) vector of head_dim values is one group
 *     of the row rule of fp8_quantize (amax, s = fl32(fmax / amax),
 *     FP8_SCALE_POW2 applies, s_inv = fl32(1 / s));
 *   FP8_KV_PER_HEAD: scale_inv [heads] fp32, fixed (calibrated) by the
 *     caller and only read: the cast multiplies by s = fl32(1 / scale_inv[h]),
 *     saturating what falls outside.  Entries must be finite and > 0.
 * Token placement: new token t goes to cache row slots[t] (device int64
 * array of n_tokens; NULL = row t); a slot outside [0, capacity) is padding
 * and is skipped.  Two new tokens with one slot race.
 * Requirements (else FP8_ERR_UNSUPPORTED_SHAPE / FP8_ERR_MISALIGNED):
 * head_dim % 8 == 0 and 8 <= head_dim <= 2048; n_tokens * heads < 2^31;
 * x, cache and out 16-byte aligned; ld and ld_out multiples of 8. */
typedef enum { FP8_KV_E4M3 = 0, FP8_KV_E5M2 = 1, FP8_KV_BF16 = 2 } fp8_kv_storage;
typedef enum { FP8_KV_PER_TOKEN_HEAD = 0, FP8_KV_PER_HEAD = 1 } fp8_kv_scaling;

/* Store n_tokens new vectors: x [n_tokens x (heads*head_dim)] (ld >=
 * heads*head_dim elements between tokens; head h of token t at
 * x + t*ld + h*head_dim), fp32 or bf16.  BF16 storage rounds fp32 input to
 * nearest even and copies bf16 input.  flags: FP8_SCALE_POW2 (per token-head
 * scales only).  diag: optional counters of the FP8 cast (as fp8_quantize). */
fp8_status fp8_kv_store(const void* x, fp8_in_dtype in_dtype, int64_t n_tokens, int64_t ld,
                        int32_t heads, int32_t head_dim, const int64_t* slots,
                        fp8_kv_storage storage, fp8_kv_scaling scaling, uint32_t flags,
                        void* cache, float* scale_inv, int64_t capacity, fp8_diag* diag,
                        void* stream);

/* Gather n_tokens cache rows (slots[t], NULL = row t) and dequantize them:
 * out row t [heads*head_dim] at out + t*ld_out (ld_out >= heads*head_dim),
 * y = fl32(decode(q) * scale_inv) as fp32 or rounded to bf16 (nearest even);
 * a BF16 cache returns its values.  Padding slots leave their out row
 * untouched. */
fp8_status fp8_kv_load(const void* cache, fp8_kv_storage storage, fp8_kv_scaling scaling,
                       const float* scale_inv, int64_t capacity, int32_t heads, int32_t head_dim,
                       const int64_t* slots, int64_t n_tokens, fp8_out_dtype out_dtype, void* out,
                       int64_t ld_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8MI_H */
