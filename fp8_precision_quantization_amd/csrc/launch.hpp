// launch.hpp -- internal host-side interface between the C-ABI layer
// (api.cpp) and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8mi.h"

namespace fp8mi {

struct QuantArgs {
    const void* x = nullptr;
    bool in_bf16 = true;
    int64_t rows = 0, cols = 0, ld = 0;
    int fmt = 0;                 // 0 = E4M3, 1 = E5M2
    int gran = 0;                // fp8_granularity
    bool pow2 = false;
    bool transpose = false;
    bool write_q = true;         // false: amax only (fp8_amax)
    bool guard = false;          // FP8_SPIKE_GUARD (delayed only)
    fp8_amax_history* hist = nullptr;
    uint8_t* q = nullptr;
    int64_t ldq = 0;
    uint8_t* q2 = nullptr;       // with transpose: the untransposed codes too (fp8_quantize_dual)
    int64_t ldq2 = 0;
    float* scale_inv = nullptr;
    float* amax = nullptr;
    fp8_diag* diag = nullptr;
    uint32_t* scratch = nullptr;  // the caller's workspace, kScratchWords words (per-tensor granularity)
    hipStream_t stream = nullptr;
    int num_cus = 256;
};

// fp8_quantize_tensors: just-in-time per-tensor quantization of up to
// FP8_MAX_TENSORS contiguous tensors in one amax launch and one cast launch.
struct MultiQuantArgs {
    int n = 0;
    bool in_bf16 = true;
    int fmt = 0;
    bool pow2 = false;
    const void* x[FP8_MAX_TENSORS] = {};
    int64_t elems[FP8_MAX_TENSORS] = {};
    uint8_t* q[FP8_MAX_TENSORS] = {};
    float* scale_inv[FP8_MAX_TENSORS] = {};
    float* amax[FP8_MAX_TENSORS] = {};
    fp8_diag* diag[FP8_MAX_TENSORS] = {};
    uint32_t* scratch = nullptr;
    hipStream_t stream = nullptr;
    int num_cus = 256;
};

struct GemmArgs {
    const uint8_t* A = nullptr;
    const uint8_t* B = nullptr;
    int fa = 0, fb = 0;
    int64_t lda = 0, ldb = 0;
    int64_t M = 0, N = 0, K = 0;
    const float* sa = nullptr;
    const float* sb = nullptr;
    bool sa_per_row = false, sb_per_row = false;
    void* C = nullptr;
    bool out_bf16 = true;
    int64_t ldc = 0;
    hipStream_t stream = nullptr;
    int num_cus = 256;
    // grouped GEMM: B holds `groups` expert matrices, b_group_stride elements
    // apart; group g is rows [group_offsets[g], group_offsets[g+1]) of A and C
    int groups = 0;
    const int32_t* group_offsets = nullptr;
    int64_t b_group_stride = 0;
    uint32_t* scratch = nullptr;
};

struct KvStoreArgs {
    const void* x = nullptr;
    bool in_bf16 = true;
    int64_t n_tokens = 0, ld = 0;
    int heads = 0, head_dim = 0;
    const int64_t* slots = nullptr;
    int64_t capacity = 0;
    int storage = 0;             // fp8_kv_storage
    bool per_head = false;       // FP8_KV_PER_HEAD
    bool pow2 = false;
    void* cache = nullptr;
    float* scale_inv = nullptr;
    fp8_diag* diag = nullptr;
    hipStream_t stream = nullptr;
};

struct KvLoadArgs {
    const void* cache = nullptr;
    int storage = 0;
    bool per_head = false;
    const float* scale_inv = nullptr;
    int64_t capacity = 0;
    int heads = 0, head_dim = 0;
    const int64_t* slots = nullptr;
    int64_t n_tokens = 0;
    bool out_bf16 = true;
    void* out = nullptr;
    int64_t ld_out = 0;
    hipStream_t stream = nullptr;
};

hipError_t launch_quantize(const QuantArgs& a);
hipError_t launch_quantize_multi(const MultiQuantArgs& a);
// Address on the current device of the workspace fp8_quantize_noalloc uses
// (a device array of kScratchWords words); taken once per device.
hipError_t static_workspace(uint32_t** out);
hipError_t launch_kv_store(const KvStoreArgs& a);
hipError_t launch_kv_load(const KvLoadArgs& a);
hipError_t launch_history_init(fp8_amax_history* h, int32_t len, hipStream_t stream);
hipError_t launch_history_set_guard(fp8_amax_history* h, float threshold, hipStream_t stream);
hipError_t launch_scaled_gemm(const GemmArgs& a);
hipError_t launch_blockscaled_gemm(const GemmArgs& a);
hipError_t launch_grouped_gemm(const GemmArgs& a);

// Words of the caller's workspace (FP8_WORKSPACE_BYTES / 4).
constexpr int kScratchWords = 16384;
// Words [kScratchGroupTable, kScratchWords) hold the grouped GEMM's table of
// 256-row tiles (a 4-word header, then 4 words per tile); the quantize
// kernels use the words below it.
constexpr int kScratchGroupTable = 8448;
constexpr int kGroupTableTiles = (kScratchWords - kScratchGroupTable - 4) / 4;

// Unit count of the element-wise tensor kernels must fit in 31 bits.
constexpr int64_t kMaxUnits = (int64_t(1) << 31) - 1;

}  // namespace fp8mi
