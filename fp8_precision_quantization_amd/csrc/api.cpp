// api.cpp -- the C ABI of libfp8mi.so: argument validation, device check and
// dispatch to the gfx950 kernels.  Every invalid combination is rejected
// before anything is launched, with a message naming the argument (the
// up-front rejection convention of [Soup, lbrq.cn], list of configuration
// errors caught at load time, including the explicit "needs hardware X").
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "fp8mi.h"
#include "launch.hpp"

namespace {

thread_local std::string g_last_error;

fp8_status fail(fp8_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

fp8_status ok() {
    g_last_error.clear();
    return FP8_OK;
}

struct DeviceInfo {
    std::atomic<int> state{0};   // 0 unknown, 1 gfx950, 2 other
    int num_cus = 0;
    char arch[64] = {0};
};

constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_dev_mutex;

// Current device must be gfx950; returns its CU count through *cus.
fp8_status check_device(int* cus) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FP8_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(FP8_ERR_UNSUPPORTED_DEVICE, "device index %d out of range", dev);
    DeviceInfo& d = g_devices[dev];
    if (d.state.load(std::memory_order_acquire) == 0) {
        std::lock_guard<std::mutex> lock(g_dev_mutex);
        if (d.state.load(std::memory_order_relaxed) == 0) {
            hipDeviceProp_t prop;
            e = hipGetDeviceProperties(&prop, dev);
            if (e != hipSuccess)
                return fail(FP8_ERR_HIP, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
            std::strncpy(d.arch, prop.gcnArchName, sizeof(d.arch) - 1);
            d.num_cus = prop.multiProcessorCount;
            const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            d.state.store(is950 ? 1 : 2, std::memory_order_release);
        }
    }
    if (d.state.load(std::memory_order_acquire) != 1)
        return fail(FP8_ERR_UNSUPPORTED_DEVICE,
                    "device %d is %s; this library needs gfx950 (MI355X / MI350X): FP8 MFMA and OCP FP8 conversion",
                    dev, d.arch);
    *cus = d.num_cus;
    return FP8_OK;
}

// The caller's workspace: needed by the per-tensor reductions and the grouped
// GEMM's tile table, optional elsewhere.
fp8_status check_workspace(bool needed, void* ws, int64_t bytes, uint32_t** out) {
    *out = static_cast<uint32_t*>(ws);
    if (!needed) return FP8_OK;
    if (ws == nullptr) return fail(FP8_ERR_INVALID_ARG, "workspace is NULL (this call needs fp8_workspace_size() bytes)");
    if (bytes < FP8_WORKSPACE_BYTES)
        return fail(FP8_ERR_INVALID_ARG, "workspace_bytes=%lld is below fp8_workspace_size()=%d", (long long)bytes,
                    FP8_WORKSPACE_BYTES);
    if ((uintptr_t)ws % 16 != 0) return fail(FP8_ERR_MISALIGNED, "workspace must be 16-byte aligned");
    return FP8_OK;
}

fp8_status launch_result(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FP8_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

bool is_aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

fp8_status check_matrix_in(const void* x, int in_dtype, int64_t rows, int64_t cols, int64_t ld) {
    if (x == nullptr && rows > 0 && cols > 0) return fail(FP8_ERR_INVALID_ARG, "x is NULL");
    if (in_dtype != FP8_IN_F32 && in_dtype != FP8_IN_BF16)
        return fail(FP8_ERR_INVALID_ARG, "in_dtype %d is not FP8_IN_F32 or FP8_IN_BF16", in_dtype);
    if (rows < 0 || cols < 0) return fail(FP8_ERR_INVALID_ARG, "negative size rows=%lld cols=%lld",
                                          (long long)rows, (long long)cols);
    if (ld < cols || ld < 1) return fail(FP8_ERR_INVALID_ARG, "ld=%lld must be >= max(cols, 1)=%lld",
                                         (long long)ld, (long long)(cols > 1 ? cols : 1));
    const int esz = in_dtype == FP8_IN_F32 ? 4 : 2;
    if (!is_aligned(x, esz)) return fail(FP8_ERR_MISALIGNED, "x is not aligned to its %d-byte element", esz);
    if (rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "rows and cols must each be <= 2^31");
    if ((rows * ((cols + 7) / 8)) > fp8mi::kMaxUnits)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "tensor too large: more than 2^34 elements");
    return FP8_OK;
}

bool valid_gran(int g) {
    return g == FP8_GRAN_TENSOR || g == FP8_GRAN_ROW || g == FP8_GRAN_BLOCK_1x128 ||
           g == FP8_GRAN_BLOCK_128x128;
}

int64_t num_groups(int gran, int64_t rows, int64_t cols) {
    switch (gran) {
    case FP8_GRAN_TENSOR: return 1;
    case FP8_GRAN_ROW: return rows;
    case FP8_GRAN_BLOCK_1x128: return rows * ((cols + 127) / 128);
    default: return ((rows + 127) / 128) * ((cols + 127) / 128);
    }
}

}  // namespace

extern "C" {

int fp8_abi_version(void) { return FP8MI_ABI_VERSION; }

const char* fp8_status_string(fp8_status s) {
    switch (s) {
    case FP8_OK: return "FP8_OK";
    case FP8_ERR_INVALID_ARG: return "FP8_ERR_INVALID_ARG";
    case FP8_ERR_UNSUPPORTED_SHAPE: return "FP8_ERR_UNSUPPORTED_SHAPE";
    case FP8_ERR_MISALIGNED: return "FP8_ERR_MISALIGNED";
    case FP8_ERR_UNSUPPORTED_DEVICE: return "FP8_ERR_UNSUPPORTED_DEVICE";
    case FP8_ERR_HIP: return "FP8_ERR_HIP";
    }
    return "FP8_ERR_UNKNOWN";
}

const char* fp8_last_error(void) { return g_last_error.c_str(); }

int64_t fp8_workspace_size(void) { return FP8_WORKSPACE_BYTES; }

fp8_status fp8_history_init(fp8_amax_history* hist, int32_t len, void* stream) {
    if (hist == nullptr) return fail(FP8_ERR_INVALID_ARG, "hist is NULL");
    if (len < 1 || len > 16) return fail(FP8_ERR_INVALID_ARG, "history length %d not in 1..16", len);
    if (!is_aligned(hist, 16)) return fail(FP8_ERR_MISALIGNED, "hist must be 16-byte aligned");
    int cus = 0;
    fp8_status st = check_device(&cus);
    if (st != FP8_OK) return st;
    return launch_result(fp8mi::launch_history_init(hist, len, (hipStream_t)stream), "fp8_history_init");
}

fp8_status fp8_history_set_guard(fp8_amax_history* hist, float threshold, void* stream) {
    if (hist == nullptr) return fail(FP8_ERR_INVALID_ARG, "hist is NULL");
    if (!is_aligned(hist, 16)) return fail(FP8_ERR_MISALIGNED, "hist must be 16-byte aligned");
    int cus = 0;
    fp8_status st = check_device(&cus);
    if (st != FP8_OK) return st;
    return launch_result(fp8mi::launch_history_set_guard(hist, threshold, (hipStream_t)stream),
                         "fp8_history_set_guard");
}

fp8_status fp8_amax(const void* x, fp8_in_dtype in_dtype, int64_t rows, int64_t cols, int64_t ld,
                    fp8_granularity gran, float* amax_out, void* workspace, int64_t workspace_bytes,
                    void* stream) {
    fp8_status st = check_matrix_in(x, in_dtype, rows, cols, ld);
    if (st != FP8_OK) return st;
    if (!valid_gran(gran)) return fail(FP8_ERR_INVALID_ARG, "granularity %d is not a fp8_granularity", (int)gran);
    if (amax_out == nullptr && num_groups(gran, rows, cols) > 0)
        return fail(FP8_ERR_INVALID_ARG, "amax_out is NULL");
    if (!is_aligned(amax_out, 4)) return fail(FP8_ERR_MISALIGNED, "amax_out is not 4-byte aligned");
    uint32_t* scratch = nullptr;
    st = check_workspace(gran == FP8_GRAN_TENSOR, workspace, workspace_bytes, &scratch);
    if (st != FP8_OK) return st;
    int cus = 0;
    st = check_device(&cus);
    if (st != FP8_OK) return st;
    if (num_groups(gran, rows, cols) == 0) return ok();
    fp8mi::QuantArgs a;
    a.x = x; a.in_bf16 = in_dtype == FP8_IN_BF16; a.rows = rows; a.cols = cols; a.ld = ld;
    a.gran = gran; a.write_q = false; a.amax = amax_out; a.ldq = cols; a.scratch = scratch;
    a.stream = (hipStream_t)stream; a.num_cus = cus;
    return launch_result(fp8mi::launch_quantize(a), "fp8_amax");
}

// fp8_quantize and fp8_quantize_dual (qt != nullptr: q untransposed plus qt
// transposed, per tensor).
static fp8_status quantize_impl(const char* what, const void* x, fp8_in_dtype in_dtype, int64_t rows, int64_t cols,
                                int64_t ld, fp8_format fmt, fp8_granularity gran, uint32_t flags,
                                fp8_amax_history* hist, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                                bool dual, float* scale_inv_out, float* amax_out, fp8_diag* diag,
                                void* workspace, int64_t workspace_bytes, void* stream) {
    fp8_status st = check_matrix_in(x, in_dtype, rows, cols, ld);
    if (st != FP8_OK) return st;
    if (fmt != FP8_E4M3 && fmt != FP8_E5M2)
        return fail(FP8_ERR_INVALID_ARG, "format %d is not FP8_E4M3 or FP8_E5M2", (int)fmt);
    if (!valid_gran(gran)) return fail(FP8_ERR_INVALID_ARG, "granularity %d is not a fp8_granularity", (int)gran);
    const uint32_t known = FP8_SCALE_POW2 | FP8_SPIKE_GUARD | (dual ? 0u : FP8_TRANSPOSE_OUT);
    if (flags & ~known) return fail(FP8_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags & ~known);
    if ((flags & FP8_SPIKE_GUARD) && hist == nullptr)
        return fail(FP8_ERR_INVALID_ARG, "FP8_SPIKE_GUARD needs delayed scaling (hist != NULL)");
    const bool transpose = dual || (flags & FP8_TRANSPOSE_OUT) != 0;
    if (transpose && !dual && gran != FP8_GRAN_TENSOR)
        return fail(FP8_ERR_INVALID_ARG, "FP8_TRANSPOSE_OUT needs FP8_GRAN_TENSOR");
    if (hist != nullptr && gran != FP8_GRAN_TENSOR)
        return fail(FP8_ERR_INVALID_ARG, "delayed scaling (hist != NULL) needs FP8_GRAN_TENSOR");
    if (hist != nullptr && !is_aligned(hist, 16)) return fail(FP8_ERR_MISALIGNED, "hist must be 16-byte aligned");
    if (q == nullptr && rows > 0 && cols > 0) return fail(FP8_ERR_INVALID_ARG, "q is NULL");
    if (dual) {
        if (qt == nullptr && rows > 0 && cols > 0) return fail(FP8_ERR_INVALID_ARG, "qt is NULL");
        if (ldq < cols || ldq < 1)
            return fail(FP8_ERR_INVALID_ARG, "ldq=%lld must be >= cols=%lld", (long long)ldq, (long long)cols);
        if (ldqt < rows || ldqt < 1)
            return fail(FP8_ERR_INVALID_ARG, "ldqt=%lld must be >= rows=%lld", (long long)ldqt, (long long)rows);
    } else {
        const int64_t qcols = transpose ? rows : cols;
        if (ldq < qcols || ldq < 1)
            return fail(FP8_ERR_INVALID_ARG, "ldq=%lld must be >= %s=%lld", (long long)ldq,
                        transpose ? "rows (transposed output)" : "cols", (long long)qcols);
    }
    const int64_t ng = num_groups(gran, rows, cols);
    if (scale_inv_out == nullptr && ng > 0) return fail(FP8_ERR_INVALID_ARG, "scale_inv_out is NULL");
    if (amax_out == nullptr && ng > 0) return fail(FP8_ERR_INVALID_ARG, "amax_out is NULL");
    if (!is_aligned(scale_inv_out, 4) || !is_aligned(amax_out, 4))
        return fail(FP8_ERR_MISALIGNED, "scale_inv_out and amax_out must be 4-byte aligned");
    if (diag != nullptr && !is_aligned(diag, 4)) return fail(FP8_ERR_MISALIGNED, "diag must be 4-byte aligned");
    uint32_t* scratch = nullptr;
    st = check_workspace(gran == FP8_GRAN_TENSOR, workspace, workspace_bytes, &scratch);
    if (st != FP8_OK) return st;
    int cus = 0;
    st = check_device(&cus);
    if (st != FP8_OK) return st;
    if (num_groups(gran, rows, cols) == 0) return ok();
    fp8mi::QuantArgs a;
    a.scratch = scratch;
    a.x = x; a.in_bf16 = in_dtype == FP8_IN_BF16; a.rows = rows; a.cols = cols; a.ld = ld;
    a.fmt = fmt; a.gran = gran; a.pow2 = (flags & FP8_SCALE_POW2) != 0; a.transpose = transpose;
    a.write_q = true; a.hist = hist; a.guard = (flags & FP8_SPIKE_GUARD) != 0;
    if (dual) {   // the kernel's main output is the transposed one
        a.q = qt; a.ldq = ldqt; a.q2 = q; a.ldq2 = ldq;
    } else {
        a.q = q; a.ldq = ldq;
    }
    a.scale_inv = scale_inv_out;
    a.amax = amax_out; a.diag = diag; a.stream = (hipStream_t)stream; a.num_cus = cus;
    return launch_result(fp8mi::launch_quantize(a), what);
}

fp8_status fp8_quantize(const void* x, fp8_in_dtype in_dtype, int64_t rows, int64_t cols, int64_t ld,
                        fp8_format fmt, fp8_granularity gran, uint32_t flags, fp8_amax_history* hist,
                        uint8_t* q, int64_t ldq, float* scale_inv_out, float* amax_out, fp8_diag* diag,
                        void* workspace, int64_t workspace_bytes, void* stream) {
    return quantize_impl("fp8_quantize", x, in_dtype, rows, cols, ld, fmt, gran, flags, hist, q, ldq, nullptr, 0,
                         false, scale_inv_out, amax_out, diag, workspace, workspace_bytes, stream);
}

fp8_status fp8_quantize_noalloc(const void* x, fp8_in_dtype in_dtype, int64_t rows, int64_t cols, int64_t ld,
                                fp8_format fmt, fp8_granularity gran, uint32_t flags, fp8_amax_history* hist,
                                uint8_t* q, int64_t ldq, float* scale_inv_out, float* amax_out, fp8_diag* diag,
                                void* stream) {
    int cus = 0;
    fp8_status st = check_device(&cus);
    if (st != FP8_OK) return st;
    uint32_t* ws = nullptr;
    const hipError_t e = fp8mi::static_workspace(&ws);
    if (e != hipSuccess)
        return fail(FP8_ERR_HIP, "fp8_quantize_noalloc: the device workspace's address: %s", hipGetErrorString(e));
    return quantize_impl("fp8_quantize_noalloc", x, in_dtype, rows, cols, ld, fmt, gran, flags, hist, q, ldq,
                         nullptr, 0, false, scale_inv_out, amax_out, diag, ws, FP8_WORKSPACE_BYTES, stream);
}

fp8_status fp8_quantize_dual(const void* x, fp8_in_dtype in_dtype, int64_t rows, int64_t cols, int64_t ld,
                             fp8_format fmt, uint32_t flags, fp8_amax_history* hist, uint8_t* q, int64_t ldq,
                             uint8_t* qt, int64_t ldqt, float* scale_inv_out, float* amax_out, fp8_diag* diag,
                             void* workspace, int64_t workspace_bytes, void* stream) {
    return quantize_impl("fp8_quantize_dual", x, in_dtype, rows, cols, ld, fmt, FP8_GRAN_TENSOR, flags, hist, q,
                         ldq, qt, ldqt, true, scale_inv_out, amax_out, diag, workspace, workspace_bytes, stream);
}

fp8_status fp8_quantize_tensors(const fp8_tensor* tensors, int32_t count, fp8_in_dtype in_dtype, fp8_format fmt,
                                uint32_t flags, void* workspace, int64_t workspace_bytes, void* stream) {
    if (tensors == nullptr) return fail(FP8_ERR_INVALID_ARG, "tensors is NULL");
    if (count < 1 || count > FP8_MAX_TENSORS)
        return fail(FP8_ERR_INVALID_ARG, "count=%d not in 1..%d", (int)count, FP8_MAX_TENSORS);
    if (in_dtype != FP8_IN_F32 && in_dtype != FP8_IN_BF16)
        return fail(FP8_ERR_INVALID_ARG, "in_dtype %d is not FP8_IN_F32 or FP8_IN_BF16", (int)in_dtype);
    if (fmt != FP8_E4M3 && fmt != FP8_E5M2)
        return fail(FP8_ERR_INVALID_ARG, "format %d is not FP8_E4M3 or FP8_E5M2", (int)fmt);
    if (flags & ~FP8_SCALE_POW2)
        return fail(FP8_ERR_INVALID_ARG, "unknown flag bits 0x%x (only FP8_SCALE_POW2 applies)",
                    flags & ~FP8_SCALE_POW2);
    fp8mi::MultiQuantArgs a;
    for (int t = 0; t < count; ++t) {
        const fp8_tensor& d = tensors[t];
        if (d.rows < 0 || d.cols < 0)
            return fail(FP8_ERR_INVALID_ARG, "tensor %d: negative size rows=%lld cols=%lld", t, (long long)d.rows,
                        (long long)d.cols);
        if (d.rows > (int64_t(1) << 31) || d.cols > (int64_t(1) << 31))
            return fail(FP8_ERR_UNSUPPORTED_SHAPE, "tensor %d: rows and cols must each be <= 2^31", t);
        const int64_t elems = d.rows * d.cols;
        if (elems / 8 > fp8mi::kMaxUnits)
            return fail(FP8_ERR_UNSUPPORTED_SHAPE, "tensor %d too large: more than 2^34 elements", t);
        if (elems > 0 && d.x == nullptr) return fail(FP8_ERR_INVALID_ARG, "tensor %d: x is NULL", t);
        if (elems > 0 && d.q == nullptr) return fail(FP8_ERR_INVALID_ARG, "tensor %d: q is NULL", t);
        if (d.scale_inv == nullptr) return fail(FP8_ERR_INVALID_ARG, "tensor %d: scale_inv is NULL", t);
        if (d.amax == nullptr) return fail(FP8_ERR_INVALID_ARG, "tensor %d: amax is NULL", t);
        if (!is_aligned(d.x, 16)) return fail(FP8_ERR_MISALIGNED, "tensor %d: x must be 16-byte aligned", t);
        if (!is_aligned(d.q, 8)) return fail(FP8_ERR_MISALIGNED, "tensor %d: q must be 8-byte aligned", t);
        if (!is_aligned(d.scale_inv, 4) || !is_aligned(d.amax, 4))
            return fail(FP8_ERR_MISALIGNED, "tensor %d: scale_inv and amax must be 4-byte aligned", t);
        if (d.diag != nullptr && !is_aligned(d.diag, 4))
            return fail(FP8_ERR_MISALIGNED, "tensor %d: diag must be 4-byte aligned", t);
        a.x[t] = d.x; a.elems[t] = elems; a.q[t] = d.q;
        a.scale_inv[t] = d.scale_inv; a.amax[t] = d.amax; a.diag[t] = d.diag;
    }
    uint32_t* scratch = nullptr;
    fp8_status st = check_workspace(true, workspace, workspace_bytes, &scratch);
    if (st != FP8_OK) return st;
    int cus = 0;
    st = check_device(&cus);
    if (st != FP8_OK) return st;
    a.n = count; a.in_bf16 = in_dtype == FP8_IN_BF16; a.fmt = fmt; a.pow2 = (flags & FP8_SCALE_POW2) != 0;
    a.scratch = scratch; a.stream = (hipStream_t)stream; a.num_cus = cus;
    return launch_result(fp8mi::launch_quantize_multi(a), "fp8_quantize_tensors");
}

static fp8_status check_gemm_common(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, int64_t M,
                                    int64_t N, int64_t K, const float* sa, const float* sb, void* C,
                                    int out_dtype, int64_t ldc) {
    if ((A == nullptr && M > 0 && K > 0) || (B == nullptr && N > 0 && K > 0))
        return fail(FP8_ERR_INVALID_ARG, "A or B is NULL");
    if (C == nullptr && M > 0 && N > 0) return fail(FP8_ERR_INVALID_ARG, "C is NULL");
    if ((sa == nullptr || sb == nullptr) && M > 0 && N > 0)
        return fail(FP8_ERR_INVALID_ARG, "a_scale_inv or b_scale_inv is NULL");
    if (out_dtype != FP8_OUT_F32 && out_dtype != FP8_OUT_BF16)
        return fail(FP8_ERR_INVALID_ARG, "out_dtype %d is not FP8_OUT_F32 or FP8_OUT_BF16", out_dtype);
    if (M < 0 || N < 0 || K < 0)
        return fail(FP8_ERR_INVALID_ARG, "negative size M=%lld N=%lld K=%lld", (long long)M, (long long)N,
                    (long long)K);
    if (M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31) || K >= (int64_t(1) << 31))
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "M, N and K must each be < 2^31");
    if (K % 16 != 0) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "K=%lld must be a multiple of 16", (long long)K);
    if (K > 0) {
        if (lda < K || ldb < K) return fail(FP8_ERR_INVALID_ARG, "lda and ldb must be >= K");
        if (!is_aligned(A, 16) || !is_aligned(B, 16))
            return fail(FP8_ERR_MISALIGNED, "A and B must be 16-byte aligned");
        if (lda % 16 != 0 || ldb % 16 != 0) return fail(FP8_ERR_MISALIGNED, "lda and ldb must be multiples of 16");
        // the loads address one 256-row tile through a 32-bit byte offset
        if (lda > (int64_t(1) << 23) || ldb > (int64_t(1) << 23))
            return fail(FP8_ERR_UNSUPPORTED_SHAPE, "lda and ldb must be <= 2^23 bytes");
    }
    if (ldc < N || ldc < 1) return fail(FP8_ERR_INVALID_ARG, "ldc=%lld must be >= N", (long long)ldc);
    if (!is_aligned(C, out_dtype == FP8_OUT_F32 ? 4 : 2))
        return fail(FP8_ERR_MISALIGNED, "C is not aligned to its element size");
    if (!is_aligned(sa, 4) || !is_aligned(sb, 4)) return fail(FP8_ERR_MISALIGNED, "scale arrays must be 4-byte aligned");
    const int64_t tiles = ((M + 255) / 256) * ((N + 127) / 128);
    if (tiles >= (int64_t(1) << 31)) return fail(FP8_ERR_UNSUPPORTED_SHAPE, "too many output tiles");
    return FP8_OK;
}

fp8_status fp8_scaled_gemm(const uint8_t* A, fp8_format fa, int64_t lda, const uint8_t* B, fp8_format fb,
                           int64_t ldb, int64_t M, int64_t N, int64_t K, const float* a_scale_inv,
                           int a_per_row, const float* b_scale_inv, int b_per_row, void* C,
                           fp8_out_dtype out_dtype, int64_t ldc, void* stream) {
    if ((fa != FP8_E4M3 && fa != FP8_E5M2) || (fb != FP8_E4M3 && fb != FP8_E5M2))
        return fail(FP8_ERR_INVALID_ARG, "formats fa=%d fb=%d must be FP8_E4M3 or FP8_E5M2", (int)fa, (int)fb);
    if ((a_per_row != 0 && a_per_row != 1) || (b_per_row != 0 && b_per_row != 1))
        return fail(FP8_ERR_INVALID_ARG, "a_per_row and b_per_row must be 0 or 1");
    fp8_status st = check_gemm_common(A, lda, B, ldb, M, N, K, a_scale_inv, b_scale_inv, C, out_dtype, ldc);
    if (st != FP8_OK) return st;
    int cus = 0;
    st = check_device(&cus);
    if (st != FP8_OK) return st;
    if (M == 0 || N == 0) return ok();
    fp8mi::GemmArgs g;
    g.A = A; g.B = B; g.fa = fa; g.fb = fb; g.lda = lda; g.ldb = ldb; g.M = M; g.N = N; g.K = K;
    g.sa = a_scale_inv; g.sb = b_scale_inv; g.sa_per_row = a_per_row; g.sb_per_row = b_per_row;
    g.C = C; g.out_bf16 = out_dtype == FP8_OUT_BF16; g.ldc = ldc; g.stream = (hipStream_t)stream;
    g.num_cus = cus;
    return launch_result(fp8mi::launch_scaled_gemm(g), "fp8_scaled_gemm");
}

fp8_status fp8_blockscaled_gemm(const uint8_t* A, int64_t lda, const uint8_t* B, int64_t ldb, int64_t M, int64_t N,
                                int64_t K, const float* a_scale_inv, const float* b_scale_inv, void* C,
                                fp8_out_dtype out_dtype, int64_t ldc, void* stream) {
    fp8_status st = check_gemm_common(A, lda, B, ldb, M, N, K, a_scale_inv, b_scale_inv, C, out_dtype, ldc);
    if (st != FP8_OK) return st;
    if (K == 0 || K % 128 != 0 || N % 128 != 0)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "block-scaled GEMM needs K > 0, K %% 128 == 0 and N %% 128 == 0 (K=%lld N=%lld)",
                    (long long)K, (long long)N);
    int cus = 0;
    st = check_device(&cus);
    if (st != FP8_OK) return st;
    if (M == 0 || N == 0) return ok();
    fp8mi::GemmArgs g;
    g.A = A; g.B = B; g.fa = FP8_E4M3; g.fb = FP8_E4M3; g.lda = lda; g.ldb = ldb; g.M = M; g.N = N; g.K = K;
    g.sa = a_scale_inv; g.sb = b_scale_inv; g.sa_per_row = true; g.sb_per_row = true;
    g.C = C; g.out_bf16 = out_dtype == FP8_OUT_BF16; g.ldc = ldc; g.stream = (hipStream_t)stream;
    g.num_cus = cus;
    return launch_result(fp8mi::launch_blockscaled_gemm(g), "fp8_blockscaled_gemm");
}

static_assert(FP8_GROUPED_MAX_TILES == fp8mi::kGroupTableTiles, "grouped GEMM table size");
static_assert(FP8_WORKSPACE_BYTES == 4 * fp8mi::kScratchWords, "workspace size");

fp8_status fp8_grouped_gemm(const uint8_t* A, fp8_format fa, int64_t lda, const uint8_t* B, fp8_format fb,
                            int64_t ldb, int64_t b_group_stride, int64_t M, int64_t N, int64_t K, int32_t groups,
                            const int32_t* group_offsets, const float* a_scale_inv, int a_per_row,
                            const float* b_scale_inv, int b_per_row, void* C, fp8_out_dtype out_dtype, int64_t ldc,
                            void* workspace, int64_t workspace_bytes, void* stream) {
    if ((fa != FP8_E4M3 && fa != FP8_E5M2) || (fb != FP8_E4M3 && fb != FP8_E5M2))
        return fail(FP8_ERR_INVALID_ARG, "formats fa=%d fb=%d must be FP8_E4M3 or FP8_E5M2", (int)fa, (int)fb);
    if ((a_per_row != 0 && a_per_row != 1) || (b_per_row != 0 && b_per_row != 1))
        return fail(FP8_ERR_INVALID_ARG, "a_per_row and b_per_row must be 0 or 1");
    fp8_status st = check_gemm_common(A, lda, B, ldb, M, N, K, a_scale_inv, b_scale_inv, C, out_dtype, ldc);
    if (st != FP8_OK) return st;
    if (groups < 1) return fail(FP8_ERR_INVALID_ARG, "groups=%d must be >= 1", (int)groups);
    if (group_offsets == nullptr) return fail(FP8_ERR_INVALID_ARG, "group_offsets is NULL");
    if (!is_aligned(group_offsets, 4)) return fail(FP8_ERR_MISALIGNED, "group_offsets must be 4-byte aligned");
    if (K > 0 && N > 0) {
        if (b_group_stride < (N - 1) * ldb + K)
            return fail(FP8_ERR_INVALID_ARG, "b_group_stride=%lld must be >= (N-1)*ldb + K = %lld",
                        (long long)b_group_stride, (long long)((N - 1) * ldb + K));
        if (b_group_stride % 16 != 0)
            return fail(FP8_ERR_MISALIGNED, "b_group_stride=%lld must be a multiple of 16", (long long)b_group_stride);
    }
    if ((M + 255) / 256 + groups > FP8_GROUPED_MAX_TILES)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "ceil(M/256) + groups = %lld exceeds FP8_GROUPED_MAX_TILES (%d)",
                    (long long)((M + 255) / 256 + groups), FP8_GROUPED_MAX_TILES);
    uint32_t* scratch = nullptr;
    st = check_workspace(true, workspace, workspace_bytes, &scratch);
    if (st != FP8_OK) return st;
    int cus = 0;
    st = check_device(&cus);
    if (st != FP8_OK) return st;
    if (M == 0 || N == 0) return ok();
    fp8mi::GemmArgs g;
    g.A = A; g.B = B; g.fa = fa; g.fb = fb; g.lda = lda; g.ldb = ldb; g.M = M; g.N = N; g.K = K;
    g.sa = a_scale_inv; g.sb = b_scale_inv; g.sa_per_row = a_per_row; g.sb_per_row = b_per_row;
    g.C = C; g.out_bf16 = out_dtype == FP8_OUT_BF16; g.ldc = ldc; g.stream = (hipStream_t)stream;
    g.num_cus = cus; g.groups = groups; g.group_offsets = group_offsets; g.b_group_stride = b_group_stride;
    g.scratch = scratch;
    return launch_result(fp8mi::launch_grouped_gemm(g), "fp8_grouped_gemm");
}

// Shape and alignment rules shared by fp8_kv_store and fp8_kv_load.
static fp8_status check_kv_common(const void* cache, int storage, int scaling, const void* scale_inv,
                                  int64_t capacity, int32_t heads, int32_t head_dim, int64_t n_tokens) {
    if (storage != FP8_KV_E4M3 && storage != FP8_KV_E5M2 && storage != FP8_KV_BF16)
        return fail(FP8_ERR_INVALID_ARG, "storage %d is not FP8_KV_E4M3, FP8_KV_E5M2 or FP8_KV_BF16", storage);
    if (scaling != FP8_KV_PER_TOKEN_HEAD && scaling != FP8_KV_PER_HEAD)
        return fail(FP8_ERR_INVALID_ARG, "scaling %d is not FP8_KV_PER_TOKEN_HEAD or FP8_KV_PER_HEAD", scaling);
    if (n_tokens < 0 || capacity < 0 || heads < 0)
        return fail(FP8_ERR_INVALID_ARG, "negative size n_tokens=%lld capacity=%lld heads=%d",
                    (long long)n_tokens, (long long)capacity, (int)heads);
    if (head_dim < 8 || head_dim > 2048 || head_dim % 8 != 0)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "head_dim=%d must be a multiple of 8 in 8..2048", (int)head_dim);
    if (heads > 0 && n_tokens >= (int64_t(1) << 31) / heads)
        return fail(FP8_ERR_UNSUPPORTED_SHAPE, "n_tokens * heads must be < 2^31");
    if (cache == nullptr && capacity > 0 && heads > 0) return fail(FP8_ERR_INVALID_ARG, "cache is NULL");
    if (!is_aligned(cache, 16)) return fail(FP8_ERR_MISALIGNED, "cache must be 16-byte aligned");
    if (storage != FP8_KV_BF16) {
        if (scale_inv == nullptr && heads > 0) return fail(FP8_ERR_INVALID_ARG, "scale_inv is NULL");
        if (!is_aligned(scale_inv, 4)) return fail(FP8_ERR_MISALIGNED, "scale_inv must be 4-byte aligned");
    }
    return FP8_OK;
}

fp8_status fp8_kv_store(const void* x, fp8_in_dtype in_dtype, int64_t n_tokens, int64_t ld, int32_t heads,
                        int32_t head_dim, const int64_t* slots, fp8_kv_storage storage, fp8_kv_scaling scaling,
                        uint32_t flags, void* cache, float* scale_inv, int64_t capacity, fp8_diag* diag,
                        void* stream) {
    fp8_status st = check_kv_common(cache, storage, scaling, scale_inv, capacity, heads, head_dim, n_tokens);
    if (st != FP8_OK) return st;
    if (in_dtype != FP8_IN_F32 && in_dtype != FP8_IN_BF16)
        return fail(FP8_ERR_INVALID_ARG, "in_dtype %d is not FP8_IN_F32 or FP8_IN_BF16", (int)in_dtype);
    if (flags & ~FP8_SCALE_POW2) return fail(FP8_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags & ~FP8_SCALE_POW2);
    const int64_t width = (int64_t)heads * head_dim;
    if (ld < width || ld < 1)
        return fail(FP8_ERR_INVALID_ARG, "ld=%lld must be >= heads*head_dim=%lld", (long long)ld, (long long)width);
    if (ld % 8 != 0) return fail(FP8_ERR_MISALIGNED, "ld=%lld must be a multiple of 8", (long long)ld);
    if (x == nullptr && n_tokens > 0 && heads > 0) return fail(FP8_ERR_INVALID_ARG, "x is NULL");
    if (!is_aligned(x, 16)) return fail(FP8_ERR_MISALIGNED, "x must be 16-byte aligned");
    if (!is_aligned(slots, 8)) return fail(FP8_ERR_MISALIGNED, "slots must be 8-byte aligned");
    if (diag != nullptr && !is_aligned(diag, 4)) return fail(FP8_ERR_MISALIGNED, "diag must be 4-byte aligned");
    int cus = 0;
    st = check_device(&cus);
    if (st != FP8_OK) return st;
    if (n_tokens == 0 || heads == 0 || capacity == 0) return ok();
    fp8mi::KvStoreArgs a;
    a.x = x; a.in_bf16 = in_dtype == FP8_IN_BF16; a.n_tokens = n_tokens; a.ld = ld; a.heads = heads;
    a.head_dim = head_dim; a.slots = slots; a.capacity = capacity; a.storage = storage;
    a.per_head = scaling == FP8_KV_PER_HEAD; a.pow2 = (flags & FP8_SCALE_POW2) != 0; a.cache = cache;
    a.scale_inv = scale_inv; a.diag = storage == FP8_KV_BF16 ? nullptr : diag; a.stream = (hipStream_t)stream;
    return launch_result(fp8mi::launch_kv_store(a), "fp8_kv_store");
}

fp8_status fp8_kv_load(const void* cache, fp8_kv_storage storage, fp8_kv_scaling scaling, const float* scale_inv,
                       int64_t capacity, int32_t heads, int32_t head_dim, const int64_t* slots, int64_t n_tokens,
                       fp8_out_dtype out_dtype, void* out, int64_t ld_out, void* stream) {
    fp8_status st = check_kv_common(cache, storage, scaling, scale_inv, capacity, heads, head_dim, n_tokens);
    if (st != FP8_OK) return st;
    if (out_dtype != FP8_OUT_F32 && out_dtype != FP8_OUT_BF16)
        return fail(FP8_ERR_INVALID_ARG, "out_dtype %d is not FP8_OUT_F32 or FP8_OUT_BF16", (int)out_dtype);
    const int64_t width = (int64_t)heads * head_dim;
    if (ld_out < width || ld_out < 1)
        return fail(FP8_ERR_INVALID_ARG, "ld_out=%lld must be >= heads*head_dim=%lld", (long long)ld_out,
                    (long long)width);
    if (ld_out % 8 != 0) return fail(FP8_ERR_MISALIGNED, "ld_out=%lld must be a multiple of 8", (long long)ld_out);
    if (out == nullptr && n_tokens > 0 && heads > 0) return fail(FP8_ERR_INVALID_ARG, "out is NULL");
    if (!is_aligned(out, 16)) return fail(FP8_ERR_MISALIGNED, "out must be 16-byte aligned");
    if (!is_aligned(slots, 8)) return fail(FP8_ERR_MISALIGNED, "slots must be 8-byte aligned");
    int cus = 0;
    st = check_device(&cus);
    if (st != FP8_OK) return st;
    if (n_tokens == 0 || heads == 0 || capacity == 0) return ok();
    fp8mi::KvLoadArgs a;
    a.cache = cache; a.storage = storage; a.per_head = scaling == FP8_KV_PER_HEAD; a.scale_inv = scale_inv;
    a.capacity = capacity; a.heads = heads; a.head_dim = head_dim; a.slots = slots; a.n_tokens = n_tokens;
    a.out_bf16 = out_dtype == FP8_OUT_BF16; a.out = out; a.ld_out = ld_out; a.stream = (hipStream_t)stream;
    return launch_result(fp8mi::launch_kv_load(a), "fp8_kv_load");
}

}  // extern "C"
