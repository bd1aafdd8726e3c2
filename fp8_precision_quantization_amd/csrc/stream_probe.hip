// stream_probe.hip -- plain HBM streaming kernels that measure the bandwidth
// ceilings the cast kernels are compared with (libfp8probe.so, loaded only by
// the benchmark): a read-only stream, a copy, and a stream that reads 16
// bytes and writes 8 for every unit, the access pattern of a bf16 -> FP8
// cast without its arithmetic.  Each workgroup streams one contiguous run of
// 16-byte units, four units in flight per thread, with non-temporal loads
// (the data is read once) and ordinary stores (as the casts store codes).
// Contiguous runs per workgroup stream faster on this chip than a
// grid-stride loop over the same units, which loses 15-25 % at 4 to 8
// workgroups per CU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kStep = (int64_t)kThreads * kUnroll;   // units one iteration covers

__device__ __forceinline__ uint4 load_nt(const uint4* p) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// This workgroup's run [beg, end) of `units` units, `chunk` per workgroup.
__device__ __forceinline__ void run_of(int64_t units, int64_t chunk, int64_t& beg, int64_t& end) {
    beg = (int64_t)blockIdx.x * chunk;
    end = beg + chunk < units ? beg + chunk : units;
}

// XOR of every word read, one result per block (so no load is dead).
__global__ __launch_bounds__(kThreads) void k_read(const uint4* __restrict__ src, int64_t units, int64_t chunk,
                                                   uint32_t* __restrict__ out) {
    __shared__ uint32_t part[kThreads / 64];
    int64_t beg, end;
    run_of(units, chunk, beg, end);
    uint32_t acc = 0;
    for (int64_t u0 = beg + threadIdx.x; u0 < end; u0 += kStep) {
        uint4 v[kUnroll];
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int64_t u = u0 + i * kThreads;
            v[i] = u < end ? load_nt(src + u) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__global__ __launch_bounds__(kThreads) void k_copy(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                   int64_t units, int64_t chunk) {
    int64_t beg, end;
    run_of(units, chunk, beg, end);
    for (int64_t u0 = beg + threadIdx.x; u0 < end; u0 += kStep) {
        uint4 v[kUnroll];
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int64_t u = u0 + i * kThreads;
            if (u < end) v[i] = load_nt(src + u);
        }
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int64_t u = u0 + i * kThreads;
            if (u < end) dst[u] = v[i];
        }
    }
}

// 16 bytes in, 8 bytes out per unit: the low byte of each 16-bit half.
__global__ __launch_bounds__(kThreads) void k_read2_write1(const uint4* __restrict__ src, uint2* __restrict__ dst,
                                                           int64_t units, int64_t chunk) {
    int64_t beg, end;
    run_of(units, chunk, beg, end);
    for (int64_t u0 = beg + threadIdx.x; u0 < end; u0 += kStep) {
        uint4 v[kUnroll];
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int64_t u = u0 + i * kThreads;
            if (u < end) v[i] = load_nt(src + u);
        }
#pragma unroll
        for (int i = 0; i < kUnroll; ++i) {
            const int64_t u = u0 + i * kThreads;
            if (u < end) {
                uint2 w;
                w.x = __builtin_amdgcn_perm(v[i].y, v[i].x, 0x06040200u);
                w.y = __builtin_amdgcn_perm(v[i].w, v[i].z, 0x06040200u);
                dst[u] = w;
            }
        }
    }
}

// Grid of blocks_per_cu workgroups per CU (fewer for a small stream), and the
// units of each one's run (a multiple of kStep).
int grid_of(int64_t units, int blocks_per_cu, int64_t* chunk) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int64_t cap = (int64_t)cus * blocks_per_cu;
    int64_t per = (units + cap - 1) / cap;
    per = (per + kStep - 1) / kStep * kStep;
    if (per < kStep) per = kStep;
    *chunk = per;
    const int64_t g = (units + per - 1) / per;
    return (int)(g < 1 ? 1 : g);
}

int status(hipError_t e) { return e == hipSuccess ? 0 : (int)e; }

}  // namespace

extern "C" {

int fp8probe_read(const void* src, int64_t bytes, uint32_t* out, int64_t out_words, int blocks_per_cu,
                  void* stream) {
    if (src == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0 ||
        blocks_per_cu < 1)
        return -1;
    const int64_t units = bytes / 16;
    int64_t chunk = 0;
    const int grid = grid_of(units, blocks_per_cu, &chunk);
    if (out_words < grid) return -2;
    hipLaunchKernelGGL(k_read, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const uint4*>(src), units, chunk, out);
    return status(hipGetLastError());
}

int fp8probe_copy(const void* src, void* dst, int64_t bytes, int blocks_per_cu, void* stream) {
    if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0 ||
        (uintptr_t)dst % 16 != 0 || blocks_per_cu < 1)
        return -1;
    const int64_t units = bytes / 16;
    int64_t chunk = 0;
    const int grid = grid_of(units, blocks_per_cu, &chunk);
    hipLaunchKernelGGL(k_copy, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const uint4*>(src), static_cast<uint4*>(dst), units, chunk);
    return status(hipGetLastError());
}

int fp8probe_read2_write1(const void* src, void* dst, int64_t src_bytes, int blocks_per_cu, void* stream) {
    if (src == nullptr || dst == nullptr || src_bytes <= 0 || src_bytes % 16 != 0 || (uintptr_t)src % 16 != 0 ||
        (uintptr_t)dst % 8 != 0 || blocks_per_cu < 1)
        return -1;
    const int64_t units = src_bytes / 16;
    int64_t chunk = 0;
    const int grid = grid_of(units, blocks_per_cu, &chunk);
    hipLaunchKernelGGL(k_read2_write1, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                       static_cast<const uint4*>(src), static_cast<uint2*>(dst), units, chunk);
    return status(hipGetLastError());
}

}  // extern "C"
