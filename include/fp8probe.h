/*
 * fp8probe.h -- C ABI of libfp8probe.so: HBM streaming probes that give the
 * bandwidth ceilings the FP8 cast kernels are measured against ("DeepL bets
 * on FP8", 1.2: memory bandwidth, not arithmetic, is often what limits).
 * Not part of the FP8 method; the benchmark loads it beside libfp8mi.so.
 *
 * Every pointer is a device pointer on the current HIP device, owned by the
 * caller.  Each call launches one kernel on `stream` (a hipStream_t as
 * void*, NULL = the null stream) and returns 0, a negative value for an
 * invalid argument (nothing launched), or the HIP error of the launch.
 * blocks_per_cu (>= 1): workgroups of 256 threads per compute unit; each
 * workgroup streams one contiguous run of the data (fewer workgroups when
 * the runs would be shorter than 16 KiB).
 */
#ifndef FP8PROBE_H
#define FP8PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16, src 16-byte aligned) once; out[b] gets the
 * XOR of the words block b read (out_words >= the grid, else -2). */
int fp8probe_read(const void* src, int64_t bytes, uint32_t* out, int64_t out_words, int blocks_per_cu,
                  void* stream);

/* Copy `bytes` (a multiple of 16; both pointers 16-byte aligned). */
int fp8probe_copy(const void* src, void* dst, int64_t bytes, int blocks_per_cu, void* stream);

/* For every 16 source bytes write 8 (the low byte of each 16-bit half):
 * src_bytes / 2 bytes written; src 16-byte and dst 8-byte aligned. */
int fp8probe_read2_write1(const void* src, void* dst, int64_t src_bytes, int blocks_per_cu, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8PROBE_H */
