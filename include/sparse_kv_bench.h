/*
 * Measurement helpers of the benchmark (libsparse_kv_bench.so), not part of
 * the decode-attention interface: a streaming-read kernel whose rate is the
 * achievable HBM read ceiling the decode kernels are compared with, and an
 * empty kernel whose launches give the fixed cost of one launch.
 */
#ifndef SPARSE_KV_BENCH_H
#define SPARSE_KV_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#pragma GCC visibility push(default)

/*
 * Read `bytes` of device memory at `buf` once, split into `workgroups`
 * equal contiguous slices (one per workgroup of 256 threads), with
 * non-temporal 16-byte loads covering whole 128-byte lines.
 *   sink  device uint32 [workgroups * 256]; written only in the unlikely case
 *         that a thread's XOR of its loaded words equals 0x9E3779B9.
 * Requires bytes / workgroups to be a multiple of 64 KiB, at least 64 KiB and
 * below 2 GiB; returns 0, -1 on invalid arguments, -3 when the launch fails.
 * Queued on `stream` (a hipStream_t); nothing is allocated.
 */
int skv_bench_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream);

/*
 * Queue one launch of a kernel that does no work, with `workgroups`
 * workgroups of 256 threads, on `stream`.  A chain of these, timed as a
 * captured graph, gives the fixed cost per launch.
 *   sink  device uint32 [workgroups * 256]; never written.
 * Returns 0, -1 on invalid arguments, -3 when the launch fails.
 */
int skv_bench_empty(int32_t workgroups, uint32_t* sink, void* stream);

/*
 * Queue one launch of a kernel whose only work is one 4-byte store per thread
 * (`workgroups` workgroups of 256 threads) into `sink`, device uint32
 * [workgroups * 256].  A chain of these gives the fixed cost of a launch that
 * writes memory.  Returns 0, -1 on invalid arguments, -3 when the launch fails.
 */
int skv_bench_store(int32_t workgroups, uint32_t* sink, void* stream);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_KV_BENCH_H */
