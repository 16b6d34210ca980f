// Probes for the benchmark: the achievable HBM read rate of this device, the
// ceiling the decode kernels are compared with beside the datasheet peak, and
// the fixed cost of one kernel launch.  Not part of the decode library (its
// own shared object).
//
// Every workgroup streams one contiguous slice of the buffer with
// non-temporal 16-byte buffer loads, each wave-wide load covering 1 KiB (8
// whole 128-byte lines), two sets of U loads in flight per lane; the loaded words are
// folded into one register per lane so the loads cannot be dropped, and a
// lane writes only when its fold equals a value it never takes in practice.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparse_kv_bench.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 16;
constexpr uint32_t kStep = kThreads * 16 * kUnroll;  // bytes per workgroup iteration (64 KiB)

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* buf, uint64_t slice, uint32_t* sink) {
  const char* base = buf + (uint64_t)blockIdx.x * slice;
  // slice <= 2 GiB: one buffer resource per workgroup; loads past it return 0
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)slice, 0x00020000);
  const uint32_t t = threadIdx.x * 16u;
  auto load = [&](u32x4 (&x)[kUnroll], uint32_t off) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      x[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(off + u * kThreads * 16u + t), 0, 2 /* nt */);
  };
  auto fold = [&](const u32x4 (&x)[kUnroll], uint32_t acc) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
    return acc;
  };
  // two sets of loads in flight: the next step's are issued before this
  // step's are folded, so the read stream never drains (a step past the
  // slice's end reads nothing: it lies outside the buffer resource)
  uint32_t acc = 0;
  u32x4 a[kUnroll], b[kUnroll];
  load(a, 0);
  for (uint32_t off = 0; off < (uint32_t)slice; off += 2 * kStep) {
    load(b, off + kStep);
    acc = fold(a, acc);
    load(a, off + 2 * kStep);
    acc = fold(b, acc);
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

// A kernel that does no work: a dependent chain of these on one stream
// (captured in a HIP graph, so the host is out of the way) takes, per launch,
// the fixed cost every kernel carries -- dispatch, the workgroups' start and
// end, the completion that the next launch waits for.  That is the floor
// under a stage made of several short launches.
__global__ __launch_bounds__(kThreads) void empty_kernel(uint32_t* sink, uint32_t never) {
  if (never == 0x9E3779B9u) sink[blockIdx.x * kThreads + threadIdx.x] = never;
}

// The same with one 4-byte store per thread: a dependent chain of these takes
// the fixed cost of a launch that writes memory (its stores drain before the
// next launch starts).
__global__ __launch_bounds__(kThreads) void store_kernel(uint32_t* sink) {
  sink[blockIdx.x * kThreads + threadIdx.x] = blockIdx.x;
}

}  // namespace

extern "C" int skv_bench_store(int32_t workgroups, uint32_t* sink, void* stream) {
  if (!sink || workgroups < 1) return -1;
  store_kernel<<<workgroups, kThreads, 0, (hipStream_t)stream>>>(sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int skv_bench_empty(int32_t workgroups, uint32_t* sink, void* stream) {
  if (!sink || workgroups < 1) return -1;
  empty_kernel<<<workgroups, kThreads, 0, (hipStream_t)stream>>>(sink, 0u);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int skv_bench_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                                     void* stream) {
  if (!buf || !sink || workgroups < 1) return -1;
  const uint64_t slice = (uint64_t)bytes / (uint64_t)workgroups;
  // offsets up to slice + 2 steps stay below 2^31 (past the slice: outside the resource)
  if (slice < kStep || slice % kStep != 0 || slice > (1ull << 31) - 4 * (uint64_t)kStep) return -1;
  stream_read_kernel<<<workgroups, kThreads, 0, (hipStream_t)stream>>>((const char*)buf, slice, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
