// Content-aware block selection for gfx950: block centroids, group scores
// against the query, and top-k with forced sink and recent blocks.
//
// Method ("Squeezed Attention" blog, Q1 / Q2 steps 1-2): every group of keys
// is represented by its centroid; the query is compared with the centroids
// and only the best groups' keys are loaded.  Here a group is a 64-token
// block and its centroid the block's mean key; the comparison is the scaled
// dot product with the sum of the GQA group's queries, one score per KV head
// and no softmax ("SparDA" summary, §2); the first block is always kept
// ("ART" summary, §2.4, attention sink), as is a recent window.
#include "device_common.hpp"
#include "kernels.hpp"

namespace skv {
namespace {

// ---- centroids: one wave per block, row layout, fp32 sums ---------------
template <typename T, int D>
__global__ __launch_bounds__(256) void centroid_kernel(const void* __restrict__ k, const int32_t* __restrict__ seq_lens,
                                                       float* __restrict__ C, int32_t Hkv, int32_t NBmax) {
  using Gm = Geo<T, D>;
  constexpr int E = Gm::E, CPR = Gm::CPR, TPI = Gm::TPI, ROWB = Gm::ROWB;
  constexpr bool BF = sizeof(T) == 2;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= NBmax) return;
  const int g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63;
  const int L = clampi(seq_lens ? seq_lens[b] : NBmax * kBlock, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;
  const size_t unit = (size_t)b * Hkv + g;
  float* crow = C + (unit * NBmax + j) * D;
  if (j >= nb) {
    for (int i = lane; i < D; i += 64) crow[i] = 0.f;
    return;
  }
  const auto rs = make_rsrc((const char*)k + unit * (size_t)NBmax * kBlock * ROWB, (uint32_t)L * ROWB);
  const uint32_t base = (uint32_t)j * kBlock * ROWB + (uint32_t)(lane / CPR) * ROWB + (uint32_t)(lane % CPR) * 16;
  float sum[E];
#pragma unroll
  for (int e = 0; e < E; ++e) sum[e] = 0.f;
#pragma unroll
  for (int i = 0; i < CPR; ++i) {
    const u32x4 x = load16_nt(rs, base + i * TPI * ROWB, 0);
    if constexpr (BF) {
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        sum[2 * e2] += bf16_lo(x[e2]);
        sum[2 * e2 + 1] += bf16_hi(x[e2]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] += __uint_as_float(x[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e)
    sum[e] = phase_sum<CPR>(sum[e]);
  const float n = (float)min(kBlock, L - j * kBlock);
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < E; ++e) crow[lane * E + e] = sum[e] / n;
  }
}

// ---- scores: 4 waves x 32 centroid rows per workgroup -------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void score_kernel(const void* __restrict__ q, const float* __restrict__ C,
                                                    const int32_t* __restrict__ seq_lens, float* __restrict__ scores,
                                                    int32_t Hq, int32_t Hkv, int32_t NBmax, float scale) {
  constexpr int LPR = D / 4;     // lanes per centroid row, 4 floats each
  constexpr int RPI = 64 / LPR;  // rows per wave-wide load
  constexpr int ROWS = 32;       // rows per wave
  constexpr int IT = ROWS / RPI;
  const int g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int G = Hq / Hkv;
  const int L = clampi(seq_lens ? seq_lens[b] : NBmax * kBlock, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;
  const size_t unit = (size_t)b * Hkv + g;
  const int c = lane % LPR;

  float qs[4] = {0.f, 0.f, 0.f, 0.f};
  for (int h = 0; h < G; ++h) {
    const T* qr = (const T*)q + ((size_t)b * Hq + (size_t)g * G + h) * D + 4 * c;
#pragma unroll
    for (int e = 0; e < 4; ++e) qs[e] += elem_f32(qr, e);
  }
  const auto rs = make_rsrc(C + unit * (size_t)NBmax * D, (uint32_t)nb * D * 4);
  const int j0 = (blockIdx.x * 4 + w) * ROWS;
  float part[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j = j0 + it * RPI + lane / LPR;
    const u32x4 x = load16_nt(rs, ((uint32_t)j * D + 4 * c) * 4, 0);
    float s = qs[0] * __uint_as_float(x[0]);
    s = fmaf(qs[1], __uint_as_float(x[1]), s);
    s = fmaf(qs[2], __uint_as_float(x[2]), s);
    s = fmaf(qs[3], __uint_as_float(x[3]), s);
    part[it] = s;
  }
  float* srow = scores + unit * NBmax;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    float s = row16_sum(part[it]);
    if constexpr (LPR == 32) s = xrow16_sum(s);
    const int j = j0 + it * RPI + lane / LPR;
    if (c == 0 && j < NBmax) srow[j] = j < nb ? s * scale : -INFINITY;
  }
}

// ---- top-k: one workgroup per (b, kv head) -------------------------------
// Order-preserving map of a float onto uint32 (-0 folded onto +0).
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of one int per thread over a 256-thread workgroup.
__device__ int block_exscan(int x, int* total, int* lds4) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) lds4[w] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = lds4[i];
    base += i < w ? v : 0;
    tot += v;
  }
  __syncthreads();
  *total = tot;
  return base + inc - x;
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
                                                   int32_t Hkv, int32_t NBmax, int32_t k, int32_t n_sink,
                                                   int32_t n_recent, int32_t max_sel, int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ n_sel) {
  __shared__ uint32_t hist[256];
  __shared__ int scan4[4];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_rem;
  const int unit = blockIdx.x, b = unit / Hkv, tid = threadIdx.x;
  const int L = clampi(seq_lens ? seq_lens[b] : NBmax * kBlock, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;
  const float* row = scores + (size_t)unit * NBmax;
  int32_t* out = idx + (size_t)unit * max_sel;

  // forced blocks: [0, sink_hi) and [rec_lo, nb); candidates: [sink_hi, rec_lo)
  const int sink_hi = min(n_sink, nb);
  const int rec_lo = max(nb - n_recent, sink_hi);
  const int ncand = rec_lo - sink_hi;
  const int kk = min(k, ncand);
  const bool take_all = kk == ncand;
  const bool ranked = kk > 0 && !take_all;

  // radix select of the kk-th largest key, 8 bits per pass
  uint32_t thr = 0;
  int need_eq = 0;
  if (ranked) {
    uint32_t prefix = 0, mask = 0;
    int rem = kk;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int j = sink_hi + tid; j < rec_lo; j += 256) {
        const uint32_t u = score_key(row[j]);
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
      const int bin = 255 - tid;  // thread 0 takes the highest digit
      const int x = (int)hist[bin];
      int tot;
      const int above = block_exscan(x, &tot, scan4);
      if (above < rem && rem <= above + x) {
        sh_prefix = prefix | ((uint32_t)bin << shift);
        sh_rem = rem - above;
      }
      __syncthreads();
      prefix = sh_prefix;
      rem = sh_rem;
      mask |= 255u << shift;
      __syncthreads();
    }
    thr = prefix;
    need_eq = rem;  // keys equal to thr still to take, lowest index first
  }

  // each thread owns a contiguous chunk so that scans follow index order
  const int CH = (nb + 255) / 256;
  const int j0 = min(tid * CH, nb), j1 = min(j0 + CH, nb);
  int eq_local = 0;
  if (ranked)
    for (int j = j0; j < j1; ++j)
      if (j >= sink_hi && j < rec_lo && score_key(row[j]) == thr) ++eq_local;
  int tot_eq;
  const int eq_before = block_exscan(eq_local, &tot_eq, scan4);

  auto chosen = [&](int j, int& eq_seen) -> bool {
    if (j < sink_hi || j >= rec_lo) return true;
    if (kk == 0) return false;
    if (take_all) return true;
    const uint32_t u = score_key(row[j]);
    if (u > thr) return true;
    if (u == thr) return eq_seen++ < need_eq;
    return false;
  };
  int eq_seen = eq_before, cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += chosen(j, eq_seen) ? 1 : 0;
  int total;
  int pos = block_exscan(cnt, &total, scan4);
  eq_seen = eq_before;
  for (int j = j0; j < j1; ++j)
    if (chosen(j, eq_seen) && pos < max_sel) out[pos++] = j;
  for (int i = total + tid; i < max_sel; i += 256) out[i] = -1;
  if (tid == 0) n_sel[unit] = min(total, max_sel);
}

// ---- importance order: one workgroup per (b, kv head) -------------------
// Block 0 first, then blocks 1 .. nb-1 by descending score, lower index first
// among equal scores ("ART" summary, §2.4, importance-first visit order).
// The nb - 1 keys (inverted score key << 32 | block) are sorted ascending by
// a bitonic network in LDS, padded to a power of two with all-ones keys.
template <int CAP>
__global__ __launch_bounds__(1024) void order_kernel(const float* __restrict__ scores,
                                                     const int32_t* __restrict__ seq_lens, int32_t Hkv,
                                                     int32_t NBmax, int32_t* __restrict__ order) {
  __shared__ uint64_t key[CAP];
  const int unit = blockIdx.x, b = unit / Hkv, tid = threadIdx.x;
  const int L = clampi(seq_lens ? seq_lens[b] : NBmax * kBlock, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;
  const float* row = scores + (size_t)unit * NBmax;
  int32_t* out = order + (size_t)unit * NBmax;
  const int nr = max(nb - 1, 0);  // blocks after the sink
  int n = 2;
  while (n < nr) n <<= 1;
  for (int i = tid; i < n; i += 1024)
    key[i] = i < nr ? ((uint64_t)~score_key(row[i + 1]) << 32) | (uint32_t)(i + 1) : ~(uint64_t)0;
  __syncthreads();
  for (int kk = 2; kk <= n; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int pr = tid; pr < (n >> 1); pr += 1024) {
        const int i = 2 * j * (pr / j) + pr % j;  // pair (i, i + j)
        const uint64_t x = key[i], y = key[i + j];
        const bool up = (i & kk) == 0;
        if ((x > y) == up) {
          key[i] = y;
          key[i + j] = x;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < NBmax; i += 1024)
    out[i] = i == 0 ? (nb > 0 ? 0 : -1) : (i < nb ? (int32_t)(uint32_t)key[i - 1] : -1);
}

}  // namespace

hipError_t launch_build_centroids(const void* k, const int32_t* seq_lens, float* c, int32_t B,
                                  int32_t Hkv, int32_t d, int32_t NBmax, int32_t dtype,
                                  hipStream_t st) {
  if (B == 0) return hipSuccess;
  const dim3 grid((NBmax + 3) / 4, Hkv, B);
  if (dtype == 1) {
    if (d == 128)
      centroid_kernel<__bf16, 128><<<grid, 256, 0, st>>>(k, seq_lens, c, Hkv, NBmax);
    else
      centroid_kernel<__bf16, 64><<<grid, 256, 0, st>>>(k, seq_lens, c, Hkv, NBmax);
  } else {
    if (d == 128)
      centroid_kernel<float, 128><<<grid, 256, 0, st>>>(k, seq_lens, c, Hkv, NBmax);
    else
      centroid_kernel<float, 64><<<grid, 256, 0, st>>>(k, seq_lens, c, Hkv, NBmax);
  }
  return hipGetLastError();
}

hipError_t launch_score(const void* q, const float* c, const int32_t* seq_lens, float* scores,
                        int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t NBmax,
                        int32_t dtype, float scale, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const dim3 grid((NBmax + 127) / 128, Hkv, B);
  if (dtype == 1) {
    if (d == 128)
      score_kernel<__bf16, 128><<<grid, 256, 0, st>>>(q, c, seq_lens, scores, Hq, Hkv, NBmax, scale);
    else
      score_kernel<__bf16, 64><<<grid, 256, 0, st>>>(q, c, seq_lens, scores, Hq, Hkv, NBmax, scale);
  } else {
    if (d == 128)
      score_kernel<float, 128><<<grid, 256, 0, st>>>(q, c, seq_lens, scores, Hq, Hkv, NBmax, scale);
    else
      score_kernel<float, 64><<<grid, 256, 0, st>>>(q, c, seq_lens, scores, Hq, Hkv, NBmax, scale);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, const int32_t* seq_lens, int32_t B, int32_t Hkv,
                       int32_t NBmax, int32_t k, int32_t n_sink, int32_t n_recent,
                       int32_t max_sel, int32_t* idx, int32_t* n_sel, hipStream_t st) {
  if (B == 0) return hipSuccess;
  topk_kernel<<<dim3(B * Hkv), 256, 0, st>>>(scores, seq_lens, Hkv, NBmax, k, n_sink, n_recent,
                                             max_sel, idx, n_sel);
  return hipGetLastError();
}

hipError_t launch_order(const float* scores, const int32_t* seq_lens, int32_t B, int32_t Hkv,
                        int32_t NBmax, int32_t* order, hipStream_t st) {
  if (B == 0) return hipSuccess;
  if (NBmax - 1 > kOrderMaxRest) return hipErrorInvalidValue;
  if (NBmax - 1 <= 4096)
    order_kernel<4096><<<dim3(B * Hkv), 1024, 0, st>>>(scores, seq_lens, Hkv, NBmax, order);
  else
    order_kernel<kOrderMaxRest><<<dim3(B * Hkv), 1024, 0, st>>>(scores, seq_lens, Hkv, NBmax, order);
  return hipGetLastError();
}

}  // namespace skv
