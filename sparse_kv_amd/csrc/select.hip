// Content-aware block selection for gfx950: block centroids (built, or
// refreshed after appends), group scores against the query, top-k with
// forced sink and recent blocks, two-level (super-block) selection, and the
// importance-first visit order.
//
// Method ("Squeezed Attention" blog, Q1 / Q2 steps 1-2): every group of keys
// is represented by its centroid; the query is compared with the centroids
// and only the best groups' keys are loaded.  Here a group is a 64-token
// block and its centroid the block's mean key; the comparison is the scaled
// dot product with the sum of the GQA group's queries, one score per KV head
// and no softmax ("SparDA" summary, §2); the first block is always kept
// ("ART" summary, §2.4, attention sink), as is a recent window.  Q2 step 4
// (hierarchical clustering) adds a coarse level of super-blocks searched
// first; ART §2.4 (importance first) orders blocks by the same scores.
#include "device_common.hpp"
#include "kernels.hpp"

namespace skv {
namespace {

// ---- centroids: one wave per block, row layout, fp32 sums ---------------
// Centroid of block j (wave-uniform) of the (b, g) unit: the mean of its
// valid keys, zeros for a block past the sequence's end.  K is contiguous
// [B, Hkv, NBmax * 64, d], or a pool of blocks addressed through pg.table.
template <typename T, int D>
__device__ void centroid_block(const void* __restrict__ k, float* __restrict__ C, int b, int g, int32_t Hkv, int j,
                               int L, int32_t NBmax, int lane, const PagedK& pg) {
  using Gm = Geo<T, D>;
  constexpr int E = Gm::E, CPR = Gm::CPR, TPI = Gm::TPI, ROWB = Gm::ROWB;
  constexpr bool BF = sizeof(T) == 2;
  const int nb = (L + kBlock - 1) / kBlock;
  const size_t unit = (size_t)b * Hkv + g;
  float* crow = C + (unit * NBmax + j) * D;
  if (j >= nb) {
    for (int i = lane; i < D; i += 64) crow[i] = 0.f;
    return;
  }
  size_t boff;
  if (pg.table) {
    const int ph = clampi(uniform_load(pg.table, (int64_t)b * pg.table_stride + j), 0, (int)(pg.pool_blocks - 1));
    boff = ((size_t)ph * Hkv + g) * (kBlock * ROWB);
  } else {
    boff = (unit * NBmax + j) * (size_t)(kBlock * ROWB);
  }
  const auto rs = make_rsrc((const char*)k + boff, (uint32_t)min(kBlock, L - j * kBlock) * ROWB);
  const uint32_t base = (uint32_t)(lane / CPR) * ROWB + (uint32_t)(lane % CPR) * 16;
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

template <typename T, int D>
__global__ __launch_bounds__(256) void centroid_kernel(const void* __restrict__ k, const int32_t* __restrict__ seq_lens,
                                                       float* __restrict__ C, int32_t Hkv, int32_t NBmax, PagedK pg) {
  const int j = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (j >= NBmax) return;
  const int g = blockIdx.y, b = blockIdx.z;
  const int L = clampi(seq_lens ? seq_lens[b] : NBmax * kBlock, 0, NBmax * kBlock);
  centroid_block<T, D>(k, C, b, g, Hkv, j, L, NBmax, threadIdx.x & 63, pg);
}

// Refresh after tokens were appended: blocks [min(prev_len, L) / 64, nb) of
// every row (the block that held the shorter end onwards), or only the last
// block without previous lengths; blocks past the end are zeroed up to the
// previous block count, so a shrunk row is cleared too.  Workgroup x of a
// unit takes blocks lo + 4x + wave, lo + 4x + wave + 4X, ...
template <typename T, int D>
__global__ __launch_bounds__(256) void centroid_update_kernel(const void* __restrict__ k,
                                                              const int32_t* __restrict__ seq_lens,
                                                              const int32_t* __restrict__ prev_lens,
                                                              float* __restrict__ C, int32_t Hkv, int32_t NBmax,
                                                              PagedK pg) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int Lmax = NBmax * kBlock;
  const int L = clampi(seq_lens ? seq_lens[b] : Lmax, 0, Lmax);
  const int nb = (L + kBlock - 1) / kBlock;
  int lo, hi;
  if (prev_lens) {
    const int P = clampi(prev_lens[b], 0, Lmax);
    lo = min(P, L) / kBlock;
    hi = max(nb, (P + kBlock - 1) / kBlock);
  } else {
    lo = max(nb - 1, 0);
    hi = nb;
  }
  for (int j = lo + blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); j < hi; j += gridDim.x * 4)
    centroid_block<T, D>(k, C, b, g, Hkv, j, L, NBmax, threadIdx.x & 63, pg);
}

// ---- scores: 4 waves x 16 centroid rows per workgroup -------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void score_kernel(const void* __restrict__ q, const float* __restrict__ C,
                                                    const int32_t* __restrict__ seq_lens, float* __restrict__ scores,
                                                    int32_t Hq, int32_t Hkv, int32_t NBmax, float scale) {
  constexpr int LPR = D / 4;     // lanes per centroid row, 4 floats each
  constexpr int RPI = 64 / LPR;  // rows per wave-wide load
  constexpr int ROWS = 16;       // rows per wave
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

// Inclusive prefix sum over the 64 lanes of a wave, in DPP: row_shr 1, 2, 4,
// 8 within rows of 16 (a lane whose source lies in the previous row adds 0),
// then row_bcast:15 adds row 0's total to row 1 and row 2's to row 3, and
// row_bcast:31 adds the first 32 lanes' total to rows 2 and 3.
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return x;
}

// Number of lanes below this one whose bit is set in a wave-wide mask.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive prefix sum of one int per thread over a 256-thread workgroup.
__device__ int block_exscan(int x, int* total, int* lds4) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_sum(x);
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

// Exclusive prefix sums of two ints per thread in one pass (same barriers
// as one): returns a's prefix, writes b's prefix and both totals.
__device__ int block_exscan2(int a, int b, int* tot_a, int* tot_b, int* pre_b) {
  __shared__ int lds[2][4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ia = wave_incl_sum(a), ib = wave_incl_sum(b);
  if (lane == 63) {
    lds[0][w] = ia;
    lds[1][w] = ib;
  }
  __syncthreads();
  int ba = 0, bb = 0, ta = 0, tb = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int va = lds[0][i], vb = lds[1][i];
    ba += i < w ? va : 0;
    bb += i < w ? vb : 0;
    ta += va;
    tb += vb;
  }
  __syncthreads();
  *tot_a = ta;
  *tot_b = tb;
  *pre_b = bb + ib - b;
  return ba + ia - a;
}

// Radix select (8 bits a pass, 256-thread workgroup) of the kk-th largest
// key among items [0, n) with elig(i): returns that key and how many items
// equal to it are to be taken (lowest indices first).  0 < kk < #eligible.
template <typename KeyF, typename EligF>
__device__ void radix_select(int n, int kk, KeyF key, EligF elig, uint32_t* hist, int* scan4, uint32_t* sh_prefix,
                             int* sh_rem, uint32_t& thr, int& need_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  int rem = kk;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      if (!elig(i)) continue;
      const uint32_t u = key(i);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    const int bin = 255 - tid;  // thread 0 takes the highest digit
    const int x = (int)hist[bin];
    int tot;
    const int above = block_exscan(x, &tot, scan4);
    if (above < rem && rem <= above + x) {
      *sh_prefix = prefix | ((uint32_t)bin << shift);
      *sh_rem = rem - above;
    }
    __syncthreads();
    prefix = *sh_prefix;
    rem = *sh_rem;
    mask |= 255u << shift;
    __syncthreads();
  }
  thr = prefix;
  need_eq = rem;
}

// The bin of a 4096-bin histogram (top 12 bits of the keys) that holds the
// kk-th largest key.  Thread t owns bins 4095 - 16 t - c (c = 0..15), read
// as four 16-byte loads into registers (hist must be 16-byte aligned); a
// block scan gives the keys in the bins above each thread's, and the one
// thread whose bins take the running count from below kk to at least kk
// returns true with the bin, how many of its keys are among the kk (rem) and
// its count.  Every thread of the workgroup must call it.
__device__ bool kth_bin(const uint32_t* hist, int kk, int* scan4, int& bin, int& rem, int& cnt) {
  const int tid = threadIdx.x;
  uint32_t hb[16];  // hb[15 - c] is bin 4095 - 16 t - c
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 h4 = *(const u32x4*)&hist[4080 - 16 * tid + 4 * i];
#pragma unroll
    for (int e = 0; e < 4; ++e) hb[4 * i + e] = h4[e];
  }
  int loc = 0;
#pragma unroll
  for (int c = 0; c < 16; ++c) loc += (int)hb[c];
  int tot;
  const int above = block_exscan(loc, &tot, scan4);  // keys in the bins above this thread's
  if (!(above < kk && kk <= above + loc)) return false;
  int a = above, fc = 0, fa = above, fh = 0;
#pragma unroll
  for (int c = 0; c < 16; ++c) {  // downwards; exactly one bin crosses kk
    const int h = (int)hb[15 - c];
    const bool here = a < kk && a + h >= kk;
    fc = here ? c : fc;
    fa = here ? a : fa;
    fh = here ? h : fh;
    a += h;
  }
  bin = 4095 - 16 * tid - fc;
  rem = kk - fa;
  cnt = fh;
  return true;
}

// The kk-th largest key in one histogram pass, for keys cheap to read twice
// (staged in LDS): a 4096-bin histogram of the top 12 key bits locates the
// bin holding it (thread t sums bins 4095 - 16t ...; one block scan), then
// that bin's keys are ranked against each other.  False -- nothing decided
// -- when that bin holds more than 256 keys (heavy ties or clustering).
// `cleared`: the histogram is already zero and that is visible to every thread.
template <typename KeyF, typename EligF>
__device__ bool select_wide(int n, int kk, KeyF key, EligF elig, uint32_t* hist, uint32_t* cand, int* scan4,
                            uint32_t* sh_prefix, int* sh_rem, uint32_t& thr, int& need_eq, bool cleared) {
  __shared__ int sh[4];
  const int tid = threadIdx.x;
  if (!cleared) {
    for (int i = tid; i < 4096; i += 256) hist[i] = 0;
    __syncthreads();
  }
  for (int i = tid; i < n; i += 256)
    if (elig(i)) atomicAdd(&hist[key(i) >> 20], 1u);
  __syncthreads();
  {
    int fb, fr, fn;
    if (kth_bin(hist, kk, scan4, fb, fr, fn)) {
      sh[0] = fb;
      sh[1] = fr;  // how many of the bin's keys are among the kk
      sh[2] = fn;
    }
  }
  if (tid == 0) sh[3] = 0;
  __syncthreads();
  const uint32_t bin = (uint32_t)sh[0];
  const int rem = sh[1], cnt = sh[2];
  if (cnt > 256) return false;
  // the bin's keys, in any order (the rank below does not depend on it); one
  // atomic per wave and pass reserves room for the wave's keys
  const int lane = tid & 63;
  for (int i0 = 0; i0 < n; i0 += 256) {
    const int i = i0 + tid;
    const bool m = i < n && elig(i) && (key(i) >> 20) == bin;
    const uint64_t mk = (uint64_t)__ballot(m);
    if (mk != 0) {
      int base = 0;
      if (lane == 0) base = atomicAdd(&sh[3], __popcll(mk));
      base = __shfl(base, 0);
      if (m) cand[base + lanes_below(mk)] = key(i);
    }
  }
  __syncthreads();
  if (tid < cnt) {
    const uint32_t x = cand[tid];
    int gt = 0, ge = 0;
    for (int c = 0; c < cnt; ++c) {
      gt += cand[c] > x ? 1 : 0;
      ge += cand[c] >= x ? 1 : 0;
    }
    if (gt < rem && rem <= ge) {  // x is the rem-th largest of the bin (equal keys write equal values)
      *sh_prefix = x;
      *sh_rem = rem - gt;
    }
  }
  __syncthreads();
  thr = *sh_prefix;
  need_eq = *sh_rem;
  __syncthreads();
  return true;
}

// Calls take(i, rank) for the kk best eligible items of [0, n) in index
// order (rank = 0, 1, ... over the taken items), ties to the lower index.
// Each thread owns a contiguous chunk, so ranks follow the index order.
// Returns the number taken.
// With WIDE, hist holds 4096 entries and cand 256, and the threshold comes
// from select_wide when it can decide (`cleared`: hist is already zero).
// ALL: every item is eligible.
template <bool WIDE = false, bool ALL = false, typename KeyF, typename EligF, typename TakeF>
__device__ int take_best(int n, int kk, KeyF key, EligF elig, TakeF take, uint32_t* hist, int* scan4,
                         uint32_t* sh_prefix, int* sh_rem, uint32_t* cand = nullptr, bool cleared = false) {
  const int tid = threadIdx.x;
  const int CH = (n + 255) / 256;
  const int i0 = min(tid * CH, n), i1 = min(i0 + CH, n);
  int n_elig = n;
  if constexpr (!ALL) {
    int ne = 0;
    for (int i = i0; i < i1; ++i) ne += elig(i) ? 1 : 0;
    block_exscan(ne, &n_elig, scan4);
  }
  const int kq = min(kk, n_elig);
  const bool ranked = kq > 0 && kq < n_elig;
  uint32_t thr = 0;
  int need_eq = 0;
  if (ranked) {
    bool done = false;
    if constexpr (WIDE)
      done = select_wide(n, kq, key, elig, hist, cand, scan4, sh_prefix, sh_rem, thr, need_eq, cleared);
    if (!done) radix_select(n, kq, key, elig, hist, scan4, sh_prefix, sh_rem, thr, need_eq);
  }
  // per chunk: keys equal to the threshold and keys above it (every
  // eligible key when nothing is ranked); the items chosen before a chunk
  // are the keys above before it plus its share of the first need_eq ties
  int eq_local = 0, gt_local = 0;
  for (int i = i0; i < i1; ++i) {
    if (!elig(i)) continue;
    if (!ranked) {
      ++gt_local;
    } else {
      const uint32_t u = key(i);
      gt_local += u > thr ? 1 : 0;
      eq_local += u == thr ? 1 : 0;
    }
  }
  int eq_tot, gt_tot, gt_before;
  const int eq_before = block_exscan2(eq_local, gt_local, &eq_tot, &gt_tot, &gt_before);
  auto chosen = [&](int i, int& eq_seen) -> bool {
    if (kq == 0 || !elig(i)) return false;
    if (!ranked) return true;
    const uint32_t u = key(i);
    if (u > thr) return true;
    if (u == thr) return eq_seen++ < need_eq;
    return false;
  };
  int rank = kq == 0 ? 0 : (ranked ? gt_before + min(eq_before, need_eq) : gt_before);
  const int total = kq == 0 ? 0 : (ranked ? gt_tot + need_eq : gt_tot);
  int eq_seen = eq_before;
  for (int i = i0; i < i1; ++i)
    if (chosen(i, eq_seen)) take(i, rank++);
  __syncthreads();
  return total;
}

// The candidates' order-preserving keys are staged in LDS once (rows of up
// to kTopkStage candidates; longer rows are read from memory in every pass),
// then take_best's radix select and index-ordered compaction pick the k.
// The staging requests kTopkPer scores per thread before storing any, and
// the first of them together with the sequence length, so a row of up to
// 256 * kTopkPer blocks costs one round trip to memory (one load at a time
// was a round trip per 256 blocks, most of the kernel's time).
constexpr int kTopkStage = 16384;
constexpr int kTopkPer = 8;

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ seq_lens,
                                                   int32_t Hkv, int32_t NBmax, int32_t k, int32_t n_sink,
                                                   int32_t n_recent, int32_t max_sel, int32_t* __restrict__ idx,
                                                   int32_t* __restrict__ n_sel) {
  __shared__ uint32_t keys[kTopkStage];
  __shared__ __attribute__((aligned(16))) uint32_t hist[4096];
  __shared__ uint32_t cand[256];
  __shared__ int scan4[4];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_rem;
  const int unit = blockIdx.x, b = unit / Hkv, tid = threadIdx.x;
  const float* row = scores + (size_t)unit * NBmax;
  int32_t* out = idx + (size_t)unit * max_sel;
  const int Lraw = seq_lens ? seq_lens[b] : NBmax * kBlock;
  // the row's first scores, requested before the length is known (with k = 0
  // no score is read: scores may be null)
  float x0[kTopkPer];
#pragma unroll
  for (int u = 0; u < kTopkPer; ++u) {
    const int jb = u * 256 + tid;
    x0[u] = (k > 0 && jb < NBmax) ? row[jb] : 0.f;
  }
  // the histogram's clear overlaps those loads
  for (int i = tid; i < 4096; i += 256) hist[i] = 0;
  const int L = clampi(Lraw, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;

  // forced blocks: [0, sink_hi) and [rec_lo, nb); candidates: [sink_hi, rec_lo)
  const int sink_hi = min(n_sink, nb);
  const int rec_lo = max(nb - n_recent, sink_hi);
  const int ncand = rec_lo - sink_hi;
  const bool staged = ncand <= kTopkStage;
  if (staged && k > 0) {
    // blocks jb = base + u * 256 + tid of the row; candidates go to keys[jb - sink_hi]
    for (int base = 0; base < rec_lo; base += 256 * kTopkPer) {
      float x[kTopkPer];
#pragma unroll
      for (int u = 0; u < kTopkPer; ++u) {
        const int jb = base + u * 256 + tid;
        x[u] = base == 0 ? x0[u] : (jb < rec_lo ? row[jb] : 0.f);
      }
#pragma unroll
      for (int u = 0; u < kTopkPer; ++u) {
        const int jb = base + u * 256 + tid;
        if (jb >= sink_hi && jb < rec_lo) keys[jb - sink_hi] = score_key(x[u]);
      }
    }
  }
  __syncthreads();
  auto key = [&](int i) { return staged ? keys[i] : score_key(row[sink_hi + i]); };
  auto put = [&](int i, int r) {
    if (sink_hi + r < max_sel) out[sink_hi + r] = sink_hi + i;
  };
  auto all = [](int) { return true; };
  // staged keys are cheap to read twice: one histogram pass usually decides
  const int npick = staged ? take_best<true, true>(ncand, k, key, all, put, hist, scan4, &sh_prefix, &sh_rem, cand,
                                                  true)
                           : take_best<false, true>(ncand, k, key, all, put, hist, scan4, &sh_prefix, &sh_rem);
  for (int j = tid; j < sink_hi; j += 256)
    if (j < max_sel) out[j] = j;
  for (int j = rec_lo + tid; j < nb; j += 256) {
    const int o = sink_hi + npick + (j - rec_lo);
    if (o < max_sel) out[o] = j;
  }
  const int total = sink_hi + npick + (nb - rec_lo);
  for (int o = total + tid; o < max_sel; o += 256) out[o] = -1;
  if (tid == 0) n_sel[unit] = min(total, max_sel);
}

// Rows of at most kTopkSmall blocks (every row of a cache of up to 128K
// tokens): thread t holds the keys of blocks t, t + 256, ... in registers
// (round u = block / 256), so no phase reads keys back from LDS one load at
// a time.  The k-th key comes from the 4096-bin histogram of the top 12 key
// bits and the rank of the <= 256 keys in its bin, as in select_wide (an
// 8-bit radix select over the keys staged in LDS when the bin holds more).
// The chosen blocks are compacted in block order from per-round counts
// (wave ballots, then per-wave totals): block 256 u + t follows every block
// of rounds before u and the blocks of round u held by lower threads.
constexpr int kTopkSmall = 2048;
constexpr int kSmallPer = kTopkSmall / 256;

__global__ __launch_bounds__(256) void topk_small_kernel(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ seq_lens, int32_t Hkv,
                                                         int32_t NBmax, int32_t k, int32_t n_sink, int32_t n_recent,
                                                         int32_t max_sel, int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ n_sel) {
  __shared__ uint32_t keys[kTopkSmall];  // the radix select's copy of the keys
  __shared__ __attribute__((aligned(16))) uint32_t hist[4096];
  __shared__ uint32_t cand[256];
  __shared__ int scan4[4];
  __shared__ int counts[2][kSmallPer][4];  // per round and wave: keys above, and equal to, the k-th key
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_rem, sh_bin, sh_bin_rem, sh_bin_cnt, sh_cnt;
  const int unit = blockIdx.x, b = unit / Hkv, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* row = scores + (size_t)unit * NBmax;
  int32_t* out = idx + (size_t)unit * max_sel;
  const int Lraw = seq_lens ? seq_lens[b] : NBmax * kBlock;
  // every score of the row is requested before the length is known (with
  // k = 0 no score is read: scores may be null)
  float x[kSmallPer];
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u) {
    const int jb = u * 256 + tid;
    x[u] = (k > 0 && jb < NBmax) ? row[jb] : 0.f;
  }
  for (int i = tid; i < 4096; i += 256) hist[i] = 0;
  if (tid == 0) sh_cnt = 0;
  const int L = clampi(Lraw, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;
  // forced blocks: [0, sink_hi) and [rec_lo, nb); candidates: [sink_hi, rec_lo)
  const int sink_hi = min(n_sink, nb);
  const int rec_lo = max(nb - n_recent, sink_hi);
  const int ncand = rec_lo - sink_hi;
  const int kq = min(k, ncand);
  const bool ranked = kq > 0 && kq < ncand;
  uint32_t key[kSmallPer];
  bool in[kSmallPer];
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u) {
    const int jb = u * 256 + tid;
    in[u] = jb >= sink_hi && jb < rec_lo;
    key[u] = in[u] ? score_key(x[u]) : 0u;
  }
  __syncthreads();  // the histogram is clear

  // the k-th largest key (thr) and how many keys equal to it are taken
  uint32_t thr = 0;
  int need_eq = 0;
  if (ranked) {
#pragma unroll
    for (int u = 0; u < kSmallPer; ++u)
      if (in[u]) atomicAdd(&hist[key[u] >> 20], 1u);
    __syncthreads();
    {
      int fb, fr, fn;
      if (kth_bin(hist, kq, scan4, fb, fr, fn)) {
        sh_bin = fb;
        sh_bin_rem = fr;  // how many of the bin's keys are among the kq
        sh_bin_cnt = fn;
      }
    }
    __syncthreads();
    const uint32_t bin = (uint32_t)sh_bin;
    const int rem = sh_bin_rem, cnt = sh_bin_cnt;
    if (cnt <= 256) {
      // the bin's keys, in any order (the rank below does not depend on it):
      // one atomic per wave reserves room for the wave's keys of every round
      uint64_t mk[kSmallPer];
      int wtot = 0;
#pragma unroll
      for (int u = 0; u < kSmallPer; ++u) {
        mk[u] = (uint64_t)__ballot(in[u] && (key[u] >> 20) == bin);
        wtot += __popcll(mk[u]);
      }
      int base = 0;
      if (lane == 0 && wtot > 0) base = atomicAdd(&sh_cnt, wtot);
      base = __shfl(base, 0);
#pragma unroll
      for (int u = 0; u < kSmallPer; ++u) {
        if ((mk[u] >> lane) & 1) cand[base + lanes_below(mk[u])] = key[u];
        base += __popcll(mk[u]);
      }
      __syncthreads();
      if (tid < cnt) {
        const uint32_t y = cand[tid];
        int gt = 0, ge = 0;
#pragma unroll 8
        for (int c = 0; c < cnt; ++c) {
          const uint32_t z = cand[c];
          gt += z > y ? 1 : 0;
          ge += z >= y ? 1 : 0;
        }
        if (gt < rem && rem <= ge) {  // y is the rem-th largest of the bin (equal keys write equal values)
          sh_prefix = y;
          sh_rem = rem - gt;
        }
      }
      __syncthreads();
      thr = sh_prefix;
      need_eq = sh_rem;
    } else {
      // heavy ties or clustering: an exact 8-bit radix select over the keys in LDS
#pragma unroll
      for (int u = 0; u < kSmallPer; ++u)
        if (in[u]) keys[u * 256 + tid - sink_hi] = key[u];
      __syncthreads();
      radix_select(
          ncand, kq, [&](int i) { return keys[i]; }, [](int) { return true; }, hist, scan4, &sh_prefix, &sh_rem,
          thr, need_eq);
    }
  }

  // per round: keys above the threshold (every candidate when nothing is
  // ranked, none when k = 0) and keys equal to it, counted per wave
  bool gtf[kSmallPer], eqf[kSmallPer];
  int gi[kSmallPer], ei[kSmallPer];  // the wave's lanes below this one with the flag
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u) {
    gtf[u] = kq > 0 && in[u] && (!ranked || key[u] > thr);
    eqf[u] = ranked && in[u] && key[u] == thr;
    const uint64_t gm = (uint64_t)__ballot(gtf[u]), em = (uint64_t)__ballot(eqf[u]);
    gi[u] = lanes_below(gm);
    ei[u] = lanes_below(em);
    if (lane == 0) {
      counts[0][u][w] = __popcll(gm);
      counts[1][u][w] = __popcll(em);
    }
  }
  __syncthreads();
  int gt_base = 0, eq_base = 0;  // keys above / equal in the rounds before u
#pragma unroll
  for (int u = 0; u < kSmallPer; ++u) {
    int g_before = gt_base + gi[u], e_before = eq_base + ei[u];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int gv = counts[0][u][v], ev = counts[1][u][v];
      g_before += v < w ? gv : 0;
      e_before += v < w ? ev : 0;
      gt_base += gv;
      eq_base += ev;
    }
    if (gtf[u] || (eqf[u] && e_before < need_eq)) {
      const int o = sink_hi + g_before + min(e_before, need_eq);
      if (o < max_sel) out[o] = u * 256 + tid;
    }
  }
  const int npick = gt_base + (ranked ? need_eq : 0);
  for (int j = tid; j < sink_hi; j += 256)
    if (j < max_sel) out[j] = j;
  for (int j = rec_lo + tid; j < nb; j += 256) {
    const int o = sink_hi + npick + (j - rec_lo);
    if (o < max_sel) out[o] = j;
  }
  const int total = sink_hi + npick + (nb - rec_lo);
  for (int o = total + tid; o < max_sel; o += 256) out[o] = -1;
  if (tid == 0) n_sel[unit] = min(total, max_sel);
}

// ---- importance order: one workgroup per (b, kv head) -------------------
// Block 0 first, then blocks 1 .. nb-1 by descending score, lower index first
// among equal scores ("ART" summary, §2.4, importance-first visit order).
// The nb - 1 keys (inverted score key << 32 | block) are sorted ascending by
// a bitonic network in LDS, padded to a power of two with all-ones keys;
// stages whose partners lie within one wave's keys run without a barrier.
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
  // one compare-exchange stage: pair (i, i + j) with i = 2 j floor(pr / j) +
  // pr mod j, j = 2^lj
  auto stage = [&](int kk, int j, int lj) {
    for (int pr = tid; pr < (n >> 1); pr += 1024) {
      const int i = ((pr >> lj) << (lj + 1)) | (pr & (j - 1));
      const uint64_t x = key[i], y = key[i + j];
      const bool up = (i & kk) == 0;
      if ((x > y) == up) {
        key[i] = y;
        key[i + j] = x;
      }
    }
  };
  for (int kk = 2, lk = 1; kk <= n; kk <<= 1, ++lk) {
    int j = kk >> 1, lj = lk - 1;
    // partners 64 or more apart may belong to other waves: a barrier a stage
    for (; j >= 64; j >>= 1, --lj) {
      stage(kk, j, lj);
      __syncthreads();
    }
    // closer partners: the 32 pairs pr = 32 c .. 32 c + 31 of a wave cover the
    // aligned 64 keys 64 c .. 64 c + 63 for every j <= 32, so the rest of this
    // merge needs no workgroup barrier
    for (; j > 0; j >>= 1, --lj) {
      stage(kk, j, lj);
      wave_lds_exchange();
    }
    __syncthreads();
  }
  for (int i = tid; i < NBmax; i += 1024)
    out[i] = i == 0 ? (nb > 0 ? 0 : -1) : (i < nb ? (int32_t)(uint32_t)key[i - 1] : -1);
}

// ---- two-level selection ---------------------------------------------------
// Super-block centroids from block centroids: the token-count-weighted mean
// of the block means is the mean of the super-block's keys.
template <int D>
__global__ __launch_bounds__(256) void super_centroid_kernel(const float* __restrict__ C,
                                                             const int32_t* __restrict__ seq_lens,
                                                             float* __restrict__ C2, int32_t Hkv, int32_t NBmax,
                                                             int32_t NSmax, int32_t group) {
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= NSmax) return;
  const int g = blockIdx.y, b = blockIdx.z, lane = threadIdx.x & 63;
  const int L = clampi(seq_lens ? seq_lens[b] : NBmax * kBlock, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;
  const size_t unit = (size_t)b * Hkv + g;
  float* out = C2 + (unit * NSmax + s) * D;
  const int j0 = s * group, j1 = min(j0 + group, nb);
  if (j0 >= j1) {
    for (int c = lane; c < D; c += 64) out[c] = 0.f;
    return;
  }
  const float* crow = C + (unit * NBmax) * D;
  float acc[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
  for (int j = j0; j < j1; ++j) {
    const float nj = (float)min(kBlock, L - j * kBlock);
#pragma unroll
    for (int e = 0; e < D / 64; ++e) acc[e] = fmaf(nj, crow[(size_t)j * D + lane + 64 * e], acc[e]);
  }
  const float n = (float)(min(L, j1 * kBlock) - j0 * kBlock);
#pragma unroll
  for (int e = 0; e < D / 64; ++e) out[lane + 64 * e] = acc[e] / n;
}

// Scores n centroid rows against the LDS query qs: 16-byte loads, D/4 lanes
// per row, and 8 load instructions in flight per wave before any reduction.
// put(r, score) is called by one lane per row.
template <int D, typename RowF, typename PutF>
__device__ void score_rows(int n, const float* qs, RowF row_of, PutF put, float scale) {
  constexpr int LPR = D / 4, RPI = 64 / LPR, NB8 = 8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane % LPR, rsub = lane / LPR;
  const f32x4 qv = *(const f32x4*)(qs + 4 * c);
  for (int base = w * RPI * NB8; base < n; base += 4 * RPI * NB8) {
    f32x4 x[NB8];
#pragma unroll
    for (int it = 0; it < NB8; ++it) {
      const int r = base + it * RPI + rsub;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      x[it] = r < n ? *(const f32x4*)(row_of(r) + 4 * c) : z;
    }
#pragma unroll
    for (int it = 0; it < NB8; ++it) {
      float v = qv[0] * x[it][0];
      v = fmaf(qv[1], x[it][1], v);
      v = fmaf(qv[2], x[it][2], v);
      v = fmaf(qv[3], x[it][3], v);
      v = row16_sum(v);
      if constexpr (LPR == 32) v = xrow16_sum(v);
      const int r = base + it * RPI + rsub;
      if (c == 0 && r < n) put(r, v * scale);
    }
  }
}

constexpr int kCoarseCap = kTwoLevelMaxSuper;
constexpr int kCandCap = kTwoLevelMaxCand;

// One 256-thread workgroup per (b, kv head): coarse scores of the super-
// blocks that hold a non-forced block, the k_coarse best opened, fine scores
// of the non-forced blocks inside them, the k best taken; forced sink and
// window blocks added; ascending output, -1 padded.
template <typename T, int D>
__global__ __launch_bounds__(256) void two_level_kernel(const void* __restrict__ q, const float* __restrict__ C,
                                                        const float* __restrict__ C2,
                                                        const int32_t* __restrict__ seq_lens, int32_t Hq,
                                                        int32_t Hkv, int32_t NBmax, int32_t NSmax, int32_t group,
                                                        int32_t k_coarse, int32_t k, int32_t n_sink,
                                                        int32_t n_recent, int32_t max_sel, float scale,
                                                        int32_t* __restrict__ idx, int32_t* __restrict__ n_sel) {
  __shared__ __align__(16) float qs[D];
  __shared__ float csc[kCoarseCap];
  __shared__ unsigned char opened[kCoarseCap];
  __shared__ int cand[kCandCap];
  __shared__ float fsc[kCandCap];
  __shared__ uint32_t hist[256];
  __shared__ int scan4[4];
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_rem;
  const int unit = blockIdx.x, b = unit / Hkv, g = unit % Hkv;
  const int tid = threadIdx.x;
  const int G = Hq / Hkv;
  const int L = clampi(seq_lens ? seq_lens[b] : NBmax * kBlock, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;
  const int sink_hi = min(n_sink, nb);
  const int rec_lo = max(nb - n_recent, sink_hi);
  int32_t* out = idx + (size_t)unit * max_sel;

  for (int c = tid; c < D; c += 256) {
    float a = 0.f;
    for (int h = 0; h < G; ++h) a += elem_f32((const T*)q + ((size_t)b * Hq + (size_t)g * G + h) * D, c);
    qs[c] = a;
  }
  // super-blocks holding a block of [sink_hi, rec_lo) form the range [es0, es1)
  const bool any = sink_hi < rec_lo;
  const int es0 = any ? sink_hi / group : 0, es1 = any ? (rec_lo + group - 1) / group : 0;
  const int nes = es1 - es0;
  __syncthreads();
  const float* C2u = C2 + (size_t)unit * NSmax * D;
  score_rows<D>(
      nes, qs, [&](int i) { return C2u + (size_t)(es0 + i) * D; }, [&](int i, float v) { csc[i] = v; }, scale);
  for (int i = tid; i < nes; i += 256) opened[i] = 0;
  __syncthreads();
  auto all = [](int) { return true; };
  take_best(
      nes, k_coarse, [&](int i) { return score_key(csc[i]); }, all, [&](int i, int) { opened[i] = 1; }, hist,
      scan4, &sh_prefix, &sh_rem);
  // candidates: the non-forced blocks of the opened super-blocks, ascending
  const int CH = (nes + 255) / 256;
  const int i0 = min(tid * CH, nes), i1 = min(i0 + CH, nes);
  auto m_lo = [&](int i) { return max((es0 + i) * group, sink_hi); };
  auto m_hi = [&](int i) { return min((es0 + i + 1) * group, rec_lo); };
  int cnt = 0;
  for (int i = i0; i < i1; ++i)
    if (opened[i]) cnt += m_hi(i) - m_lo(i);
  int ncand;
  int pos = block_exscan(cnt, &ncand, scan4);
  for (int i = i0; i < i1; ++i)
    if (opened[i])
      for (int j = m_lo(i); j < m_hi(i); ++j)
        if (pos < kCandCap) cand[pos++] = j;
  ncand = min(ncand, kCandCap);
  __syncthreads();
  const float* Cu = C + (size_t)unit * NBmax * D;
  score_rows<D>(
      ncand, qs, [&](int i) { return Cu + (size_t)cand[i] * D; }, [&](int i, float v) { fsc[i] = v; }, scale);
  __syncthreads();
  const int npick = take_best(
      ncand, k, [&](int i) { return score_key(fsc[i]); }, all,
      [&](int i, int r) {
        if (sink_hi + r < max_sel) out[sink_hi + r] = cand[i];
      },
      hist, scan4, &sh_prefix, &sh_rem);
  for (int j = tid; j < sink_hi; j += 256)
    if (j < max_sel) out[j] = j;
  for (int j = rec_lo + tid; j < nb; j += 256) {
    const int o = sink_hi + npick + (j - rec_lo);
    if (o < max_sel) out[o] = j;
  }
  const int total = sink_hi + npick + (nb - rec_lo);
  for (int o = total + tid; o < max_sel; o += 256) out[o] = -1;
  if (tid == 0) n_sel[unit] = min(total, max_sel);
}

}  // namespace

hipError_t launch_build_centroids(const void* k, const int32_t* seq_lens, float* c, int32_t B,
                                  int32_t Hkv, int32_t d, int32_t NBmax, int32_t dtype,
                                  hipStream_t st, PagedK pg) {
  if (B == 0) return hipSuccess;
  const dim3 grid((NBmax + 3) / 4, Hkv, B);
  if (dtype == 1) {
    if (d == 128)
      centroid_kernel<__bf16, 128><<<grid, 256, 0, st>>>(k, seq_lens, c, Hkv, NBmax, pg);
    else
      centroid_kernel<__bf16, 64><<<grid, 256, 0, st>>>(k, seq_lens, c, Hkv, NBmax, pg);
  } else {
    if (d == 128)
      centroid_kernel<float, 128><<<grid, 256, 0, st>>>(k, seq_lens, c, Hkv, NBmax, pg);
    else
      centroid_kernel<float, 64><<<grid, 256, 0, st>>>(k, seq_lens, c, Hkv, NBmax, pg);
  }
  return hipGetLastError();
}

hipError_t launch_update_centroids(const void* k, const int32_t* seq_lens, const int32_t* prev_lens, float* c,
                                   int32_t B, int32_t Hkv, int32_t d, int32_t NBmax, int32_t dtype,
                                   int32_t span_hint, hipStream_t st, PagedK pg) {
  if (B == 0) return hipSuccess;
  const int X = clampi((span_hint + 3) / 4, 1, (NBmax + 3) / 4);
  const dim3 grid(X, Hkv, B);
  if (dtype == 1) {
    if (d == 128)
      centroid_update_kernel<__bf16, 128><<<grid, 256, 0, st>>>(k, seq_lens, prev_lens, c, Hkv, NBmax, pg);
    else
      centroid_update_kernel<__bf16, 64><<<grid, 256, 0, st>>>(k, seq_lens, prev_lens, c, Hkv, NBmax, pg);
  } else {
    if (d == 128)
      centroid_update_kernel<float, 128><<<grid, 256, 0, st>>>(k, seq_lens, prev_lens, c, Hkv, NBmax, pg);
    else
      centroid_update_kernel<float, 64><<<grid, 256, 0, st>>>(k, seq_lens, prev_lens, c, Hkv, NBmax, pg);
  }
  return hipGetLastError();
}

hipError_t launch_score(const void* q, const float* c, const int32_t* seq_lens, float* scores,
                        int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t NBmax,
                        int32_t dtype, float scale, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const dim3 grid((NBmax + 63) / 64, Hkv, B);
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
  if (NBmax <= kTopkSmall)
    topk_small_kernel<<<dim3(B * Hkv), 256, 0, st>>>(scores, seq_lens, Hkv, NBmax, k, n_sink, n_recent, max_sel,
                                                     idx, n_sel);
  else
    topk_kernel<<<dim3(B * Hkv), 256, 0, st>>>(scores, seq_lens, Hkv, NBmax, k, n_sink, n_recent, max_sel, idx,
                                               n_sel);
  return hipGetLastError();
}

hipError_t launch_super_centroids(const float* c, const int32_t* seq_lens, float* c2, int32_t B, int32_t Hkv,
                                  int32_t d, int32_t NBmax, int32_t group, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const int NS = (NBmax + group - 1) / group;
  const dim3 grid((NS + 3) / 4, Hkv, B);
  if (d == 128)
    super_centroid_kernel<128><<<grid, 256, 0, st>>>(c, seq_lens, c2, Hkv, NBmax, NS, group);
  else
    super_centroid_kernel<64><<<grid, 256, 0, st>>>(c, seq_lens, c2, Hkv, NBmax, NS, group);
  return hipGetLastError();
}

hipError_t launch_two_level(const void* q, const float* c, const float* c2, const int32_t* seq_lens, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t d, int32_t NBmax, int32_t dtype, float scale,
                            int32_t group, int32_t k_coarse, int32_t k, int32_t n_sink, int32_t n_recent,
                            int32_t max_sel, int32_t* idx, int32_t* n_sel, hipStream_t st) {
  if (B == 0) return hipSuccess;
  const int NS = (NBmax + group - 1) / group;
  const dim3 grid(B * Hkv);
#define SKV_TWO_LEVEL(T, D)                                                                                  \
  two_level_kernel<T, D><<<grid, 256, 0, st>>>(q, c, c2, seq_lens, Hq, Hkv, NBmax, NS, group, k_coarse, k, \
                                               n_sink, n_recent, max_sel, scale, idx, n_sel)
  if (dtype == 1) {
    if (d == 128)
      SKV_TWO_LEVEL(__bf16, 128);
    else
      SKV_TWO_LEVEL(__bf16, 64);
  } else {
    if (d == 128)
      SKV_TWO_LEVEL(float, 128);
    else
      SKV_TWO_LEVEL(float, 64);
  }
#undef SKV_TWO_LEVEL
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
