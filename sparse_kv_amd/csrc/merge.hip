// Exact online-softmax merge of partial attention states, for gfx950.
//
// Method: per-shard (here: per-split) attention states are combined into the
// exact global attention by the online softmax merge ("Pulsar Attention"
// summary, Phase 2): M = max_r m_r over non-empty states,
// w_r = l_r exp(m_r - M), out = sum_r w_r o_r / sum_r w_r.
//
#include "device_common.hpp"
#include "kernels.hpp"

namespace skv {
namespace {

// One wave64 per output row, four rows per workgroup.  Lane i holds channels
// i * d/64 .. of the output.  The first kChunk split outputs of the row are
// loaded together with the split states, so a merge of up to kChunk splits
// costs one round trip to memory; further splits follow kChunk at a time.
// A state with l = 0 is empty: it never touches the sums, whatever its o.
constexpr int kChunk = 32;

template <int PER>
__device__ __forceinline__ void load_row_part(const float* src, float (&x)[PER]) {
  if constexpr (PER == 2) {
    const float2 v = *(const float2*)src;
    x[0] = v.x;
    x[1] = v.y;
  } else {
    x[0] = src[0];
  }
}

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(int32_t rows, int32_t S, const float* __restrict__ m,
                                                    const float* __restrict__ l, const float* __restrict__ o,
                                                    float* __restrict__ out, float* __restrict__ m_out,
                                                    float* __restrict__ l_out) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (row >= rows) return;
  const float* mr = m + (size_t)row * S;
  const float* lr = l + (size_t)row * S;
  const float* orow = o + (size_t)row * S * D + lane * PER;

  // the first chunk of split outputs, in flight with the states
  float x[kChunk][PER];
#pragma unroll
  for (int i = 0; i < kChunk; ++i) {
    if (i < S) {
      load_row_part<PER>(orow + (size_t)i * D, x[i]);
    } else {
#pragma unroll
      for (int k = 0; k < PER; ++k) x[i][k] = 0.f;
    }
  }
  // states of splits lane, lane + 64, ...: the first 64 stay in registers
  const float m0 = lane < S ? mr[lane] : -INFINITY;
  const float l0 = lane < S ? lr[lane] : 0.f;
  float mx = l0 > 0.f ? m0 : -INFINITY;
  for (int s = lane + 64; s < S; s += 64)
    if (lr[s] > 0.f) mx = fmaxf(mx, mr[s]);
  const float M = wave_max(mx);

  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < S; s0 += 64) {
      float ls = l0, ms = m0;
      if (s0 > 0) {
        const int s = s0 + lane;
        ls = s < S ? lr[s] : 0.f;
        ms = s < S ? mr[s] : -INFINITY;
      }
      // lane i holds the weight of split s0 + i
      const float wt = ls > 0.f ? ls * fast_exp2((ms - M) * kLog2e) : 0.f;
      wsum += wt;
      const int n = min(64, S - s0);
      for (int c = 0; c < n; c += kChunk) {
        float y[kChunk][PER];
        if (s0 + c == 0) {
#pragma unroll
          for (int i = 0; i < kChunk; ++i)
#pragma unroll
            for (int k = 0; k < PER; ++k) y[i][k] = x[i][k];
        } else {
#pragma unroll
          for (int i = 0; i < kChunk; ++i) {
            if (c + i < n) {
              load_row_part<PER>(orow + (size_t)(s0 + c + i) * D, y[i]);
            } else {
#pragma unroll
              for (int k = 0; k < PER; ++k) y[i][k] = 0.f;
            }
          }
        }
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
          if (c + i < n) {
            const float f = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), c + i));
#pragma unroll
            for (int k = 0; k < PER; ++k) acc[k] = f != 0.f ? fmaf(f, y[i][k], acc[k]) : acc[k];
          }
        }
      }
    }
  }
  const float L = wave_sum(wsum);
  float* dst = out + (size_t)row * D + lane * PER;
#pragma unroll
  for (int k = 0; k < PER; ++k) dst[k] = L > 0.f ? acc[k] / L : 0.f;
  if (lane == 0) {
    if (m_out) m_out[row] = L > 0.f ? M : -INFINITY;
    if (l_out) l_out[row] = L;
  }
}

// Two-level merge in one launch: the S = shards * inner states of a row are
// merged per shard (inner consecutive states) into shard states (M_k, L_k,
// O_k), and those across shards into the output: with w_s = l_s e^(m_s - M_k)
// and W_k = L_k e^(M_k - M), out = sum_k W_k O_k / sum_k W_k and
// O_k = sum_{s in k} w_s o_s / L_k, i.e. out = sum_s (W_k / L_k) w_s o_s /
// sum_k W_k -- the merge of the inner states followed by the merge of the
// shard states, as one weighted sum.  One wave per row, S <= 64: lane s holds
// state s, and every split output is loaded in one round trip.
template <int D>
__global__ __launch_bounds__(256) void merge2_kernel(int32_t rows, int32_t shards, int32_t inner,
                                                     const float* __restrict__ m, const float* __restrict__ l,
                                                     const float* __restrict__ o, float* __restrict__ out) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (row >= rows) return;
  const int S = shards * inner;
  const float* orow = o + (size_t)row * S * D + lane * PER;
  // every split output, in flight with the states
  float y[64][PER];
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (i < S) {
      load_row_part<PER>(orow + (size_t)i * D, y[i]);
    } else {
#pragma unroll
      for (int e = 0; e < PER; ++e) y[i][e] = 0.f;
    }
  }
  const float ms = lane < S ? m[(size_t)row * S + lane] : -INFINITY;
  const float ls = lane < S ? l[(size_t)row * S + lane] : 0.f;
  const int my_shard = lane / inner;
  // first level: shard k's (M_k, L_k) into lane k; w_s into lane s
  float Mk = -INFINITY, Lk = 0.f, wt = 0.f;
  for (int k = 0; k < shards; ++k) {
    const bool mine = lane < S && my_shard == k && ls > 0.f;
    const float M = wave_max(mine ? ms : -INFINITY);
    const float w = mine ? ls * fast_exp2((ms - M) * kLog2e) : 0.f;
    if (my_shard == k) wt = w;
    const float L = wave_sum(w);
    if (lane == k) {
      Mk = L > 0.f ? M : -INFINITY;
      Lk = L;
    }
  }
  // second level: the shard weights W_k, and each split's coefficient
  const float Mall = wave_max(Lk > 0.f ? Mk : -INFINITY);
  const float Wk = Lk > 0.f ? Lk * fast_exp2((Mk - Mall) * kLog2e) : 0.f;
  const float Wsum = wave_sum(Wk);
  const int src = min(my_shard, 63);
  const float Ws = __shfl(Wk, src), Ls = __shfl(Lk, src);
  const float coef = (wt > 0.f && Ls > 0.f) ? wt * (Ws / Ls) : 0.f;
  float res[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) res[e] = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (i < S) {
      const float f = readlane(coef, i);
#pragma unroll
      for (int e = 0; e < PER; ++e) res[e] = f != 0.f ? fmaf(f, y[i][e], res[e]) : res[e];
    }
  }
  float* dst = out + (size_t)row * D + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[e] = Wsum > 0.f ? res[e] / Wsum : 0.f;
}

}  // namespace

hipError_t launch_merge2(int32_t rows, int32_t shards, int32_t inner, int32_t d, const float* m, const float* l,
                         const float* o, float* out, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4);
  if (d == 128)
    merge2_kernel<128><<<grid, 256, 0, st>>>(rows, shards, inner, m, l, o, out);
  else
    merge2_kernel<64><<<grid, 256, 0, st>>>(rows, shards, inner, m, l, o, out);
  return hipGetLastError();
}

hipError_t launch_merge(int32_t rows, int32_t S, int32_t d, const float* m, const float* l,
                        const float* o, float* out, float* m_out, float* l_out, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4);
  if (d == 128)
    merge_kernel<128><<<grid, 256, 0, st>>>(rows, S, m, l, o, out, m_out, l_out);
  else
    merge_kernel<64><<<grid, 256, 0, st>>>(rows, S, m, l, o, out, m_out, l_out);
  return hipGetLastError();
}

}  // namespace skv
