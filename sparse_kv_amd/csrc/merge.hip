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

// One workgroup (4 wave64s) per output row.  Wave w takes the splits
// s = w, w + 4, ...; within a wave the lanes first hold one split each (max
// and weights, staged in LDS), then d/64 channels each while the split
// outputs are accumulated.  The 4 partial sums meet in LDS.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(int32_t rows, int32_t S, const float* __restrict__ m,
                                                    const float* __restrict__ l, const float* __restrict__ o,
                                                    float* __restrict__ out, float* __restrict__ m_out,
                                                    float* __restrict__ l_out) {
  constexpr int PER = D / 64;
  constexpr int NW = 4;
  __shared__ float red[NW][D];
  __shared__ float red_w[NW], red_m[NW];
  __shared__ float wts[NW][64];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const float* mr = m + (size_t)row * S;
  const float* lr = l + (size_t)row * S;

  // global max over the non-empty splits
  float mx = -INFINITY;
  for (int s = w + NW * lane; s < S; s += NW * 64)
    if (lr[s] > 0.f) mx = fmaxf(mx, mr[s]);
  mx = wave_max(mx);
  if (lane == 0) red_m[w] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float wsum = 0.f;
  if (M != -INFINITY) {
    for (int s0 = w; s0 < S; s0 += NW * 64) {
      // lane i holds the weight of split s0 + NW * i
      const int s = s0 + NW * lane;
      float wt = 0.f;
      if (s < S) {
        const float ls = lr[s];
        wt = ls > 0.f ? ls * fast_exp2((mr[s] - M) * kLog2e) : 0.f;
      }
      wsum += wt;
      wts[w][lane] = wt;  // read back by the same wave only
      const int n = min(64, (S - s0 + NW - 1) / NW);
      const float* ob = o + ((size_t)row * S + s0) * D + lane * PER;
#pragma unroll 8
      for (int i = 0; i < n; ++i) {
        const float f = wts[w][i];
        const float* os = ob + (size_t)NW * i * D;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const float x = os[k];
          acc[k] = f != 0.f ? fmaf(f, x, acc[k]) : acc[k];  // empty splits never touch acc
        }
      }
    }
  }
  wsum = wave_sum(wsum);
#pragma unroll
  for (int k = 0; k < PER; ++k) red[w][lane * PER + k] = acc[k];
  if (lane == 0) red_w[w] = wsum;
  __syncthreads();
  if (w == 0) {
    const float L = red_w[0] + red_w[1] + red_w[2] + red_w[3];
    float* dst = out + (size_t)row * D + lane * PER;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int c = lane * PER + k;
      const float a = red[0][c] + red[1][c] + red[2][c] + red[3][c];
      dst[k] = L > 0.f ? a / L : 0.f;
    }
    if (lane == 0) {
      if (m_out) m_out[row] = L > 0.f ? M : -INFINITY;
      if (l_out) l_out[row] = L;
    }
  }
}

}  // namespace

hipError_t launch_merge(int32_t rows, int32_t S, int32_t d, const float* m, const float* l,
                        const float* o, float* out, float* m_out, float* l_out, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const dim3 grid(rows);
  if (d == 128)
    merge_kernel<128><<<grid, 256, 0, st>>>(rows, S, m, l, o, out, m_out, l_out);
  else
    merge_kernel<64><<<grid, 256, 0, st>>>(rows, S, m, l, o, out, m_out, l_out);
  return hipGetLastError();
}

}  // namespace skv
