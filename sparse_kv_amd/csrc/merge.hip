// Exact online-softmax merge of partial attention states, for gfx950.
//
// Method: per-shard (here: per-split) attention states are combined into the
// exact global attention by the online softmax merge ("Pulsar Attention"
// summary, Phase 2): M = max_r m_r over non-empty states,
// w_r = l_r exp(m_r - M), out = sum_r w_r o_r / sum_r w_r.
//
// One wave64 per output row; each lane owns d/64 consecutive channels.  The
// split loop reads each state once; the (m, l) reads are wave-uniform.
#include "device_common.hpp"
#include "kernels.hpp"

namespace skv {
namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(int32_t rows, int32_t S, const float* __restrict__ m,
                                                    const float* __restrict__ l, const float* __restrict__ o,
                                                    float* __restrict__ out, float* __restrict__ m_out,
                                                    float* __restrict__ l_out) {
  constexpr int PER = D / 64;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const float* mr = m + (size_t)row * S;
  const float* lr = l + (size_t)row * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s)
    if (lr[s] > 0.f) M = fmaxf(M, mr[s]);
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float L = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ls = lr[s];
      if (ls > 0.f) {
        const float f = ls * fast_exp2((mr[s] - M) * kLog2e);
        L += f;
        const float* os = o + ((size_t)row * S + s) * D + lane * PER;
#pragma unroll
        for (int k = 0; k < PER; ++k) acc[k] = fmaf(f, os[k], acc[k]);
      }
    }
  }
  float* dst = out + (size_t)row * D + lane * PER;
#pragma unroll
  for (int k = 0; k < PER; ++k) dst[k] = L > 0.f ? acc[k] / L : 0.f;
  if (lane == 0) {
    if (m_out) m_out[row] = L > 0.f ? M : -INFINITY;
    if (l_out) l_out[row] = L;
  }
}

}  // namespace

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
