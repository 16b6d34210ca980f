// Decode attention with ART run-time termination, for gfx950.
//
// Method ("ART (Attention Run-time Termination)" summary): KV blocks are
// folded into the streaming attention state in a visit order (§2.1, §2.4,
// block 0 first); after each fold a small probe of the partial output is
// compared with the previous one -- magnitude change and direction change
// (§2.2) -- and attention stops once both stay below their thresholds for
// p consecutive blocks (§2.3).
//
// One workgroup = one (b, kv head); its 8 wave64s work in rounds.  In round
// r wave w computes the softmax state of the block at visit position 8r+w
// on its own (block-local max, denominator, P.V with the same MFMA-logit /
// fp32-VALU-P.V scheme as the split-KV kernel) and publishes the block's
// (m, l) and the probe channels of its P.V in LDS.  Wave 0 then replays the
// fold of the round's blocks strictly in visit order on the probe channels
// only -- one 16-lane row per query head, lane = probe channel -- which is
// all the stop rule reads, and records each head's stop position.  Finally
// every wave adds its block into its private running state for the heads
// whose stop is not before that position.  The decisions are therefore
// exactly those of one-block-at-a-time streaming; the cost of the round
// structure is read-ahead of at most 7 blocks past the last stop, reported
// in blocks_fetched.  When every head of the group has stopped the
// workgroup ends; the 8 private states are merged through LDS at the end.
#include "device_common.hpp"
#include "kernels.hpp"

namespace skv {
namespace {

constexpr int kW = 8;       // waves per workgroup = blocks per round
constexpr int kPMax = 16;   // probe channels supported

template <typename T, int D, int GR>
struct ArtSmem {
  using Gm = Geo<T, D>;
  static constexpr int GP = 4 * GR;
  static constexpr int PCH = (kPMax + Gm::E - 1) / Gm::E;  // chunks holding probe channels
  static constexpr int PW = PCH * Gm::E;
  // round buffers
  static constexpr int P_OFF = 0;                                   // [kW][64 * GP]
  static constexpr int PR_OFF = P_OFF + kW * 64 * GP;               // [kW][NPH][GP][PW]
  static constexpr int ROUND_END = PR_OFF + kW * Gm::NPH * GP * PW;
  // end-of-kernel reduction, overlaps the round buffers
  static constexpr int RED_END = kW * GP * D;
  static constexpr int FLOATS = ROUND_END > RED_END ? ROUND_END : RED_END;
};

template <typename T, int D, int GR>
__global__ __launch_bounds__(kW * 64) void art_kernel(ArtArgs p) {
  using Gm = Geo<T, D>;
  using SM = ArtSmem<T, D, GR>;
  constexpr int GP = SM::GP;
  constexpr int E = Gm::E, CPR = Gm::CPR, TPI = Gm::TPI, KA = Gm::KA, ROWB = Gm::ROWB, NPH = Gm::NPH;
  constexpr int PCH = SM::PCH, PW = SM::PW;
  constexpr bool BF = sizeof(T) == 2;

  __shared__ float smem[SM::FLOATS];
  __shared__ float blk_m[kW][GP], blk_l[kW][GP];
  __shared__ float red_m[kW][GP], red_l[kW][GP];
  __shared__ int stop_t[GP];
  __shared__ int s_done;

  const int unit = blockIdx.x;
  const int b = unit / p.Hkv, g = unit % p.Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int G = p.Hq / p.Hkv;
  const int NBmax = p.NBmax;
  const int L = clampi(p.seq_lens ? p.seq_lens[b] : NBmax * kBlock, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;
  const int P = p.probe_dim;

  const size_t slice = (size_t)NBmax * kBlock * ROWB;
  const auto krs = make_rsrc((const char*)p.k + unit * slice, (uint32_t)L * ROWB);
  const auto vrs = make_rsrc((const char*)p.v + unit * slice, (uint32_t)L * ROWB);

  const int arow = lane & 15, kg = lane >> 4;
  const int aq = 4 * (arow & 3) + (arow >> 2);
  const bool aq_ok = aq < G;
  const T* qrow = (const T*)p.q + ((size_t)b * p.Hq + (size_t)g * G + (aq_ok ? aq : 0)) * D;
  u32x4 qop[KA];
#pragma unroll
  for (int a = 0; a < KA; ++a) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    qop[a] = aq_ok ? *(const u32x4*)(qrow + (4 * a + kg) * E) : z;
  }
  const float scale2 = p.scale * kLog2e;
  const uint32_t kvo = (uint32_t)arow * ROWB + (uint32_t)kg * 16;
  const uint32_t vvo = (uint32_t)(lane / CPR) * ROWB + (uint32_t)(lane % CPR) * 16;
  const int chunk = lane % CPR, phase = lane / CPR;

  if (threadIdx.x < GP) stop_t[threadIdx.x] = INT_MAX;

  // private running state of this wave (uniform m, l per query slot)
  float wm[GP], wl[GP], acc[GP][E];
#pragma unroll
  for (int q = 0; q < GP; ++q) {
    wm[q] = -INFINITY;
    wl[q] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[q][e] = 0.f;
  }

  // wave 0: sequential fold of the probe channels, lane = 16 * (q % 4) + channel
  const int pk = lane & 15;
  float fM[GR], fL[GR], fA[GR], fx[GR], fn[GR];
  int fcnt[GR], fstop[GR];
#pragma unroll
  for (int r = 0; r < GR; ++r) {
    fM[r] = -INFINITY;
    fL[r] = 0.f;
    fA[r] = 0.f;
    fx[r] = 0.f;
    fn[r] = 0.f;
    fcnt[r] = 0;
    fstop[r] = -1;
  }

  float* pl = smem + SM::P_OFF + w * 64 * GP;
  float* prw = smem + SM::PR_OFF + w * NPH * GP * PW;
  int rounds = 0;
  __syncthreads();

  for (int base = 0; base < nb; base += kW) {
    ++rounds;
    const int t = base + w;
    const bool active = t < nb;
    float mb[GR], lb[GR];
    float ab[GP][E];
    if (active) {
      const int j = p.order ? clampi(p.order[(size_t)unit * NBmax + t], 0, nb - 1) : (t == 0 ? 0 : nb - t);
      const uint32_t soff = (uint32_t)j * kBlock * ROWB;
      u32x4 kr[4][KA];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int a = 0; a < KA; ++a) kr[t4][a] = load16(krs, soff + kvo + t4 * 16 * ROWB + a * 64, 0);
      u32x4 vr[CPR];
#pragma unroll
      for (int i = 0; i < CPR; ++i) vr[i] = load16(vrs, soff + vvo + i * TPI * ROWB, 0);

      f32x4 sc[4];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int a = 0; a < KA; ++a) {
          if constexpr (BF) {
            c = mfma_bf16(qop[a], kr[t4][a], c);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              c = mfma_f32(__uint_as_float(qop[a][e]), __uint_as_float(kr[t4][a][e]), c);
          }
        }
        sc[t4] = c;
      }
      const int nvalid = min(kBlock, L - j * kBlock);
#pragma unroll
      for (int r = 0; r < GR; ++r) {
        float s[4];
        float mx = -INFINITY;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          s[t4] = (16 * t4 + arow < nvalid) ? sc[t4][r] * scale2 : -INFINITY;
          mx = fmaxf(mx, s[t4]);
        }
        mx = row16_max(mx);
        float ps = 0.f;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          const float pv = fast_exp2(s[t4] - mx);
          ps += pv;
          pl[(16 * t4 + arow) * GP + 4 * r + kg] = pv;
        }
        mb[r] = mx;
        lb[r] = row16_sum(ps);
      }
#pragma unroll
      for (int q = 0; q < GP; ++q)
#pragma unroll
        for (int e = 0; e < E; ++e) ab[q][e] = 0.f;
#pragma unroll
      for (int i = 0; i < CPR; ++i) {
        const int tk = i * TPI + phase;
        float pq[GP];
#pragma unroll
        for (int r = 0; r < GR; ++r) {
          const f32x4 x = *(const f32x4*)(pl + tk * GP + 4 * r);
          pq[4 * r] = x[0];
          pq[4 * r + 1] = x[1];
          pq[4 * r + 2] = x[2];
          pq[4 * r + 3] = x[3];
        }
        float vf[E];
        if constexpr (BF) {
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            vf[2 * e2] = bf16_lo(vr[i][e2]);
            vf[2 * e2 + 1] = bf16_hi(vr[i][e2]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) vf[e] = __uint_as_float(vr[i][e]);
        }
#pragma unroll
        for (int q = 0; q < GP; ++q)
#pragma unroll
          for (int e = 0; e < E; ++e) ab[q][e] = fmaf(pq[q], vf[e], ab[q][e]);
      }
      // publish the block's (m, l) and the probe channels of its P.V
      if (arow == 0) {
#pragma unroll
        for (int r = 0; r < GR; ++r) {
          blk_m[w][4 * r + kg] = mb[r];
          blk_l[w][4 * r + kg] = lb[r];
        }
      }
      if (P > 0 && chunk < PCH) {
#pragma unroll
        for (int q = 0; q < GP; ++q)
#pragma unroll
          for (int e = 0; e < E; ++e) prw[(phase * GP + q) * PW + chunk * E + e] = ab[q][e];
      }
    }
    __syncthreads();

    if (w == 0) {
      const int t_end = min(base + kW, nb);
      if (P > 0) {
        for (int tt = base; tt < t_end; ++tt) {
          const int ww = tt - base;
          const float* prb = smem + SM::PR_OFF + ww * NPH * GP * PW;
#pragma unroll
          for (int r = 0; r < GR; ++r) {
            const int q = 4 * r + kg;
            if (q < G && fstop[r] < 0) {  // uniform over the 16-lane row
              const float mq = blk_m[ww][q], lq = blk_l[ww][q];
              float a = 0.f;
              if (pk < P) {
#pragma unroll
                for (int ph = 0; ph < NPH; ++ph) a += prb[(ph * GP + q) * PW + pk];
              }
              const float Mn = fmaxf(fM[r], mq);
              const float al = fast_exp2(fM[r] - Mn), be = fast_exp2(mq - Mn);
              fA[r] = al * fA[r] + be * a;
              fL[r] = al * fL[r] + be * lq;
              fM[r] = Mn;
              const float x = fA[r] / fL[r];
              const float n1 = sqrtf(row16_sum(x * x));
              if (tt >= 1) {
                const float n0 = fn[r];
                const float ds = fabsf(n1 - n0);
                float dd = INFINITY;
                if (n1 > 0.f && n0 > 0.f) {
                  // 1 - cos as half the squared distance of the unit vectors
                  const float u = x / n1 - fx[r] / n0;
                  dd = 0.5f * row16_sum(u * u);
                }
                const bool stable = ds < p.tau && dd < p.phi;
                fcnt[r] = stable ? fcnt[r] + 1 : 0;
                if (fcnt[r] >= p.patience) fstop[r] = tt;
              }
              fx[r] = x;
              fn[r] = n1;
            }
          }
        }
      }
      bool live = false;
#pragma unroll
      for (int r = 0; r < GR; ++r) {
        const int q = 4 * r + kg;
        if (q < G && fstop[r] < 0) live = true;
        if (pk == 0 && q < G && fstop[r] >= 0) stop_t[q] = fstop[r];
      }
      const bool any_live = __ballot(live) != 0;
      if (lane == 0) s_done = (!any_live || t_end >= nb) ? 1 : 0;
    }
    __syncthreads();

    if (active) {
#pragma unroll
      for (int q = 0; q < GP; ++q) {
        if (q < G && t <= stop_t[q]) {
          const float mq = readlane(mb[q >> 2], 16 * (q & 3));
          const float lq = readlane(lb[q >> 2], 16 * (q & 3));
          const float Mn = fmaxf(wm[q], mq);
          const float al = fast_exp2(wm[q] - Mn), be = fast_exp2(mq - Mn);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[q][e] = al * acc[q][e] + be * ab[q][e];
          wl[q] = al * wl[q] + be * lq;
          wm[q] = Mn;
        }
      }
    }
    if (s_done) break;
  }

  // merge the 8 private states
#pragma unroll
  for (int q = 0; q < GP; ++q)
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int off = CPR; off < 64; off <<= 1) acc[q][e] += __shfl_xor(acc[q][e], off);
  __syncthreads();
  float* red = smem;  // [kW][GP][D]
  if (lane < CPR) {
#pragma unroll
    for (int q = 0; q < GP; ++q)
#pragma unroll
      for (int e = 0; e < E; ++e) red[(w * GP + q) * D + lane * E + e] = acc[q][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < GP; ++q) {
      red_m[w][q] = wm[q];
      red_l[w][q] = wl[q];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kW * 64) {
    const int q = idx / D, dd = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) M = fmaxf(M, red_m[ww][q]);
    float ls = 0.f, os = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kW; ++ww) {
        const float f = fast_exp2(red_m[ww][q] - M);
        ls = fmaf(red_l[ww][q], f, ls);
        os = fmaf(red[(ww * GP + q) * D + dd], f, os);
      }
    }
    p.out[((size_t)b * p.Hq + (size_t)g * G + q) * D + dd] = ls > 0.f ? os / ls : 0.f;
  }
  if (threadIdx.x < G) {
    const int st = stop_t[threadIdx.x];
    p.stop_pos[(size_t)b * p.Hq + (size_t)g * G + threadIdx.x] = nb == 0 ? -1 : (st == INT_MAX ? nb - 1 : st);
  }
  if (threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[unit] = min(rounds * kW, nb);
}

template <typename T, int D>
hipError_t launch_art_t(const ArtArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const dim3 grid(a.B * a.Hkv);
  if (G <= 4)
    art_kernel<T, D, 1><<<grid, kW * 64, 0, st>>>(a);
  else
    art_kernel<T, D, 2><<<grid, kW * 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_art(const ArtArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (a.dtype == 1) return a.d == 128 ? launch_art_t<__bf16, 128>(a, st) : launch_art_t<__bf16, 64>(a, st);
  return a.d == 128 ? launch_art_t<float, 128>(a, st) : launch_art_t<float, 64>(a, st);
}

}  // namespace skv
