// Decode attention with ART run-time termination, for gfx950.
//
// Method ("ART (Attention Run-time Termination)" summary): KV blocks are
// folded into the streaming attention state in a visit order (§2.1, §2.4,
// block 0 first); after each fold a small probe of the partial output is
// compared with the previous one -- magnitude change and direction change
// (§2.2) -- and attention stops once both stay below their thresholds for
// p consecutive blocks (§2.3).
//
// One workgroup = one (b, kv head), split by role:
//   * NP producer waves (7, or 15 when the grid has fewer units than CUs)
//     stream blocks: producer i takes visit positions i, i+NP, i+2NP, ...; for each it loads the block (16-byte buffer loads),
//     forms the G x 64 logits on MFMA, the block-local softmax, and P.V in
//     fp32, and publishes the block's state (m, l, unnormalised P.V of all
//     channels) into an R-slot ring in LDS (R = NP + 1).
//   * 1 folder wave folds the published states strictly in visit order into
//     the running state -- the exact sequence of a one-block-at-a-time
//     streaming kernel -- and after every fold evaluates the stop rule per
//     query head on the probe channels (one 16-lane row per head).  A head
//     that stops freezes its state; when every head of the group has
//     stopped (or the blocks run out) the folder writes the outputs.
// Ring protocol (acquire/release on LDS words): a producer may start
// position t only once position t-R has been folded, so read-ahead past the
// final stop is at most R blocks (counted in blocks_fetched); the folder
// waits for slot t%R to hold position t.  The folder is never blocked by a
// producer that is itself blocked: the owner of the next position to fold
// always has its slot free.  Producers leave when the folder signals done.
#include "device_common.hpp"
#include "kernels.hpp"

namespace skv {
namespace {


__device__ __forceinline__ int ld_acq(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void st_rel(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// NP producer waves, R ring slots (R also bounds the read-ahead).
template <typename T, int D, int GR, int NP, int R>
struct ArtShared {
  static constexpr int GP = 4 * GR;
  static constexpr int kNP = NP, kR = R;
  float p_lds[NP][64 * GP];
  float slot_acc[R][GP][D];
  float slot_m[R][GP];
  float slot_l[R][GP];
  int slot_pos[R];
  int folded;
  int done;
  int fetched;
};

template <typename T, int D, int GR, typename SH>
__device__ void art_producer(const ArtArgs& p, SH& sh, int pi, int unit, int b, int g, int G,
                             int L, int nb) {
  using Gm = Geo<T, D>;
  constexpr int GP = 4 * GR;
  constexpr int E = Gm::E, CPR = Gm::CPR, TPI = Gm::TPI, KA = Gm::KA, ROWB = Gm::ROWB;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int kNP = SH::kNP, kR = SH::kR;
  const int lane = threadIdx.x & 63;
  const int NBmax = p.NBmax;

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
  const int phase = lane / CPR;
  float* pl = sh.p_lds[pi];

  for (int t = pi; t < nb; t += kNP) {
    // bounded read-ahead: position t may start once t - kR has been folded
    bool go = false;
    while (true) {
      if (ld_acq(&sh.done)) break;
      if (ld_acq(&sh.folded) > t - kR) {
        go = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!go) return;
    if (lane == 0) atomicAdd(&sh.fetched, 1);
    const int j = p.order ? clampi(p.order[(size_t)unit * NBmax + t], 0, nb - 1) : (t == 0 ? 0 : nb - t);
    const uint32_t soff = (uint32_t)j * kBlock * ROWB;
    u32x4 kr[4][KA];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int a = 0; a < KA; ++a) kr[t4][a] = load16(krs, soff + kvo + t4 * 16 * ROWB + a * 64, 0);
    u32x4 vr[CPR];
#pragma unroll
    for (int i = 0; i < CPR; ++i) vr[i] = load16_nt(vrs, soff + vvo + i * TPI * ROWB, 0);

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
    float mb[GR], lb[GR];
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
    float ab[GP][E];
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
    // sum the token phases, publish the block state, then its position
#pragma unroll
    for (int q = 0; q < GP; ++q)
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int off = CPR; off < 64; off <<= 1) ab[q][e] += __shfl_xor(ab[q][e], off);
    const int s = t % kR;
    if (lane < CPR) {
#pragma unroll
      for (int q = 0; q < GP; ++q)
#pragma unroll
        for (int e = 0; e < E; ++e) sh.slot_acc[s][q][lane * E + e] = ab[q][e];
    }
    if (arow == 0) {
#pragma unroll
      for (int r = 0; r < GR; ++r) {
        sh.slot_m[s][4 * r + kg] = mb[r];
        sh.slot_l[s][4 * r + kg] = lb[r];
      }
    }
    if (lane == 0) st_rel(&sh.slot_pos[s], t);
  }
}

template <typename T, int D, int GR, typename SH>
__device__ void art_folder(const ArtArgs& p, SH& sh, int b, int g, int G, int nb) {
  constexpr int FE = D / 16;  // channels per folder lane: lane = 16 * (q % 4) + c
  constexpr int kR = SH::kR;
  const int lane = threadIdx.x & 63;
  const int q4 = lane >> 4, c = lane & 15;
  const int P = p.probe_dim;
  float M[GR], Ls[GR], A[GR][FE], xp[GR][FE], n0[GR];  // xp: previous unit probe
  int cnt[GR], stopT[GR];
#pragma unroll
  for (int r = 0; r < GR; ++r) {
    M[r] = -INFINITY;
    Ls[r] = 0.f;
    n0[r] = 0.f;
    cnt[r] = 0;
    stopT[r] = -1;
#pragma unroll
    for (int e = 0; e < FE; ++e) {
      A[r][e] = 0.f;
      xp[r][e] = 0.f;
    }
  }
  for (int t = 0; t < nb; ++t) {
    const int s = t % kR;
    while (ld_acq(&sh.slot_pos[s]) != t) __builtin_amdgcn_s_sleep(1);
    bool live = false;
#pragma unroll
    for (int r = 0; r < GR; ++r) {
      const int q = 4 * r + q4;
      if (q < G && stopT[r] < 0) {  // uniform over the 16-lane row
        const float mq = sh.slot_m[s][q], lq = sh.slot_l[s][q];
        const float Mn = fmaxf(M[r], mq);
        const float al = fast_exp2(M[r] - Mn), be = fast_exp2(mq - Mn);
#pragma unroll
        for (int e = 0; e < FE; ++e) A[r][e] = al * A[r][e] + be * sh.slot_acc[s][q][c * FE + e];
        Ls[r] = al * Ls[r] + be * lq;
        M[r] = Mn;
        if (P > 0) {
          // probe x = A / L on the first P channels; unit vector u = x / |x|
          const float rl = fast_rcp(Ls[r]);
          float x[FE];
          float n2 = 0.f;
#pragma unroll
          for (int e = 0; e < FE; ++e) {
            x[e] = (c * FE + e < P) ? A[r][e] * rl : 0.f;
            n2 = fmaf(x[e], x[e], n2);
          }
          n2 = row16_sum(n2);
          const float i1 = n2 > 0.f ? fast_rsq(n2) : 0.f;
          const float n1 = n2 * i1;
          float u[FE];
#pragma unroll
          for (int e = 0; e < FE; ++e) u[e] = x[e] * i1;
          if (t >= 1) {
            const float ds = fabsf(n1 - n0[r]);
            float dd = INFINITY;
            if (n1 > 0.f && n0[r] > 0.f) {
              // 1 - cos as half the squared distance of the unit vectors
              float u2 = 0.f;
#pragma unroll
              for (int e = 0; e < FE; ++e) {
                const float du = u[e] - xp[r][e];
                u2 = fmaf(du, du, u2);
              }
              dd = 0.5f * row16_sum(u2);
            }
            const bool stable = ds < p.tau && dd < p.phi;
            cnt[r] = stable ? cnt[r] + 1 : 0;
            if (cnt[r] >= p.patience) stopT[r] = t;
          }
#pragma unroll
          for (int e = 0; e < FE; ++e) xp[r][e] = u[e];
          n0[r] = n1;
        }
        if (stopT[r] < 0) live = true;
      }
    }
    if (lane == 0) st_rel(&sh.folded, t + 1);
    if (__ballot(live) == 0) break;
  }
  if (lane == 0) st_rel(&sh.done, 1);
  // outputs: the frozen (or final) state of every head
#pragma unroll
  for (int r = 0; r < GR; ++r) {
    const int q = 4 * r + q4;
    if (q < G) {
      float* dst = p.out + ((size_t)b * p.Hq + (size_t)g * G + q) * D + c * FE;
#pragma unroll
      for (int e = 0; e < FE; ++e) dst[e] = Ls[r] > 0.f ? A[r][e] / Ls[r] : 0.f;
      if (c == 0)
        p.stop_pos[(size_t)b * p.Hq + (size_t)g * G + q] = nb == 0 ? -1 : (stopT[r] >= 0 ? stopT[r] : nb - 1);
    }
  }
}

template <typename T, int D, int GR, int NP, int R>
__global__ __launch_bounds__((NP + 1) * 64) void art_kernel(ArtArgs p) {
  using SH = ArtShared<T, D, GR, NP, R>;
  __shared__ SH sh;
  const int unit = blockIdx.x;
  const int b = unit / p.Hkv, g = unit % p.Hkv;
  const int w = threadIdx.x >> 6;
  const int G = p.Hq / p.Hkv;
  const int NBmax = p.NBmax;
  const int L = clampi(p.seq_lens ? p.seq_lens[b] : NBmax * kBlock, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;
  if (threadIdx.x < R) sh.slot_pos[threadIdx.x] = -1;
  if (threadIdx.x == 0) {
    sh.folded = 0;
    sh.done = 0;
    sh.fetched = 0;
  }
  __syncthreads();
  if (w == 0) {
    // the folder is the serial chain of the kernel: let the SIMD arbiter
    // prefer it over the producer waves that share its SIMD
    __builtin_amdgcn_s_setprio(3);
    art_folder<T, D, GR, SH>(p, sh, b, g, G, nb);
  }
  else
    art_producer<T, D, GR, SH>(p, sh, w - 1, unit, b, g, G, L, nb);
  __syncthreads();
  if (threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[unit] = sh.fetched;
}

// With at least one (b, kv head) unit per CU the chip is bandwidth-bound and
// the 8-block read-ahead keeps over-fetch small; with fewer units each
// workgroup must pull more bandwidth by itself, so it gets 15 producers and a
// 16-block window.
template <typename T, int D>
hipError_t launch_art_t(const ArtArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int units = a.B * a.Hkv;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  const dim3 grid(units);
  if (G > 4)
    art_kernel<T, D, 2, 7, 8><<<grid, 8 * 64, 0, st>>>(a);
  else if (units >= cus)
    art_kernel<T, D, 1, 7, 8><<<grid, 8 * 64, 0, st>>>(a);
  else
    art_kernel<T, D, 1, 15, 16><<<grid, 16 * 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_art(const ArtArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (a.dtype == 1) return a.d == 128 ? launch_art_t<__bf16, 128>(a, st) : launch_art_t<__bf16, 64>(a, st);
  return a.d == 128 ? launch_art_t<float, 128>(a, st) : launch_art_t<float, 64>(a, st);
}

}  // namespace skv
