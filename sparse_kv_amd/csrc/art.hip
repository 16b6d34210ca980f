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
//   * 7 producer waves stream blocks: producer i takes visit positions
//     i, i+7, i+14, ... (loads software-pipelined across positions when the
//     grid has fewer units than CUs); for each it loads the block (16-byte buffer loads),
//     forms the G x 64 logits on MFMA, the block-local softmax, and P.V in
//     fp32, and publishes the block's state (m, l, unnormalised P.V of all
//     channels) into an R-slot ring in LDS (R = 8, or 16 when pipelined).
//   * 1 folder wave folds the published states strictly in visit order into
//     the running state -- the exact sequence of a one-block-at-a-time
//     streaming kernel -- and after every fold evaluates the stop rule per
//     query head on the probe channels (one decision lane per head, so the
//     serial chain has no cross-lane reductions).  A head
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

// NP producer waves, R ring slots (R also bounds the read-ahead), PF: producers
// software-pipeline their loads across positions.
template <typename T, int D, int GR, int NP, int R, bool PF>
struct ArtShared {
  static constexpr int GP = 4 * GR;
  static constexpr int kNP = NP, kR = R;
  static constexpr bool kPF = PF;
  float p_lds[NP][64 * GP];
  float slot_acc[R][GP][D];
  float slot_m[R][GP];
  float slot_l[R][GP];
  int slot_pos[R];
  int folded;
  int done;
  int fetched;
};

// Producer wave pi: visit positions pi, pi + NP, ...  With SH::kPF the loads
// are software-pipelined as in the split-KV kernel: the next position's K is
// requested right after this block's logits and its V right after this
// block's P.V (when the read-ahead window already allows it), so HBM latency
// hides behind this block's arithmetic with no extra registers.
template <typename T, int D, int GR, typename SH>
__device__ void art_producer(const ArtArgs& p, SH& sh, int pi, int unit, int b, int g, int G, int L, int nb) {
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

  auto block_of = [&](int t) {
    return p.order ? clampi(p.order[(size_t)unit * NBmax + t], 0, nb - 1) : (t == 0 ? 0 : nb - t);
  };
  // read-ahead window: position t may start once t - kR has been folded
  auto window_open = [&](int t) { return ld_acq(&sh.folded) > t - kR; };
  auto window_wait = [&](int t) {
    while (true) {
      if (ld_acq(&sh.done)) return false;
      if (window_open(t)) return true;
      __builtin_amdgcn_s_sleep(1);
    }
  };
  u32x4 kr[4][KA], vr[CPR];
  // soff = byte offset of a block, or kNoBlock: past the buffers' range limit
  // (slices are at most 2 GiB), so the loads return zeros and touch no memory
  constexpr uint32_t kNoBlock = 0x80000000u;
  auto load_k = [&](uint32_t soff) {
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int a = 0; a < KA; ++a) kr[t4][a] = load16(krs, soff + kvo + t4 * 16 * ROWB + a * 64, 0);
  };
  auto load_v = [&](uint32_t soff) {
#pragma unroll
    for (int i = 0; i < CPR; ++i) vr[i] = load16_nt(vrs, soff + vvo + i * TPI * ROWB, 0);
  };
  auto block_off = [&](int j) {
    if (lane == 0) atomicAdd(&sh.fetched, 1);
    return (uint32_t)j * kBlock * ROWB;
  };

  int t = pi;
  if (t >= nb || !window_wait(t)) return;
  int j = block_of(t);
  {
    const uint32_t so = block_off(j);
    load_k(so);
    load_v(so);
  }
  while (true) {
    const int tn = t + kNP;
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
    bool pf = false;
    int jn = 0;
    uint32_t son = kNoBlock;
    if constexpr (SH::kPF) {
      // unconditional loads keep one register lifetime; a closed window
      // aims them past the range limit
      pf = tn < nb && !ld_acq(&sh.done) && window_open(tn);
      if (pf) {
        jn = block_of(tn);
        son = block_off(jn);
      }
      load_k(son);
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
    if constexpr (SH::kPF) load_v(son);
    // sum the token phases, publish the block state, then its position
#pragma unroll
    for (int q = 0; q < GP; ++q)
#pragma unroll
      for (int e = 0; e < E; ++e) ab[q][e] = phase_sum<CPR>(ab[q][e]);
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

    if (tn >= nb) return;
    if (!pf) {
      if (!window_wait(tn)) return;
      jn = block_of(tn);
      const uint32_t so = block_off(jn);
      load_k(so);
      load_v(so);
    }
    t = tn;
    j = jn;
  }
}

// The folder wave.  Lane q < G is the decision lane of query head q: it keeps
// that head's running max and denominator and the probe channels of its
// running output, and evaluates the stop rule with no cross-lane traffic.
// Every lane (row q % 4, channels c * FE ..) also folds its slice of the full
// running output with the decision lanes' rescale factors, read back with
// readlane; a head stops contributing after its stop position.
template <typename T, int D, int GR, typename SH>
__device__ void art_folder(const ArtArgs& p, SH& sh, int b, int g, int G, int nb) {
  constexpr int FE = D / 16;  // output channels per lane
  constexpr int PW = 16;      // probe channels a decision lane can hold (probe_dim <= 16)
  constexpr int kR = SH::kR;
  const int lane = threadIdx.x & 63;
  const int q4 = lane >> 4, c = lane & 15;
  const int P = p.probe_dim;
  const bool dec = lane < G;
  const int dq = dec ? lane : 0;

  float dM = -INFINITY, dL = 0.f, dn0 = 0.f;
  float dA[PW], du[PW];
#pragma unroll
  for (int k = 0; k < PW; ++k) {
    dA[k] = 0.f;
    du[k] = 0.f;
  }
  int dcnt = 0, dstop = -1;
  float A[GR][FE];
#pragma unroll
  for (int r = 0; r < GR; ++r)
#pragma unroll
    for (int e = 0; e < FE; ++e) A[r][e] = 0.f;

  for (int t = 0; t < nb; ++t) {
    const int s = t % kR;
    while (ld_acq(&sh.slot_pos[s]) != t) __builtin_amdgcn_s_sleep(1);
    // the block's slice of the full output for this lane
    float a[GR][FE];
#pragma unroll
    for (int r = 0; r < GR; ++r)
#pragma unroll
      for (int e = 0; e < FE; ++e) a[r][e] = sh.slot_acc[s][4 * r + q4][c * FE + e];

    // decision lanes: fold m, l and the probe channels, then the stop rule
    float al = 1.f, be = 0.f;
    int inc = 0;
    if (dec && dstop < 0) {
      inc = 1;
      const float mb = sh.slot_m[s][dq], lb = sh.slot_l[s][dq];
      const float Mn = fmaxf(dM, mb);
      al = fast_exp2(dM - Mn);
      be = fast_exp2(mb - Mn);
      dL = al * dL + be * lb;
      dM = Mn;
      if (P > 0) {
        const float rl = fast_rcp(dL);
        float x[PW];
        float n2 = 0.f;
#pragma unroll
        for (int k = 0; k < PW; ++k) {
          const float ak = k < P ? sh.slot_acc[s][dq][k] : 0.f;
          dA[k] = al * dA[k] + be * ak;
          x[k] = dA[k] * rl;
          n2 = fmaf(x[k], x[k], n2);
        }
        const float i1 = n2 > 0.f ? fast_rsq(n2) : 0.f;
        const float n1 = n2 * i1;
        float u2 = 0.f;
#pragma unroll
        for (int k = 0; k < PW; ++k) {
          const float uk = x[k] * i1;
          const float d = uk - du[k];
          u2 = fmaf(d, d, u2);
          du[k] = uk;
        }
        if (t >= 1) {
          const float ds = fabsf(n1 - dn0);
          // 1 - cos as half the squared distance of the unit vectors
          const float dd = (n1 > 0.f && dn0 > 0.f) ? 0.5f * u2 : INFINITY;
          const bool stable = ds < p.tau && dd < p.phi;
          dcnt = stable ? dcnt + 1 : 0;
          if (dcnt >= p.patience) dstop = t;
        }
        dn0 = n1;
      }
    }
    // every lane folds its slice of the full output with its head's factors
#pragma unroll
    for (int r = 0; r < GR; ++r) {
      float alr = 1.f, ber = 0.f;
      int incr = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float aj = readlane(al, 4 * r + j), bj = readlane(be, 4 * r + j);
        const int ij = __builtin_amdgcn_readlane(inc, 4 * r + j);
        alr = q4 == j ? aj : alr;
        ber = q4 == j ? bj : ber;
        incr = q4 == j ? ij : incr;
      }
      if (incr) {
#pragma unroll
        for (int e = 0; e < FE; ++e) A[r][e] = alr * A[r][e] + ber * a[r][e];
      }
    }
    if (lane == 0) st_rel(&sh.folded, t + 1);
    if (__ballot(dec && dstop < 0) == 0) break;
  }
  if (lane == 0) st_rel(&sh.done, 1);
  // outputs: the frozen (or final) state of every head
#pragma unroll
  for (int r = 0; r < GR; ++r) {
    float Lr = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lj = readlane(dL, 4 * r + j);
      Lr = q4 == j ? lj : Lr;
    }
    const int q = 4 * r + q4;
    if (q < G) {
      float* dst = p.out + ((size_t)b * p.Hq + (size_t)g * G + q) * D + c * FE;
#pragma unroll
      for (int e = 0; e < FE; ++e) dst[e] = Lr > 0.f ? A[r][e] / Lr : 0.f;
    }
  }
  if (dec) p.stop_pos[(size_t)b * p.Hq + (size_t)g * G + lane] = nb == 0 ? -1 : (dstop >= 0 ? dstop : nb - 1);
}

template <typename T, int D, int GR, int NP, int R, bool PF>
__global__ __launch_bounds__((NP + 1) * 64) void art_kernel(ArtArgs p) {
  using SH = ArtShared<T, D, GR, NP, R, PF>;
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
// workgroup must pull more bandwidth by itself, so its producers pipeline
// their loads across positions within a 16-block window.
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
    art_kernel<T, D, 2, 7, 8, false><<<grid, 8 * 64, 0, st>>>(a);
  else if (units >= cus)
    art_kernel<T, D, 1, 7, 8, false><<<grid, 8 * 64, 0, st>>>(a);
  else
    art_kernel<T, D, 1, 7, 16, true><<<grid, 8 * 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_art(const ArtArgs& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (a.dtype == 1) return a.d == 128 ? launch_art_t<__bf16, 128>(a, st) : launch_art_t<__bf16, 64>(a, st);
  return a.d == 128 ? launch_art_t<float, 128>(a, st) : launch_art_t<float, 64>(a, st);
}

}  // namespace skv
