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
//     i, i+7, i+14, ...; for each it loads the block (16-byte buffer loads),
//     forms the G x 64 logits on MFMA, the block-local softmax, and P.V in
//     fp32, and publishes the block's state (m, l, unnormalised P.V of all
//     channels) into an R-slot ring in LDS (R = 8 when every CU has a unit,
//     else 16).
//   * 1 folder wave folds the published states strictly in visit order into
//     the running state -- the result of a one-block-at-a-time streaming
//     kernel -- a batch of whole groups of consecutive published positions at
//     a time, and evaluates the stop rule per query head at every position of
//     the batch.
//     A head that stops freezes its state; when every head of the group has
//     stopped (or the positions run out) the folder writes the outputs.
// Visit positions come from the default order, an explicit order, or a
// list of blocks (ART over a selection, §2.4), optionally cut to a count.
// Ring protocol (acquire/release on LDS words): a producer may start
// position t only once position t-R has been folded, so read-ahead past the
// final stop is at most R blocks (counted in blocks_fetched); the folder
// waits for slot t%R to hold position t.  The folder is never blocked by a
// producer that is itself blocked: the owner of the next position to fold
// always has its slot free.  Producers leave when the folder signals done.
//
// With fewer (b, kv head) units than half the CUs, a second form spreads each
// unit over up to 4 workgroups (art_mc_kernel below), with further
// workgroups joining the units still running as CUs free up: the ring moves
// to a caller-provided workspace in device memory (128 slots, device-scope
// accesses), producers claim visit positions from a per-unit counter, and
// four folder waves (one per query head, or per two heads when G > 4) fold
// batches of up to 64 (32) positions.  Folders take whole aligned groups of
// positions and carry the running state from group to group, so every
// result is bitwise reproducible whatever the timing of the producers.
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

// Per-wave LDS of a workgroup with NP producer waves: each producer's
// scratch holds its block's K rows (KROWS, padded by 16 bytes per row so the
// MFMA-layout reads are free of bank conflicts), then the block's softmax
// weights, which reuse the space once the logits are formed; the folders'
// output-fold weights.
constexpr int kMaxFolders = 8;
template <typename T, int D, int GR, int NP>
struct ArtWaves {
  static constexpr int GP = 4 * GR;
  static constexpr int kNP = NP;
  static constexpr int kRowB = D * (int)sizeof(T);
  static constexpr bool kKRows = GR == 1 && kRowB <= 256;
  static constexpr int kKStride = kRowB + 16;
  static constexpr int kScratch = kKRows ? 64 * kKStride : 64 * GP * 4;
  __attribute__((aligned(16))) char scratch[NP][kScratch];
  float fold_w[kMaxFolders][64];  // per folder: (head, batch position) output weights
  float fold_a[kMaxFolders][16];  // per folder: per (head, group) rescale of the running output
};

// The ring through which producers hand block states (m, l, unnormalised
// P.V of all channels, per query row) to the folders.  R slots: position t's
// state lives in slot t % R and is marked by writing t into pos[t % R].  One
// window word per folder: its count of folded positions, or kDoneMark once
// it has finished.  Producers go by the least of them and stop when every
// folder has finished.
constexpr int kDoneMark = 1 << 30;
// Read-ahead allowed once f positions are folded: the ring size, but no more
// than max(64, f), so a head that stops early wastes few blocks (a 32-block
// floor held the producers back while the first positions were folded).
template <int R>
__device__ __forceinline__ int window_span(int f) {
  return min(R, max(64, f));
}

// In LDS: one workgroup per (b, kv head).  Acquire/release on LDS words.
template <int GP, int D, int R>
struct LdsRing {
  static constexpr int kR = R;
  __attribute__((aligned(16))) float acc[R][GP][D];
  float m[R][GP];
  float l[R][GP];
  int pos[R];
  int folded, fetched;
  __device__ void init(int tid) {
    if (tid < R) pos[tid] = -1;
    if (tid == 0) {
      folded = 0;
      fetched = 0;
    }
  }
  template <int E>
  __device__ void put_acc(int s, int q, int col, const float (&v)[E]) {
#pragma unroll
    for (int e = 0; e < E; ++e) acc[s][q][col + e] = v[e];
  }
  __device__ void put_ml(int s, int q, float mv, float lv) {
    m[s][q] = mv;
    l[s][q] = lv;
  }
  __device__ f32x4 acc4(int s, int q, int col) { return *(const f32x4*)&acc[s][q][col]; }
  __device__ float m_at(int s, int q) { return m[s][q]; }
  __device__ float l_at(int s, int q) { return l[s][q]; }
  static constexpr int kMaxBatch = R;
  __device__ int window() { return ld_acq(&folded); }
  __device__ int window_load() { return ld_acq(&folded); }
  static __device__ int window_of(int v) { return v; }
  __device__ void set_folded(int, int v) { st_rel(&folded, v); }
  template <int FE>
  __device__ void acc_row(int s, int q, int col, float (&x)[FE]) {
#pragma unroll
    for (int e = 0; e < FE; ++e) x[e] = acc[s][q][col + e];
  }
  __device__ int poll(int s) { return ld_acq(&pos[s]); }
  __device__ void acquire() {}

  // one wave's LDS writes complete in order, so lane 0's release covers them
  __device__ void publish(int s, int t, int lane) {
    if (lane == 0) st_rel(&pos[s], t);
  }
  __device__ void count_fetch(int lane) {
    if (lane == 0) atomicAdd(&fetched, 1);
  }
};

// In global memory: the workgroups of one (b, kv head), on different CUs
// and, in general, different XCDs.  Every access to the ring is a
// device-scope one: stores write through to the device's coherence point
// and loads read from it, so no wave ever writes back or invalidates a whole
// L2 (with hundreds of producer waves doing so per block, that costs tens
// of microseconds a block).  Order comes from completion: a producer waits
// for its state stores to complete before it stores the position, the
// folder issues its state loads only after it has read the position, and it
// waits for them to complete before it advances the window.
template <int GP, int D, int R, int NF, int EP = 4>
struct GlobalRing {
  static constexpr int kR = R;
  static constexpr int kMaxBatch = R / 2;  // the producers work on the other half
  // control words, on separate 128-byte lines: the folders' counts of
  // folded positions (polled by every producer), the position claims, the
  // accounting words
  enum Ctrl { kFolded = 0, kNext = 32, kFetched = 64, kFolder, kNumCtrl = 96 };
  static_assert(NF <= 8 && R * 4 <= 512, "control and position areas");
  static constexpr uint32_t kPosOff = 0, kCtrlOff = 512;
  static constexpr uint32_t kMOff = kCtrlOff + 512;
  static_assert(kNumCtrl * 4 <= 512, "control area");
  static constexpr uint32_t kLOff = kMOff + ((uint32_t)R * GP * 4 + 255) / 256 * 256;
  static constexpr uint32_t kAccOff = kLOff + ((uint32_t)R * GP * 4 + 255) / 256 * 256;
  static constexpr uint32_t kBytes = kAccOff + ((uint32_t)R * GP * D * 4 + 255) / 256 * 256;
  static constexpr int kSc1 = 16;  // cache policy: device scope
  int* pos;
  int* ctrl;
  __amdgpu_buffer_rsrc_t rs;
  int* local_fetched = nullptr;  // this workgroup's fetch count (LDS)
  __device__ GlobalRing(char* ws, int unit) {
    char* u = ws + (size_t)unit * kBytes;
    pos = (int*)(u + kPosOff);
    ctrl = (int*)(u + kCtrlOff);
    rs = make_rsrc(u, kBytes);
  }
  // channel col of a row: producer lane l holds channels l EP .. l EP + EP - 1
  // and stores them as EP / 4 16-byte pieces; piece h of every lane is laid
  // out contiguously, so each store instruction covers whole 32-byte sectors
  static __device__ uint32_t acc_off(int s, int q, int col) {
    const uint32_t l = (uint32_t)col / EP, h = ((uint32_t)col % EP) / 4, w = (uint32_t)col % 4;
    return kAccOff + ((uint32_t)s * GP + q) * D * 4 + (h * (D / EP) + l) * 16 + w * 4;
  }
  template <int E>
  __device__ void put_acc(int s, int q, int col, const float (&v)[E]) {
    static_assert(E % 4 == 0, "16-byte stores");
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const u32x4 x = {__float_as_uint(v[e]), __float_as_uint(v[e + 1]), __float_as_uint(v[e + 2]),
                       __float_as_uint(v[e + 3])};
      __builtin_amdgcn_raw_buffer_store_b128(x, rs, (int)acc_off(s, q, col + e), 0, kSc1);
    }
  }
  __device__ void put_ml(int s, int q, float mv, float lv) {
    const int o = (s * GP + q) * 4;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mv), rs, (int)kMOff + o, 0, kSc1);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lv), rs, (int)kLOff + o, 0, kSc1);
  }
  __device__ f32x4 acc4(int s, int q, int col) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)acc_off(s, q, col), 0, kSc1);
    return f32x4{__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3])};
  }
  __device__ float m_at(int s, int q) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)kMOff + (s * GP + q) * 4, 0, kSc1));
  }
  __device__ float l_at(int s, int q) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)kLOff + (s * GP + q) * 4, 0, kSc1));
  }
  // vmcnt(0), with no memory access moved across it by the compiler
  static __device__ void wait_memory() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("" ::: "memory");
  }
  // the least count of folded positions over the folders (kDoneMark: all done)
  __device__ int window_load() {
    const int lane = threadIdx.x & 63;
    return lane < NF ? __hip_atomic_load(&ctrl[kFolded + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : kDoneMark;
  }
  __device__ int window() { return window_of(window_load()); }
  static __device__ int window_of(int v) {
    v = min(v, __shfl_xor(v, 1));
    v = min(v, __shfl_xor(v, 2));
    v = min(v, __shfl_xor(v, 4));
    return __builtin_amdgcn_readfirstlane(v);
  }
  __device__ void set_folded(int f, int v) {
    wait_memory();  // the batch's slot loads are complete before the slots are handed back
    __hip_atomic_store(&ctrl[kFolded + f], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  template <int FE>
  __device__ void acc_row(int s, int q, int col, float (&x)[FE]) {
    if constexpr (FE % 4 == 0) {
#pragma unroll
      for (int e = 0; e < FE; e += 4) {
        const f32x4 v = acc4(s, q, col + e);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[e + i] = v[i];
      }
    } else if constexpr (FE == 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)acc_off(s, q, col), 0, kSc1);
      x[0] = __uint_as_float(v[0]);
      x[1] = __uint_as_float(v[1]);
    } else {
      static_assert(FE == 1, "row slice of 1, 2 or 4k floats");
      x[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)acc_off(s, q, col), 0, kSc1));
    }
  }
  __device__ int poll(int s) { return __hip_atomic_load(&pos[s], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
  // state loads stay after the position loads that admitted them
  __device__ void acquire() { asm volatile("" ::: "memory"); }
  __device__ void publish(int s, int t, int lane) {
    wait_memory();  // this wave's state stores are complete
    if (lane == 0) __hip_atomic_store(&pos[s], t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ void count_fetch(int lane) {
    if (lane == 0) atomicAdd(local_fetched, 1);
  }
};

// Single-workgroup form: the per-wave LDS plus the ring in LDS.
template <typename T, int D, int GR, int NP, int R>
struct ArtShared : ArtWaves<T, D, GR, NP> {
  LdsRing<4 * GR, D, R> ring;
};

// Visit positions of one producer wave: a fixed stride (one workgroup per
// unit), or claimed from a per-unit counter (several workgroups per unit,
// whichever of them are resident).  Claims run one position ahead so their
// round trip overlaps a block's work; a wave's claims increase, so the
// smallest position not yet published always belongs to a wave that is at
// it and whose window admits it.
struct StridedPositions {
  int t0, stride;
  __device__ int first() { return t0; }
  __device__ int next(int t) { return t + stride; }
};
struct ClaimedPositions {
  int* counter;
  int pending = 0;
  __device__ void claim() {
    if ((threadIdx.x & 63) == 0) pending = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ int take() {
    const int t = __builtin_amdgcn_readfirstlane(pending);
    claim();
    return t;
  }
  __device__ int first() {
    claim();
    return take();
  }
  __device__ int next(int) { return take(); }
};

// Producer wave pi: visit positions from POS.  Each block is loaded
// whole before its logits, softmax and P.V; with NP producers per
// workgroup, NP blocks are in flight per CU.  V is read in the row layout
// (whole 128-byte lines per instruction, non-temporal).  K is read the same
// way when SH::kKRows and moved into the MFMA operand layout through LDS:
// the operand layout read straight from memory touches half of 16 lines
// per instruction, which a CU streams about 30% slower than whole lines --
// and with fewer units than CUs each unit runs at its CU's read limit.
template <typename T, int D, int GR, typename SH, typename RING, typename POS>
__device__ void art_producer(const ArtArgs& p, SH& sh, RING& ring, POS& pos, int pi, int unit, int b, int g, int G,
                             int L, int nb, int nv) {
  using Gm = Geo<T, D>;
  constexpr int GP = 4 * GR;
  constexpr int E = Gm::E, CPR = Gm::CPR, TPI = Gm::TPI, KA = Gm::KA, ROWB = Gm::ROWB;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int kR = RING::kR;
  const int lane = threadIdx.x & 63;
  const int NBmax = p.NBmax;

  const bool paged = p.table != nullptr;
  const size_t slice = paged ? 0 : (size_t)NBmax * kBlock * ROWB;
  auto krs = make_rsrc((const char*)p.k + unit * slice, (uint32_t)L * ROWB);
  auto vrs = make_rsrc((const char*)p.v + unit * slice, (uint32_t)L * ROWB);
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
  char* scr = sh.scratch[pi];
  float* pl = (float*)scr;
  constexpr bool KROWS = SH::kKRows;
  constexpr int KSTR = SH::kKStride;

  // visit position -> block; explicit order entries come through the scalar
  // cache, one block ahead
  auto order_at = [&](int t) {
    return (p.order && t < nv) ? uniform_load(p.order, (int64_t)unit * p.order_stride + t) : 0;
  };
  auto block_from = [&](int t, int o) { return p.order ? clampi(o, 0, nb - 1) : (t == 0 ? 0 : nb - t); };
  // read-ahead window: position t may start once the folders are within
  // window_span of it (f: a count of folded positions read earlier); false
  // once they have finished.  A fresh count is read for every block, while
  // that block's state stores complete: a look per block keeps read-ahead
  // (and over-fetch past the stop) in check and shows soon after that the
  // folders have finished.
  auto window_wait = [&](int t, int f) {
    while (true) {
      if (f >= kDoneMark) return false;
      if (f > t - window_span<kR>(f)) return true;
      __builtin_amdgcn_s_sleep(1);
      f = ring.window();
    }
  };
  u32x4 kr[4][KA], vr[CPR];
  u32x4 kraw[KROWS ? CPR : 1];
  auto load_k = [&](uint32_t soff) {
    if constexpr (KROWS) {
#pragma unroll
      for (int i = 0; i < CPR; ++i) kraw[i] = load16_nt(krs, soff + vvo + i * TPI * ROWB, 0);
    } else {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int a = 0; a < KA; ++a) kr[t4][a] = load16(krs, soff + kvo + t4 * 16 * ROWB + a * 64, 0);
    }
  };
  // K rows -> MFMA operand layout (row 16 t4 + arow, 16-byte chunk 4 a + kg)
  auto k_to_operands = [&]() {
    if constexpr (KROWS) {
#pragma unroll
      for (int i = 0; i < CPR; ++i)
        *(u32x4*)(scr + (i * TPI + phase) * KSTR + (lane % CPR) * 16) = kraw[i];
      wave_lds_exchange();
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int a = 0; a < KA; ++a) kr[t4][a] = *(const u32x4*)(scr + (16 * t4 + arow) * KSTR + (4 * a + kg) * 16);
      wave_lds_exchange();  // the weight table reuses the space
    }
  };
  auto load_v = [&](uint32_t soff) {
#pragma unroll
    for (int i = 0; i < CPR; ++i) vr[i] = load16_nt(vrs, soff + vvo + i * TPI * ROWB, 0);
  };
  // byte offset of block j in krs / vrs; a paged cache points them at the
  // block's own pool run (valid tokens only) and uses offset 0
  auto block_off = [&](int j) {
    ring.count_fetch(lane);
    if (paged) {
      const int ph = clampi(uniform_load(p.table, (int64_t)b * p.table_stride + j), 0, (int)(p.pool_blocks - 1));
      const size_t off = ((size_t)ph * p.Hkv + g) * (kBlock * ROWB);
      const uint32_t n = (uint32_t)min(kBlock, L - j * kBlock) * ROWB;
      krs = make_rsrc((const char*)p.k + off, n);
      vrs = make_rsrc((const char*)p.v + off, n);
      return 0u;
    }
    return (uint32_t)j * kBlock * ROWB;
  };

  int t = pos.first();
  if (t >= nv || !window_wait(t, ring.window())) return;
  int j = block_from(t, order_at(t));
  {
    const uint32_t so = block_off(j);
    load_k(so);
    load_v(so);
  }
  while (true) {
    const int tn = pos.next(t);
    const int onext = order_at(tn);
    k_to_operands();
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
    wave_lds_exchange();  // P rows written above are read across lanes below
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
    wave_lds_exchange();  // before the next block overwrites P
    // sum the token phases, publish the block state, then its position
#pragma unroll
    for (int q = 0; q < GP; ++q)
#pragma unroll
      for (int e = 0; e < E; ++e) ab[q][e] = phase_sum<CPR>(ab[q][e]);
    const int s = t % kR;
    if (lane < CPR) {
#pragma unroll
      for (int q = 0; q < GP; ++q) ring.put_acc(s, q, lane * E, ab[q]);
    }
    if (arow == 0) {
#pragma unroll
      for (int r = 0; r < GR; ++r) ring.put_ml(s, 4 * r + kg, mb[r], lb[r]);
    }
    const int wv = ring.window_load();  // read while the state stores complete
    ring.publish(s, t, lane);

    if (tn >= nv || !window_wait(tn, RING::window_of(wv))) return;
    j = block_from(tn, onext);
    const uint32_t so = block_off(j);
    load_k(so);
    load_v(so);
    t = tn;
  }
}

// Online-softmax merge of an earlier state (me, le, ae) into a later one
// (m, l, a), in the log2 domain; (-inf, 0, 0) is the identity.
template <int PW>
__device__ __forceinline__ void merge_into(float me, float le, const float (&ae)[PW], float& m, float& l,
                                           float (&a)[PW]) {
  const float M = fmaxf(me, m);
  const float Ms = M == -INFINITY ? 0.f : M;
  const float se = fast_exp2(me - Ms), sx = fast_exp2(m - Ms);
  l = se * le + sx * l;
#pragma unroll
  for (int k = 0; k < PW; ++k) a[k] = se * ae[k] + sx * a[k];
  m = M;
}

// The value of lane - K for groups of CH lanes (the caller discards lanes
// whose source lies outside their group): row_shr:K when groups stay within
// rows of 16 lanes, a lane permute when they span rows.
template <int K, int CH>
__device__ __forceinline__ float shr(float x) {
  if constexpr (CH <= 16)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + K, 0xF, 0xF, false));
  else if constexpr (CH == 64 && K == 1)  // wave_shr:1 (lane 0 gets 0)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x138, 0xF, 0xF, false));
  else
    return __shfl(x, ((int)threadIdx.x - K) & 63);
}

// One step of an inclusive online-softmax scan within aligned groups of GS
// lanes (GS <= 16, so a group never crosses a row of 16 lanes): the lane at
// group offset o >= K merges in the state of lane - K.
template <int K, int GS, int PW>
__device__ __forceinline__ void group_scan_step(int j, float& m, float& l, float (&a)[PW]) {
  if constexpr (K < GS) {
    const float me = shr<K, 16>(m), le = shr<K, 16>(l);
    float ae[PW];
#pragma unroll
    for (int k = 0; k < PW; ++k) ae[k] = shr<K, 16>(a[k]);
    if (j % GS >= K) merge_into<PW>(me, le, ae, m, l, a);
  }
}

// The value of lane src, for a src that is the same across each head's CH
// lanes (wave-uniform when one head fills the wave).
template <int CH>
__device__ __forceinline__ float from_lane(float x, int src) {
  if constexpr (CH == 64)
    return readlane(x, __builtin_amdgcn_readfirstlane(src));
  else
    return __shfl(x, src);
}

// Probe of a state: norm n and unit direction u of the first P channels of
// the normalised partial output (u = 0 when n = 0).
template <int PW>
__device__ __forceinline__ void probe_of(float L, const float (&A)[PW], float& n, float (&u)[PW]) {
  const float rl = L > 0.f ? fast_rcp(L) : 0.f;
  float n2 = 0.f;
#pragma unroll
  for (int k = 0; k < PW; ++k) {
    u[k] = A[k] * rl;
    n2 = fmaf(u[k], u[k], n2);
  }
  const float i1 = n2 > 0.f ? fast_rsq(n2) : 0.f;
  n = n2 * i1;
#pragma unroll
  for (int k = 0; k < PW; ++k) u[k] *= i1;
}

// A folder wave.  It folds published block states strictly in visit order,
// as a one-block-at-a-time streaming kernel would, but a batch at a time:
// every whole aligned group of GS consecutive positions already published
// (up to CH = 64 / HPW positions and the ring's batch cap; the sequence's
// last group may be short) is taken at once.  Folder f owns heads
// f * HPW .. f * HPW + HPW - 1; in the scan layout lane (h, j) = h * CH + j
// holds head h's state of the batch's block j.  Every running state is
// computed the same way whatever the batch boundaries, so results are
// bitwise reproducible however the producers' timing falls: an online-
// softmax scan within each group gives the group's prefix states, the state
// before each group follows from the one before the batch by merging in the
// groups' totals one group after another, and each position's running state
// is that carry merged with its prefix.  Each lane then evaluates the stop
// rule for its position; consecutive-stable runs come from the ballot of the
// per-position decisions.  A head that stops keeps its state at its stop
// position.  The full output (all d channels) is folded group by group: lane
// (h, j) holds channels j * D / CH .. of head h, rescales them to each
// group's closing max and adds the group's blocks with weights
// exp2(m_i - M), staged in LDS.  PW probe channels are carried
// (probe_dim <= PW).
template <typename T, int D, int HPW, int PW, typename SH, typename RING>
__device__ void art_folder(const ArtArgs& p, SH& sh, RING& ring, int f, int b, int g, int G, int nv) {
  constexpr int CH = 64 / HPW;  // batch positions per head; lanes per head
  // positions per group: few groups per batch keep the serial carry chain
  // short; small groups keep the folder from waiting on a straggling block
  constexpr int GS = CH >= 64 ? 16 : (CH >= 32 ? 8 : 4);
  constexpr int kR = RING::kR;
  constexpr int NBT = CH < RING::kMaxBatch ? CH : RING::kMaxBatch;  // largest batch
  constexpr int FE = D / CH;    // output channels per lane
  constexpr uint64_t RM = CH == 64 ? ~0ull : ((1ull << CH) - 1ull);
  static_assert(PW % 4 == 0 && PW <= 16 && FE >= 1, "layout");
  static_assert(NBT % GS == 0 && kR % GS == 0, "whole groups per batch and ring");
  const int lane = threadIdx.x & 63;
  const int hh = lane / CH, j = lane % CH;  // scan and output layout
  const int head = f * HPW + hh;            // head of the unit
  const int P = p.probe_dim;
  float* fold_w = sh.fold_w[f];
  float* fold_a = sh.fold_a[f];  // per (head, group): rescale of the output before the group

  // running state of head hh, identical in the CH lanes of its group
  float cM = -INFINITY, cL = 0.f, cA[PW];
#pragma unroll
  for (int k = 0; k < PW; ++k) cA[k] = 0.f;
  int ccnt = 0, dstop = -1;
  bool live = head < G;
  float A[FE];
#pragma unroll
  for (int e = 0; e < FE; ++e) A[e] = 0.f;

  int t0 = 0;
  // a folder with no real head (padded groups) takes no part
  while (__ballot(live) != 0 && t0 < nv) {
    // length of the published run of positions t0, t0 + 1, ..., cut to
    // whole groups short of the sequence's end
    const int tj = t0 + j;
    const bool pub = j < NBT && tj < nv && ring.poll(tj % kR) == tj;
    const uint64_t pm = (uint64_t)__ballot(pub) & RM;  // group 0 checks every position
    int n = ~pm == 0 ? 64 : __builtin_ctzll(~pm);
    if (t0 + n < nv) n -= n % GS;
    if (n == 0) {
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    ring.acquire();
    // the output rows of the batch's first chunk, in flight with its states
    // and through the scan; later chunks are read in the fold
    constexpr int CK0 = (64 / FE < 32 ? 64 / FE : 32) < NBT ? (64 / FE < 32 ? 64 / FE : 32) : NBT;
    constexpr int CK = CK0 < GS ? GS : CK0;
    static_assert(CK % GS == 0, "chunks of whole groups");
    float x0[CK][FE];
#pragma unroll
    for (int jj = 0; jj < CK; ++jj) ring.acc_row((t0 + min(jj, n - 1)) % kR, head, j * FE, x0[jj]);
    const bool in = live && j < n;
    const int s = tj % kR;
    float m = -INFINITY, l = 0.f, a[PW];
#pragma unroll
    for (int k = 0; k < PW; ++k) a[k] = 0.f;
    if (in) {
      m = ring.m_at(s, head);
      l = ring.l_at(s, head);
#pragma unroll
      for (int k4 = 0; k4 < PW / 4; ++k4) {
        const f32x4 x = ring.acc4(s, head, 4 * k4);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[4 * k4 + e] = 4 * k4 + e < P ? x[e] : 0.f;
      }
    }
    const float mb = m;
    // prefix states within each group
    group_scan_step<1, GS, PW>(j, m, l, a);
    group_scan_step<2, GS, PW>(j, m, l, a);
    group_scan_step<4, GS, PW>(j, m, l, a);
    group_scan_step<8, GS, PW>(j, m, l, a);
    // the state before each group, group after group from the state before
    // the batch, into (gM, gL, gA) of the lanes of that group
    float gM = cM, gL = cL, gA[PW];
#pragma unroll
    for (int k = 0; k < PW; ++k) gA[k] = cA[k];
    {
      float xM = cM, xL = cL, xA[PW];
#pragma unroll
      for (int k = 0; k < PW; ++k) xA[k] = cA[k];
      const int ng = (n + GS - 1) / GS;
      for (int q = 1; q < ng; ++q) {
        const int src = hh * CH + q * GS - 1;  // the previous group's last block (groups before the last are whole)
        float tM = from_lane<CH>(m, src), tL = from_lane<CH>(l, src);
        float tA[PW];
#pragma unroll
        for (int k = 0; k < PW; ++k) tA[k] = from_lane<CH>(a[k], src);
        merge_into<PW>(xM, xL, xA, tM, tL, tA);
        xM = tM;
        xL = tL;
#pragma unroll
        for (int k = 0; k < PW; ++k) xA[k] = tA[k];
        if (j / GS == q) {
          gM = xM;
          gL = xL;
#pragma unroll
          for (int k = 0; k < PW; ++k) gA[k] = xA[k];
        }
      }
    }
    // running state after block j = carry of its group (+) its group prefix
    merge_into<PW>(gM, gL, gA, m, l, a);
    float nrm, u[PW];
    probe_of<PW>(l, a, nrm, u);
    float cn, cu[PW];
    probe_of<PW>(cL, cA, cn, cu);
    float np = shr<1, CH>(nrm), up[PW];
#pragma unroll
    for (int k = 0; k < PW; ++k) up[k] = shr<1, CH>(u[k]);
    if (j == 0) {
      np = cn;
#pragma unroll
      for (int k = 0; k < PW; ++k) up[k] = cu[k];
    }
    float u2 = 0.f;
#pragma unroll
    for (int k = 0; k < PW; ++k) {
      const float dk = u[k] - up[k];
      u2 = fmaf(dk, dk, u2);
    }
    const float ds = fabsf(nrm - np);
    // 1 - cos as half the squared distance of the unit vectors
    const float dd = (nrm > 0.f && np > 0.f) ? 0.5f * u2 : INFINITY;
    const bool st = in && tj >= 1 && ds < p.tau && dd < p.phi;
    // consecutive stable steps ending at j (plus the run carried in)
    const uint64_t rowb = ((uint64_t)__ballot(st) >> (hh * CH)) & RM;
    const uint64_t z = ~rowb & ((2ull << j) - 1ull);
    const int run = z == 0 ? j + 1 + ccnt : j - (63 - __builtin_clzll(z));
    const bool hit = st && run >= p.patience;
    const uint64_t rowh = ((uint64_t)__ballot(hit) >> (hh * CH)) & RM;
    const int jend = rowh ? __builtin_ctzll(rowh) : n - 1;
    // the new running state: the state at jend
    const int src = hh * CH + jend;
    const float nM = from_lane<CH>(m, src), nL = from_lane<CH>(l, src);
    const int nrun = CH == 64 ? __builtin_amdgcn_readlane(run, __builtin_amdgcn_readfirstlane(src)) : __shfl(run, src);
    float nA[PW];
#pragma unroll
    for (int k = 0; k < PW; ++k) nA[k] = k < P ? from_lane<CH>(a[k], src) : 0.f;
    // output fold weights: each block of a group up to jend relative to the
    // running max where the group closes (its last block, or jend), and per
    // group the rescale of the output from the max before the group
    const int gq = j / GS;
    const int gend = min(gq * GS + GS - 1, jend);
    const float Me = __shfl(m, hh * CH + gend);  // per lane: its group's closing max
    const float Mes = Me == -INFINITY ? 0.f : Me;
    fold_w[lane] = (in && j <= jend) ? fast_exp2(mb - Mes) : 0.f;
    if (j % GS == 0 && j < NBT) fold_a[hh * (CH / GS) + gq] = (live && j <= jend) ? fast_exp2(gM - Mes) : 1.f;
    wave_lds_exchange();  // the weights are read by the other lanes
    {
      // chunks of positions whose rows are all loaded before any is used;
      // positions past the batch reread its last slot with weight 0
      for (int j0 = 0; j0 < n; j0 += CK) {
        float x[CK][FE];
#pragma unroll
        for (int jj = 0; jj < CK; ++jj) {
          if (j0 == 0) {
#pragma unroll
            for (int e = 0; e < FE; ++e) x[jj][e] = x0[jj][e];
          } else {
            ring.acc_row((t0 + min(j0 + jj, n - 1)) % kR, head, j * FE, x[jj]);
          }
        }
        // the chunk's weights and group rescales, read from LDS together
        // (16-byte loads) before any is used; positions past the batch
        // carry weight 0 and groups past it rescale by 1
        float wt[CK], ga[CK / GS];
#pragma unroll
        for (int jj = 0; jj < CK; jj += 4) {
          const f32x4 w4 = *(const f32x4*)&fold_w[hh * CH + j0 + jj];
#pragma unroll
          for (int e = 0; e < 4; ++e) wt[jj + e] = j0 + jj + e < n ? w4[e] : 0.f;
        }
#pragma unroll
        for (int gg = 0; gg < CK / GS; ++gg) ga[gg] = fold_a[hh * (CH / GS) + j0 / GS + gg];
#pragma unroll
        for (int jj = 0; jj < CK; ++jj) {
          if (jj % GS == 0 && j0 + jj < n) {
#pragma unroll
            for (int e = 0; e < FE; ++e) A[e] *= ga[jj / GS];
          }
#pragma unroll
          for (int e = 0; e < FE; ++e) A[e] = fmaf(wt[jj], x[jj][e], A[e]);
        }
      }
    }
    wave_lds_exchange();  // before the next batch overwrites the weights
    if (live) {
      cM = nM;
      cL = nL;
#pragma unroll
      for (int k = 0; k < PW; ++k) cA[k] = nA[k];
      if (rowh) {
        dstop = t0 + jend;
        live = false;
      } else {
        ccnt = nrun;
      }
    }
    t0 += n;
    // once every head has stopped, the window is not advanced past this
    // batch's start: read-ahead stays within the window of the stop
    if (__ballot(live) == 0) break;
    if (lane == 0) ring.set_folded(f, t0);
  }
  if (lane == 0) ring.set_folded(f, kDoneMark);
  // outputs: the frozen (or final) state of every head
  if (head < G) {
    float* dst = p.out + ((size_t)b * p.Hq + (size_t)g * G + head) * D + j * FE;
#pragma unroll
    for (int e = 0; e < FE; ++e) dst[e] = cL > 0.f ? A[e] / cL : 0.f;
    if (j == 0) p.stop_pos[(size_t)b * p.Hq + (size_t)g * G + head] = dstop >= 0 ? dstop : nv - 1;
  }
}

// probe_dim <= 8 carries half the probe channels through the scan
template <typename T, int D, int HPW, typename SH, typename RING>
__device__ void art_fold(const ArtArgs& p, SH& sh, RING& ring, int f, int b, int g, int G, int nv) {
  if (p.probe_dim <= 8)
    art_folder<T, D, HPW, 8>(p, sh, ring, f, b, g, G, nv);
  else
    art_folder<T, D, HPW, 16>(p, sh, ring, f, b, g, G, nv);
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
  // visit positions: the whole sequence, or the first n_visit entries of the order
  const int nv = p.n_visit ? clampi(p.n_visit[unit], 0, min(nb, p.order_stride)) : nb;
  sh.ring.init(threadIdx.x);
  __syncthreads();
  if (w == 0) {
    // the folder is the serial chain of the kernel: let the SIMD arbiter
    // prefer it over the producer waves that share its SIMD
    __builtin_amdgcn_s_setprio(3);
    art_fold<T, D, 4 * GR>(p, sh, sh.ring, 0, b, g, G, nv);
  }
  else
  {
    const int pi = __builtin_amdgcn_readfirstlane(w - 1);
    StridedPositions pos{pi, NP};
    art_producer<T, D, GR>(p, sh, sh.ring, pos, pi, unit, b, g, G, L, nb, nv);
  }
  __syncthreads();
  if (threadIdx.x == 0 && p.blocks_fetched) p.blocks_fetched[unit] = sh.ring.fetched;
}

// Several workgroups per (b, kv head) unit, for grids that would leave most
// CUs idle: one CU streams well under its share of HBM bandwidth, so a unit
// on one CU is bound by that CU.  The unit's workgroups share a ring in
// global memory; the first wave 0 to arrive folds, the other wave 0s leave,
// and every producer wave claims positions from the unit's counter, so
// progress never depends on which workgroups are resident.  The grid holds
// `groups` workgroups per unit, then late workgroups: each of those joins a
// unit whose folders are still at work when it starts (units stop at very
// different positions, and these add producers to the ones still running
// once the early finishers have freed their CUs), or leaves if none is.
// Every workgroup adds its fetch count to the unit's total on the way out
// and raises the reported count to the total it saw, so the report ends as
// the total whichever workgroup leaves last.
template <int GP, int D, int R>
__global__ __launch_bounds__(128) void art_ring_init(char* ws, int32_t* blocks_fetched) {
  using RING = GlobalRing<GP, D, R, 4>;
  RING ring(ws, blockIdx.x);
  if (threadIdx.x < R) ring.pos[threadIdx.x] = -1;
  if (threadIdx.x < RING::kNumCtrl) ring.ctrl[threadIdx.x] = 0;
  if (threadIdx.x == 0 && blocks_fetched) blocks_fetched[blockIdx.x] = 0;
}

template <typename T, int D, int GR, int NP>
struct ArtMcShared : ArtWaves<T, D, GR, NP> {
  int fetched;
  int role;  // 0: this workgroup's first waves fold
  int join;  // a late workgroup's unit (-1: every unit has finished)
};

template <typename T, int D, int GR, int NP, int R>
__global__ __launch_bounds__((NP + 1) * 64) void art_mc_kernel(ArtArgs p, char* ws, int groups) {
  using SH = ArtMcShared<T, D, GR, NP>;
  // folder waves: one per query head for G <= 4, one per two heads for G <= 8,
  // so the folding workgroup always keeps NP + 1 - NF producer waves of its
  // own (its unit progresses even if no other workgroup of it is resident)
  constexpr int NF = 4;
  static_assert(NF <= kMaxFolders && NF < NP, "folder waves and producers of the folding workgroup");
  using RING = GlobalRing<4 * GR, D, R, NF, Geo<T, D>::E>;
  __shared__ SH sh;
  const int units = p.B * p.Hkv;
  int unit = (int)blockIdx.x % units;
  if ((int)blockIdx.x >= units * groups) {
    // a late workgroup: the first unit, from its own on, whose folders have
    // not all finished (units <= 128: two looks per lane at most)
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      int pick = -1;
      for (int base = 0; base < units && pick < 0; base += 64) {
        const int u = (unit + base + lane) % units;
        bool active = false;
        if (base + lane < units) {
          RING r(ws, u);
          int done = 0;
#pragma unroll
          for (int f = 0; f < NF; ++f)
            done += __hip_atomic_load(&r.ctrl[RING::kFolded + f], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= kDoneMark;
          active = done < NF;
        }
        const uint64_t act = (uint64_t)__ballot(active);
        if (act) pick = (unit + base + (int)__builtin_ctzll(act)) % units;
      }
      if (lane == 0) sh.join = pick;
    }
    __syncthreads();
    if (sh.join < 0) return;  // the whole workgroup
    unit = sh.join;
  }
  const int b = unit / p.Hkv, g = unit % p.Hkv;
  const int w = threadIdx.x >> 6;
  const int G = p.Hq / p.Hkv;
  const int NBmax = p.NBmax;
  const int L = clampi(p.seq_lens ? p.seq_lens[b] : NBmax * kBlock, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;
  const int nv = p.n_visit ? clampi(p.n_visit[unit], 0, min(nb, p.order_stride)) : nb;
  RING ring(ws, unit);
  if (threadIdx.x == 0) {
    sh.fetched = 0;
    sh.role = __hip_atomic_fetch_add(&ring.ctrl[RING::kFolder], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  ring.local_fetched = &sh.fetched;
  const bool folds = sh.role == 0;
  if (folds && w < NF) {
    __builtin_amdgcn_s_setprio(3);
    art_fold<T, D, GR>(p, sh, ring, __builtin_amdgcn_readfirstlane(w), b, g, G, nv);
  } else if (w > 0) {
    ClaimedPositions pos{&ring.ctrl[RING::kNext]};
    art_producer<T, D, GR>(p, sh, ring, pos, __builtin_amdgcn_readfirstlane(w - 1), unit, b, g, G, L, nb, nv);
  }
  __syncthreads();
  // the unit's running total including this workgroup's fetches; the report
  // is raised to it (the caller's counts were zeroed by the ring reset)
  if (threadIdx.x == 0) {
    const int total = sh.fetched + __hip_atomic_fetch_add(&ring.ctrl[RING::kFetched], sh.fetched, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
    if (p.blocks_fetched) atomicMax(&p.blocks_fetched[unit], total);
  }
}

template <int D>
constexpr size_t art_ring_bytes(int G) {
  return G > 4 ? GlobalRing<8, D, kArtRingSlots, 4>::kBytes : GlobalRing<4, D, kArtRingSlots, 4>::kBytes;
}

template <typename T, int D, int GR>
hipError_t launch_art_mc(const ArtArgs& a, char* ws, int groups, int late, hipStream_t st) {
  const int units = a.B * a.Hkv;
  art_ring_init<4 * GR, D, kArtRingSlots><<<units, 128, 0, st>>>(ws, a.blocks_fetched);
  art_mc_kernel<T, D, GR, 7, kArtRingSlots><<<units * groups + late, 8 * 64, 0, st>>>(a, ws, groups);
  return hipGetLastError();
}

// With at least one (b, kv head) unit per CU the chip is bandwidth-bound and
// an 8-block read-ahead keeps over-fetch past the stop small.  With fewer
// units each workgroup streams at its CU's own limit and the folder, not
// bandwidth, decides how far producers may run ahead: a 16-block window
// lets them work on while it folds.
template <typename T, int D>
hipError_t launch_art_t(const ArtArgs& a, void* ws, size_t ws_bytes, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int units = a.B * a.Hkv;
  // the form depends on the CU count of the device the work is queued on
  int dev = 0, cus = 0;
  const hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  if (ws && units <= kArtMcMaxUnits && 2 * units <= cus && ws_bytes >= (size_t)units * art_ring_bytes<D>(G)) {
    // one workgroup per CU at the start, then as many again that join the
    // units still running as CUs free up
    const int groups = min(kArtMcMaxGroups, cus / units);
    const int late = units * groups;
    return G > 4 ? launch_art_mc<T, D, 2>(a, (char*)ws, groups, late, st)
                 : launch_art_mc<T, D, 1>(a, (char*)ws, groups, late, st);
  }
  const dim3 grid(units);
  const bool wide = units >= cus;
  if (G > 4) {
    if (wide)
      art_kernel<T, D, 2, 7, 8><<<grid, 8 * 64, 0, st>>>(a);
    else
      art_kernel<T, D, 2, 7, 16><<<grid, 8 * 64, 0, st>>>(a);
  } else {
    if (wide)
      art_kernel<T, D, 1, 7, 8><<<grid, 8 * 64, 0, st>>>(a);
    else
      art_kernel<T, D, 1, 7, 16><<<grid, 8 * 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_art(const ArtArgs& a, hipStream_t st, void* ws, size_t ws_bytes) {
  if (a.B == 0) return hipSuccess;
  if (a.dtype == 1)
    return a.d == 128 ? launch_art_t<__bf16, 128>(a, ws, ws_bytes, st) : launch_art_t<__bf16, 64>(a, ws, ws_bytes, st);
  return a.d == 128 ? launch_art_t<float, 128>(a, ws, ws_bytes, st) : launch_art_t<float, 64>(a, ws, ws_bytes, st);
}

size_t art_workspace_bytes(int32_t units, int32_t G, int32_t d) {
  if (units < 1 || units > kArtMcMaxUnits) return 0;
  return (size_t)units * (d == 128 ? art_ring_bytes<128>(G) : art_ring_bytes<64>(G));
}

}  // namespace skv
