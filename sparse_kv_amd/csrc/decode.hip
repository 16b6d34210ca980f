// Split-KV streaming decode attention over a block-organised KV cache
// (dense block ranges and listed blocks), for gfx950.
//
// Method: FlashAttention-style tile-wise accumulation with a running
// (max, denominator, output) state per split ("ART (Attention Run-time
// Termination)" summary, §2.1); the per-split states are merged exactly by
// online softmax afterwards ("Pulsar Attention" summary, Phase 2).  The
// listed-block form is attention over the selected keys only ("Squeezed
// Attention" blog, Q2 step 3).
//
// One workgroup = one (split, kv head, batch row); 4 wave64s take the
// split's blocks round-robin, one 64-token block per wave at a time:
//   * K of the block is read with 16-byte buffer loads straight into the
//     B-operand layout of a 16x16 MFMA (lane%16 = token, lane/16 = 16-byte
//     slice of the row) and multiplied with the group's G queries, which sit
//     in rows 4*(q%4) + q/4 of the A operand so that the logits of query q
//     land in register q/4 of lane group q%4 -- every lane then owns one
//     (query, token) logit per 16-token group and the softmax needs no
//     duplicated work.
//   * The exponentiated weights go through a 64 x G float table in LDS and
//     are re-read in the row layout used for V (lane%CPR = 16-byte chunk,
//     lane/CPR = token phase; one wave-wide load covers whole rows), where
//     P.V is accumulated in fp32 with VALU FMAs: P is never rounded to bf16.
//   * V is read with streaming (non-temporal) loads, whole rows per
//     instruction.  K is read the same way when a padded 64-row tile per
//     wave fits in LDS (G <= 4 and rows of at most 256 bytes) and moved into
//     the MFMA operand layout there; otherwise it is read straight into that
//     layout, half a 128-byte line per instruction, through L2 so that the
//     second half is an L2 hit.
//   * Reads past the sequence end hit the buffer range limit and return
//     zeros (the whole byte offset goes in the VGPR offset, which is what the
//     range check covers); their logits are masked to -inf.
//   * A paged cache (PAGED) keeps every (block, kv head) run contiguous in a
//     pool; each block then gets a buffer resource of its own, over its valid
//     tokens, from the block table entry read through the scalar cache.
// At the end the 4 waves' states are merged through LDS and the split's
// (m, l, o) is written, o normalised, m in natural-log units.
// Measured on MI355X at 128K context, batch 8: 6.99 TB/s (87% of the 8 TB/s
// datasheet peak, 99% of a non-temporal streaming-read probe) with 4 splits
// per (b, kv head), i.e. one workgroup per CU for the whole stream.  The
// software-pipelined loop (one workgroup per CU by register use) beat a plain
// loop at 2-3 workgroups per CU, 6.93 against 6.86 TB/s, and whole-line K
// through LDS beat the operand-layout reads by another ~1%.
#include "device_common.hpp"
#include "kernels.hpp"

namespace skv {
namespace {

constexpr int kWaves = 4;

template <typename T, int D, int GR, bool SPARSE, bool PAGED>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs p) {
  using Gm = Geo<T, D>;
  constexpr int GP = 4 * GR;  // query slots: G <= GP
  constexpr int E = Gm::E, CPR = Gm::CPR, TPI = Gm::TPI, KA = Gm::KA, ROWB = Gm::ROWB;
  constexpr bool BF = sizeof(T) == 2;

  // per-wave scratch: the block's K rows (KROWS; 16 bytes of padding per row
  // keep the operand-layout reads free of bank conflicts), then its softmax
  // weights, which reuse the space once the logits are formed
  constexpr bool KROWS = GR == 1 && ROWB <= 256;
  constexpr int KSTR = ROWB + 16;
  constexpr int SCR = KROWS ? 64 * KSTR : 64 * GP * 4;
  __shared__ __attribute__((aligned(16))) char scratch[kWaves][SCR];
  __shared__ float red_acc[kWaves][GP][D];
  __shared__ float red_m[kWaves][GP];
  __shared__ float red_l[kWaves][GP];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = p.Hq / p.Hkv;
  const int NBmax = p.NBmax;
  const int L = clampi(p.seq_lens ? p.seq_lens[b] : NBmax * kBlock, 0, NBmax * kBlock);
  const int nb = (L + kBlock - 1) / kBlock;
  const size_t unit = (size_t)b * p.Hkv + g;

  int lo, hi;
  if constexpr (SPARSE) {
    const int n = nb > 0 ? clampi(p.n_sel[unit], 0, p.max_sel) : 0;
    lo = (int)((int64_t)split * n / p.S);
    hi = (int)((int64_t)(split + 1) * n / p.S);
  } else {
    const int e = p.block_end < 0 ? nb : min(p.block_end, nb);
    const int bb = min(p.block_begin, e);
    const int n = e - bb;
    lo = bb + (int)((int64_t)split * n / p.S);
    hi = bb + (int)((int64_t)(split + 1) * n / p.S);
  }

  const size_t slice = PAGED ? 0 : (size_t)NBmax * kBlock * ROWB;
  const auto krs = make_rsrc((const char*)p.k + unit * slice, (uint32_t)L * ROWB);
  const auto vrs = make_rsrc((const char*)p.v + unit * slice, (uint32_t)L * ROWB);
  // paged: the pool run of logical block j, and its valid bytes
  auto pool_off = [&](int j) {
    const int ph = clampi(uniform_load(p.table, (int64_t)b * p.table_stride + j), 0, (int)(p.pool_blocks - 1));
    return ((size_t)ph * p.Hkv + g) * (kBlock * ROWB);
  };
  auto valid_bytes = [&](int j) { return (uint32_t)min(kBlock, L - j * kBlock) * ROWB; };

  // A operand: row i of the 16-row tile holds query 4*(i%4) + i/4.
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

  float m_run[GR], l_run[GR];
  float acc[GP][E];
#pragma unroll
  for (int r = 0; r < GR; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
#pragma unroll
  for (int q = 0; q < GP; ++q)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[q][e] = 0.f;

  char* scr = scratch[w];
  float* pl = (float*)scr;
  const int32_t* list = SPARSE ? p.block_idx + unit * (size_t)p.max_sel : nullptr;

  // Software pipeline: the next block's K is requested as soon as this
  // block's logits are formed, its V as soon as this block's P.V is done, so
  // every wave keeps a block's worth of loads in flight while it computes.
  u32x4 kr[4][KA];
  u32x4 vr[CPR];
  u32x4 kraw[KROWS ? CPR : 1];
  auto block_at = [&](int pos) { return SPARSE ? clampi(uniform_load(list, pos), 0, nb - 1) : pos; };
  auto load_k = [&](int j) {
    auto rs = krs;
    uint32_t soff = (uint32_t)j * kBlock * ROWB;
    if constexpr (PAGED) {
      rs = make_rsrc((const char*)p.k + pool_off(j), valid_bytes(j));
      soff = 0;
    }
    if constexpr (KROWS) {
#pragma unroll
      for (int i = 0; i < CPR; ++i) kraw[i] = load16_nt(rs, soff + vvo + i * TPI * ROWB, 0);
    } else {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int a = 0; a < KA; ++a) kr[t4][a] = load16(rs, soff + kvo + t4 * 16 * ROWB + a * 64, 0);
    }
  };
  // K rows -> MFMA operand layout (row 16 t4 + arow, 16-byte chunk 4 a + kg)
  auto k_to_operands = [&]() {
    if constexpr (KROWS) {
#pragma unroll
      for (int i = 0; i < CPR; ++i)
        *(u32x4*)(scr + (i * TPI + lane / CPR) * KSTR + (lane % CPR) * 16) = kraw[i];
      wave_lds_exchange();
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int a = 0; a < KA; ++a) kr[t4][a] = *(const u32x4*)(scr + (16 * t4 + arow) * KSTR + (4 * a + kg) * 16);
      wave_lds_exchange();  // the weight table reuses the space
    }
  };
  auto load_v = [&](int j) {
    auto rs = vrs;
    uint32_t soff = (uint32_t)j * kBlock * ROWB;
    if constexpr (PAGED) {
      rs = make_rsrc((const char*)p.v + pool_off(j), valid_bytes(j));
      soff = 0;
    }
#pragma unroll
    for (int i = 0; i < CPR; ++i) vr[i] = load16_nt(rs, soff + vvo + i * TPI * ROWB, 0);
  };
  int jn = 0;
  if (lo + w < hi) {
    jn = block_at(lo + w);
    load_k(jn);
    load_v(jn);
  }

  for (int pos = lo + w; pos < hi; pos += kWaves) {
    const int j = jn;
    const bool more = pos + kWaves < hi;
    k_to_operands();

    // logits: sc[t4][r] = <q_{4r + kg}, k_{16 t4 + arow}>
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
    if (more) {
      jn = block_at(pos + kWaves);
      load_k(jn);
    }

    const int nvalid = min(kBlock, L - j * kBlock);
    float alpha[GR];
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
      const float mnew = fmaxf(m_run[r], mx);
      alpha[r] = fast_exp2(m_run[r] - mnew);
      m_run[r] = mnew;
      float ps = 0.f;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const float pv = fast_exp2(s[t4] - mnew);
        ps += pv;
        pl[(16 * t4 + arow) * GP + 4 * r + kg] = pv;
      }
      l_run[r] = l_run[r] * alpha[r] + ps;
    }
    wave_lds_exchange();  // P rows written above are read across lanes below

    // rescale the running P.V sums when a query's max moved
    float al[GP];
    bool moved = false;
#pragma unroll
    for (int q = 0; q < GP; ++q) {
      al[q] = readlane(alpha[q >> 2], 16 * (q & 3));
      moved |= al[q] != 1.f;
    }
    if (moved) {
#pragma unroll
      for (int q = 0; q < GP; ++q)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[q][e] *= al[q];
    }

    // P.V in the row layout
#pragma unroll
    for (int i = 0; i < CPR; ++i) {
      const int t = i * TPI + lane / CPR;
      float pq[GP];
#pragma unroll
      for (int r = 0; r < GR; ++r) {
        const f32x4 x = *(const f32x4*)(pl + t * GP + 4 * r);
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
        for (int e = 0; e < E; ++e) acc[q][e] = fmaf(pq[q], vf[e], acc[q][e]);
    }
    wave_lds_exchange();  // before the next block overwrites P
    if (more) load_v(jn);
  }

  // wave state: l over the 16 lanes of each row, P.V over the token phases
#pragma unroll
  for (int r = 0; r < GR; ++r) l_run[r] = row16_sum(l_run[r]);
#pragma unroll
  for (int q = 0; q < GP; ++q)
#pragma unroll
    for (int e = 0; e < E; ++e)
      acc[q][e] = phase_sum<CPR>(acc[q][e]);

  if (arow == 0) {
#pragma unroll
    for (int r = 0; r < GR; ++r) {
      red_m[w][4 * r + kg] = m_run[r];
      red_l[w][4 * r + kg] = l_run[r];
    }
  }
  if (lane < CPR) {
#pragma unroll
    for (int q = 0; q < GP; ++q)
#pragma unroll
      for (int e = 0; e < E; ++e) red_acc[w][q][lane * E + e] = acc[q][e];
  }
  __syncthreads();

  // merge the waves and write the split state
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int q = idx / D, dd = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, red_m[ww][q]);
    float ls = 0.f, os = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        const float f = fast_exp2(red_m[ww][q] - M);
        ls = fmaf(red_l[ww][q], f, ls);
        os = fmaf(red_acc[ww][q][dd], f, os);
      }
    }
    const size_t row = ((size_t)b * p.Hq + (size_t)g * G + q) * p.S + split;
    p.o[row * D + dd] = ls > 0.f ? os / ls : 0.f;
    if (dd == 0) {
      p.m[row] = ls > 0.f ? M * kLn2 : -INFINITY;
      p.l[row] = ls;
    }
  }
}

template <typename T, int D, int GR>
hipError_t launch_t(const DecodeArgs& a, bool sparse, hipStream_t st) {
  const dim3 grid(a.S, a.Hkv, a.B);
  const bool paged = a.table != nullptr;
  if (sparse) {
    if (paged)
      decode_kernel<T, D, GR, true, true><<<grid, 256, 0, st>>>(a);
    else
      decode_kernel<T, D, GR, true, false><<<grid, 256, 0, st>>>(a);
  } else {
    if (paged)
      decode_kernel<T, D, GR, false, true><<<grid, 256, 0, st>>>(a);
    else
      decode_kernel<T, D, GR, false, false><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const DecodeArgs& a, bool sparse, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  return G <= 4 ? launch_t<T, D, 1>(a, sparse, st) : launch_t<T, D, 2>(a, sparse, st);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool sparse, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  if (a.dtype == 1)
    return a.d == 128 ? launch_g<__bf16, 128>(a, sparse, st) : launch_g<__bf16, 64>(a, sparse, st);
  return a.d == 128 ? launch_g<float, 128>(a, sparse, st) : launch_g<float, 64>(a, sparse, st);
}

}  // namespace skv
