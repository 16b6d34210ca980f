// C ABI of the decode-attention library: argument checks and kernel dispatch.
// Every kernel is queued on the caller's stream and nothing here allocates,
// frees or synchronises.  The one piece of device state is the static scratch
// array of attn_decode_routed_static (with its per-device address cache).
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "kernels.hpp"
#include "sparse_kv.h"

// Scratch of attn_decode_routed_static: one copy per device, for the life of
// the process.  Host code never uses the array's name as an address (on the
// host it is only a handle to the symbol); each device's address is taken
// once, with that device current, and kept (static_scratch below).
static __device__ __align__(256) char scratch[ATTN_ROUTED_STATIC_BYTES];

namespace {

constexpr int32_t kMaxGrid = 65535;

int check_dims(const attn_dims* d) {
  if (!d) return ATTN_ERR_INVALID_ARG;
  if (d->batch < 0 || d->batch > kMaxGrid) return ATTN_ERR_INVALID_ARG;
  if (d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_kv_heads > kMaxGrid) return ATTN_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return ATTN_ERR_INVALID_ARG;
  if (d->head_dim < 1 || d->block_size < 1 || d->max_blocks < 1) return ATTN_ERR_INVALID_ARG;
  if (d->dtype != ATTN_F32 && d->dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(d->scale)) return ATTN_ERR_INVALID_ARG;
  if (d->head_dim != 64 && d->head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (d->block_size != 64) return ATTN_ERR_UNSUPPORTED;
  if (d->num_q_heads / d->num_kv_heads > 8) return ATTN_ERR_UNSUPPORTED;
  // one (b, kv head) slice of K or V is one buffer resource, whose range
  // (the slice's valid bytes) is a signed 32-bit field
  const uint64_t row_bytes = (uint64_t)d->head_dim * (d->dtype == ATTN_BF16 ? 2 : 4);
  if ((uint64_t)d->max_blocks * 64 * row_bytes > (1ull << 31)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

skv::DecodeArgs decode_args(const attn_dims* d, const void* q, const void* k, const void* v,
                            const int32_t* seq_lens, int32_t S, float* m, float* l, float* o) {
  skv::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.seq_lens = seq_lens;
  a.m = m;
  a.l = l;
  a.o = o;
  a.B = d->batch;
  a.Hq = d->num_q_heads;
  a.Hkv = d->num_kv_heads;
  a.d = d->head_dim;
  a.NBmax = d->max_blocks;
  a.S = S;
  a.block_begin = 0;
  a.block_end = -1;
  a.dtype = d->dtype;
  a.scale = d->scale;
  return a;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct RoutedLayout {
  size_t m, l, o, sm, sl, so, total;  // byte offsets into the workspace
};

RoutedLayout routed_layout(const attn_dims* d, int32_t n_shards, int32_t sps, int32_t sa_splits) {
  const size_t rows = (size_t)d->batch * d->num_q_heads;
  const int64_t S = (int64_t)n_shards * sps;
  const size_t Smax = (size_t)(S > sa_splits ? S : sa_splits);
  RoutedLayout r{};
  size_t off = 0;
  r.m = off;
  off += align256(rows * Smax * 4);
  r.l = off;
  off += align256(rows * Smax * 4);
  r.o = off;
  off += align256(rows * Smax * d->head_dim * 4);
  r.sm = off;
  off += align256(rows * n_shards * 4);
  r.sl = off;
  off += align256(rows * n_shards * 4);
  r.so = off;
  off += align256(rows * n_shards * d->head_dim * 4);
  r.total = off;
  return r;
}

// Paged cache: the pools, the pool size and the table must be given, and the
// table must hold a row of at least max_blocks entries.
int check_paged(const attn_dims* d, const attn_paged_kv* kv, bool need_v) {
  if (!kv || !kv->k_pool || (need_v && !kv->v_pool) || !kv->block_table) return ATTN_ERR_INVALID_ARG;
  if (kv->pool_blocks < 1 || kv->table_stride < d->max_blocks) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

void set_paged(skv::DecodeArgs& a, const attn_paged_kv* kv) {
  a.k = kv->k_pool;
  a.v = kv->v_pool;
  a.table = kv->block_table;
  a.table_stride = kv->table_stride;
  a.pool_blocks = kv->pool_blocks;
}

// Host-side checks shared by the routed entry points (nothing is queued on failure).
int routed_check(const attn_dims* dims, int32_t n_layers, const uint8_t* route_mask, const void* const* q,
                 const void* const* k, const void* const* v, int32_t n_shards, int32_t splits_per_shard,
                 const int32_t* sa_block_idx, const int32_t* sa_n_sel, int32_t sa_max_sel, int32_t sa_splits,
                 float* const* out) {
  int st = check_dims(dims);
  if (st) return st;
  if (n_layers < 0 || !route_mask || !q || !k || !v || !out) return ATTN_ERR_INVALID_ARG;
  if (n_shards < 1 || splits_per_shard < 1 || sa_splits < 1 || sa_splits > (1 << 24)) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)n_shards * splits_per_shard > (1 << 24)) return ATTN_ERR_INVALID_ARG;
  if ((int64_t)dims->batch * dims->num_q_heads * n_shards > 0x7fffffff) return ATTN_ERR_INVALID_ARG;
  bool any_sa = false;
  for (int32_t i = 0; i < n_layers; ++i) {
    if (!q[i] || !k[i] || !v[i] || !out[i]) return ATTN_ERR_INVALID_ARG;
    any_sa |= route_mask[i] == 0;
  }
  if (any_sa && (!sa_block_idx || !sa_n_sel || sa_max_sel < 1)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

// The layers of a routed stack, queued in order; ws holds routed_layout's buffers.
int routed_run(const attn_dims* dims, int32_t n_layers, const uint8_t* route_mask, const void* const* q,
               const void* const* k, const void* const* v, const int32_t* seq_lens, int32_t n_shards,
               int32_t splits_per_shard, const int32_t* sa_block_idx, const int32_t* sa_n_sel, int32_t sa_max_sel,
               int32_t sa_splits, char* ws, float* const* out, hipStream_t s) {
  if (dims->batch == 0 || n_layers == 0) return ATTN_OK;
  const RoutedLayout lay = routed_layout(dims, n_shards, splits_per_shard, sa_splits);
  float* m = (float*)(ws + lay.m);
  float* l = (float*)(ws + lay.l);
  float* o = (float*)(ws + lay.o);
  float* sm = (float*)(ws + lay.sm);
  float* sl = (float*)(ws + lay.sl);
  float* so = (float*)(ws + lay.so);
  const int32_t rows = dims->batch * dims->num_q_heads;
  const int32_t S = n_shards * splits_per_shard;
  for (int32_t i = 0; i < n_layers; ++i) {
    hipError_t e;
    if (route_mask[i]) {
      // full attention: shard-aligned splits, merged per shard, then across
      // shards (both levels in one launch when a row's states fit one wave)
      skv::DecodeArgs a = decode_args(dims, q[i], k[i], v[i], seq_lens, S, m, l, o);
      e = skv::launch_decode(a, false, s);
      if (e == hipSuccess && S <= 64) {
        e = skv::launch_merge2(rows, n_shards, splits_per_shard, dims->head_dim, m, l, o, out[i], s);
      } else if (e == hipSuccess) {
        e = skv::launch_merge(rows * n_shards, splits_per_shard, dims->head_dim, m, l, o, so, sm, sl, s);
        if (e == hipSuccess)
          e = skv::launch_merge(rows, n_shards, dims->head_dim, sm, sl, so, out[i], nullptr, nullptr, s);
      }
    } else {
      skv::DecodeArgs a = decode_args(dims, q[i], k[i], v[i], seq_lens, sa_splits, m, l, o);
      a.block_idx = sa_block_idx;
      a.n_sel = sa_n_sel;
      a.max_sel = sa_max_sel;
      e = skv::launch_decode(a, true, s);
      if (e == hipSuccess) e = skv::launch_merge(rows, sa_splits, dims->head_dim, m, l, o, out[i], nullptr, nullptr, s);
    }
    if (e != hipSuccess) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
char* scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// The device that work queued on `s` runs on.
int stream_device(hipStream_t s, int* dev) {
  const hipError_t e = s ? hipStreamGetDevice(s, dev) : hipGetDevice(dev);
  if (e != hipSuccess) return ATTN_ERR_HIP;
  return *dev >= 0 && *dev < kMaxDevices ? ATTN_OK : ATTN_ERR_UNSUPPORTED;
}

int static_scratch(hipStream_t s, char** ptr) {
  int dev = 0;
  int st = stream_device(s, &dev);
  if (st) return st;
  std::call_once(scratch_once[dev], [dev] {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    scratch_err[dev] = e;
    scratch_ptr[dev] = e == hipSuccess ? (char*)p : nullptr;
  });
  if (scratch_err[dev] != hipSuccess || !scratch_ptr[dev]) return ATTN_ERR_HIP;
  *ptr = scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK:
      return "ok";
    case ATTN_ERR_INVALID_ARG:
      return "invalid argument";
    case ATTN_ERR_UNSUPPORTED:
      return "unsupported shape or dtype (head_dim must be 64 or 128, block_size 64, Hq/Hkv <= 8)";
    case ATTN_ERR_HIP:
      return "HIP launch or runtime error";
    case ATTN_ERR_WORKSPACE:
      return "workspace too small";
    default:
      return "unknown status";
  }
}

int attn_decode_dense(const attn_dims* dims, const void* q, const void* k, const void* v,
                      const int32_t* seq_lens, int32_t block_begin, int32_t block_end,
                      int32_t num_splits, float* m, float* l, float* o, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !k || !v || !m || !l || !o) return ATTN_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > (1 << 24) || block_begin < 0) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  skv::DecodeArgs a = decode_args(dims, q, k, v, seq_lens, num_splits, m, l, o);
  a.block_begin = block_begin;
  a.block_end = block_end;
  return hip_status(skv::launch_decode(a, false, (hipStream_t)stream));
}

int attn_decode_dense_paged(const attn_dims* dims, const void* q, const attn_paged_kv* kv, const int32_t* seq_lens,
                            int32_t block_begin, int32_t block_end, int32_t num_splits, float* m, float* l,
                            float* o, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_paged(dims, kv, true))) return st;
  if (!q || !m || !l || !o) return ATTN_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > (1 << 24) || block_begin < 0) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  skv::DecodeArgs a = decode_args(dims, q, nullptr, nullptr, seq_lens, num_splits, m, l, o);
  set_paged(a, kv);
  a.block_begin = block_begin;
  a.block_end = block_end;
  return hip_status(skv::launch_decode(a, false, (hipStream_t)stream));
}

int attn_decode_sparse_paged(const attn_dims* dims, const void* q, const attn_paged_kv* kv,
                             const int32_t* seq_lens, const int32_t* block_idx, const int32_t* n_sel,
                             int32_t max_sel, int32_t num_splits, float* m, float* l, float* o, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_paged(dims, kv, true))) return st;
  if (!q || !block_idx || !n_sel || !m || !l || !o) return ATTN_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > (1 << 24) || max_sel < 1) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  skv::DecodeArgs a = decode_args(dims, q, nullptr, nullptr, seq_lens, num_splits, m, l, o);
  set_paged(a, kv);
  a.block_idx = block_idx;
  a.n_sel = n_sel;
  a.max_sel = max_sel;
  return hip_status(skv::launch_decode(a, true, (hipStream_t)stream));
}

int attn_merge_states(int32_t rows, int32_t num_splits, int32_t head_dim, const float* m,
                      const float* l, const float* o, float* out, float* m_out, float* l_out,
                      void* stream) {
  if (rows < 0 || num_splits < 1) return ATTN_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return head_dim < 1 ? ATTN_ERR_INVALID_ARG : ATTN_ERR_UNSUPPORTED;
  if (!m || !l || !o || !out) return ATTN_ERR_INVALID_ARG;
  if (rows == 0) return ATTN_OK;
  return hip_status(skv::launch_merge(rows, num_splits, head_dim, m, l, o, out, m_out, l_out,
                                      (hipStream_t)stream));
}

int attn_build_centroids(const attn_dims* dims, const void* k, const int32_t* seq_lens,
                         float* centroids, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!k || !centroids) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  return hip_status(skv::launch_build_centroids(k, seq_lens, centroids, dims->batch, dims->num_kv_heads,
                                                dims->head_dim, dims->max_blocks, dims->dtype,
                                                (hipStream_t)stream));
}

int attn_build_centroids_paged(const attn_dims* dims, const attn_paged_kv* kv, const int32_t* seq_lens,
                               float* centroids, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_paged(dims, kv, false))) return st;
  if (!centroids) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  const skv::PagedK pg{kv->block_table, kv->table_stride, kv->pool_blocks};
  return hip_status(skv::launch_build_centroids(kv->k_pool, seq_lens, centroids, dims->batch, dims->num_kv_heads,
                                                dims->head_dim, dims->max_blocks, dims->dtype,
                                                (hipStream_t)stream, pg));
}

int attn_update_centroids_paged(const attn_dims* dims, const attn_paged_kv* kv, const int32_t* seq_lens,
                                const int32_t* prev_lens, int32_t span_hint, float* centroids, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_paged(dims, kv, false))) return st;
  if (!centroids || span_hint < 1) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  const skv::PagedK pg{kv->block_table, kv->table_stride, kv->pool_blocks};
  return hip_status(skv::launch_update_centroids(kv->k_pool, seq_lens, prev_lens, centroids, dims->batch,
                                                 dims->num_kv_heads, dims->head_dim, dims->max_blocks,
                                                 dims->dtype, span_hint, (hipStream_t)stream, pg));
}

int attn_update_centroids(const attn_dims* dims, const void* k, const int32_t* seq_lens,
                          const int32_t* prev_lens, int32_t span_hint, float* centroids, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!k || !centroids || span_hint < 1) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  return hip_status(skv::launch_update_centroids(k, seq_lens, prev_lens, centroids, dims->batch,
                                                 dims->num_kv_heads, dims->head_dim, dims->max_blocks,
                                                 dims->dtype, span_hint, (hipStream_t)stream));
}

int attn_score_centroids(const attn_dims* dims, const void* q, const float* centroids,
                         const int32_t* seq_lens, float* scores, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !centroids || !scores) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  return hip_status(skv::launch_score(q, centroids, seq_lens, scores, dims->batch, dims->num_q_heads,
                                      dims->num_kv_heads, dims->head_dim, dims->max_blocks, dims->dtype,
                                      dims->scale, (hipStream_t)stream));
}

int attn_select_topk(const attn_dims* dims, const float* scores, const int32_t* seq_lens,
                     int32_t k, int32_t n_sink_blocks, int32_t n_recent_blocks, int32_t max_sel,
                     int32_t* block_idx, int32_t* n_sel, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (k < 0 || n_sink_blocks < 0 || n_recent_blocks < 0 || max_sel < 1) return ATTN_ERR_INVALID_ARG;
  if (!block_idx || !n_sel || (k > 0 && !scores)) return ATTN_ERR_INVALID_ARG;
  const int64_t need = (int64_t)n_sink_blocks + n_recent_blocks + k;
  if ((int64_t)max_sel < (need < dims->max_blocks ? need : (int64_t)dims->max_blocks)) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  return hip_status(skv::launch_topk(scores, seq_lens, dims->batch, dims->num_kv_heads, dims->max_blocks, k,
                                     n_sink_blocks, n_recent_blocks, max_sel, block_idx, n_sel,
                                     (hipStream_t)stream));
}

int attn_build_super_centroids(const attn_dims* dims, const float* centroids, const int32_t* seq_lens,
                               int32_t group, float* super_centroids, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!centroids || !super_centroids || group < 1) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  return hip_status(skv::launch_super_centroids(centroids, seq_lens, super_centroids, dims->batch,
                                                dims->num_kv_heads, dims->head_dim, dims->max_blocks, group,
                                                (hipStream_t)stream));
}

int attn_select_two_level(const attn_dims* dims, const void* q, const float* centroids,
                          const float* super_centroids, const int32_t* seq_lens, int32_t group,
                          int32_t k_coarse, int32_t k, int32_t n_sink_blocks, int32_t n_recent_blocks,
                          int32_t max_sel, int32_t* block_idx, int32_t* n_sel, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !centroids || !super_centroids || !block_idx || !n_sel) return ATTN_ERR_INVALID_ARG;
  if (group < 1 || k_coarse < 0 || k < 0 || n_sink_blocks < 0 || n_recent_blocks < 0 || max_sel < 1)
    return ATTN_ERR_INVALID_ARG;
  const int64_t need = (int64_t)n_sink_blocks + n_recent_blocks + k;
  if ((int64_t)max_sel < (need < dims->max_blocks ? need : (int64_t)dims->max_blocks)) return ATTN_ERR_INVALID_ARG;
  const int64_t ns = ((int64_t)dims->max_blocks + group - 1) / group;
  if (ns > skv::kTwoLevelMaxSuper) return ATTN_ERR_UNSUPPORTED;
  if ((k_coarse < ns ? (int64_t)k_coarse : ns) * group > skv::kTwoLevelMaxCand) return ATTN_ERR_UNSUPPORTED;
  if (dims->batch == 0) return ATTN_OK;
  return hip_status(skv::launch_two_level(q, centroids, super_centroids, seq_lens, dims->batch, dims->num_q_heads,
                                          dims->num_kv_heads, dims->head_dim, dims->max_blocks, dims->dtype,
                                          dims->scale, group, k_coarse, k, n_sink_blocks, n_recent_blocks, max_sel,
                                          block_idx, n_sel, (hipStream_t)stream));
}

int attn_decode_sparse(const attn_dims* dims, const void* q, const void* k, const void* v,
                       const int32_t* seq_lens, const int32_t* block_idx, const int32_t* n_sel,
                       int32_t max_sel, int32_t num_splits, float* m, float* l, float* o,
                       void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !k || !v || !block_idx || !n_sel || !m || !l || !o) return ATTN_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > (1 << 24) || max_sel < 1) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  skv::DecodeArgs a = decode_args(dims, q, k, v, seq_lens, num_splits, m, l, o);
  a.block_idx = block_idx;
  a.n_sel = n_sel;
  a.max_sel = max_sel;
  return hip_status(skv::launch_decode(a, true, (hipStream_t)stream));
}

static int art_common(const attn_dims* dims, const void* q, const void* k, const void* v,
                      const int32_t* seq_lens, const int32_t* order, int32_t order_stride,
                      const int32_t* n_visit, float tau, float phi, int32_t patience,
                      int32_t probe_dim, float* out, int32_t* stop_pos, int32_t* blocks_fetched,
                      void* stream, const attn_paged_kv* kv = nullptr, void* workspace = nullptr,
                      size_t workspace_bytes = 0) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !k || !v || !out || !stop_pos) return ATTN_ERR_INVALID_ARG;
  if (patience < 1 || probe_dim < 0 || isnan(tau) || isnan(phi)) return ATTN_ERR_INVALID_ARG;
  if (probe_dim > 16 || probe_dim > dims->head_dim) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)dims->batch * dims->num_kv_heads > 0x7fffffff) return ATTN_ERR_INVALID_ARG;
  if (dims->batch == 0) return ATTN_OK;
  skv::ArtArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.seq_lens = seq_lens;
  a.order = order;
  a.order_stride = order_stride;
  a.n_visit = n_visit;
  a.tau = tau;
  a.phi = phi;
  a.patience = patience;
  a.probe_dim = probe_dim;
  a.out = out;
  a.stop_pos = stop_pos;
  a.blocks_fetched = blocks_fetched;
  a.B = dims->batch;
  a.Hq = dims->num_q_heads;
  a.Hkv = dims->num_kv_heads;
  a.d = dims->head_dim;
  a.NBmax = dims->max_blocks;
  a.dtype = dims->dtype;
  a.scale = dims->scale;
  if (kv) {
    a.table = kv->block_table;
    a.table_stride = kv->table_stride;
    a.pool_blocks = kv->pool_blocks;
  }
  return hip_status(skv::launch_art(a, (hipStream_t)stream, workspace, workspace_bytes));
}

int attn_decode_art_paged(const attn_dims* dims, const void* q, const attn_paged_kv* kv, const int32_t* seq_lens,
                          const int32_t* order, float tau, float phi, int32_t patience, int32_t probe_dim,
                          float* out, int32_t* stop_pos, int32_t* blocks_fetched, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if ((st = check_paged(dims, kv, true))) return st;
  return art_common(dims, q, kv->k_pool, kv->v_pool, seq_lens, order, dims->max_blocks, nullptr, tau, phi,
                    patience, probe_dim, out, stop_pos, blocks_fetched, stream, kv);
}

int attn_decode_art(const attn_dims* dims, const void* q, const void* k, const void* v,
                    const int32_t* seq_lens, const int32_t* order, float tau, float phi,
                    int32_t patience, int32_t probe_dim, float* out, int32_t* stop_pos,
                    int32_t* blocks_fetched, void* stream) {
  const int32_t stride = dims ? dims->max_blocks : 0;
  return art_common(dims, q, k, v, seq_lens, order, stride, nullptr, tau, phi, patience, probe_dim,
                    out, stop_pos, blocks_fetched, stream);
}

size_t attn_art_workspace_bytes(const attn_dims* dims) {
  if (check_dims(dims) != ATTN_OK) return 0;
  const int64_t units = (int64_t)dims->batch * dims->num_kv_heads;
  if (units > skv::kArtMcMaxUnits) return 0;
  return skv::art_workspace_bytes((int32_t)units, dims->num_q_heads / dims->num_kv_heads, dims->head_dim);
}

// The workspace an ART call across workgroups needs: null when none is
// needed (the call then runs one workgroup per unit); *st non-zero on error.
static void* art_workspace(const attn_dims* dims, void* workspace, size_t workspace_bytes, int* st) {
  *st = check_dims(dims);
  if (*st) return nullptr;
  const size_t need = attn_art_workspace_bytes(dims);
  if (need && !workspace) *st = ATTN_ERR_INVALID_ARG;
  else if (workspace_bytes < need) *st = ATTN_ERR_WORKSPACE;
  return need ? workspace : nullptr;
}

int attn_decode_art_ws(const attn_dims* dims, const void* q, const void* k, const void* v,
                       const int32_t* seq_lens, const int32_t* order, float tau, float phi,
                       int32_t patience, int32_t probe_dim, void* workspace, size_t workspace_bytes,
                       float* out, int32_t* stop_pos, int32_t* blocks_fetched, void* stream) {
  int st;
  void* ws = art_workspace(dims, workspace, workspace_bytes, &st);
  if (st) return st;
  return art_common(dims, q, k, v, seq_lens, order, dims->max_blocks, nullptr, tau, phi, patience, probe_dim,
                    out, stop_pos, blocks_fetched, stream, nullptr, ws, workspace_bytes);
}

int attn_decode_art_list_ws(const attn_dims* dims, const void* q, const void* k, const void* v,
                            const int32_t* seq_lens, const int32_t* block_list, const int32_t* n_list,
                            int32_t max_list, float tau, float phi, int32_t patience, int32_t probe_dim,
                            void* workspace, size_t workspace_bytes, float* out, int32_t* stop_pos,
                            int32_t* blocks_fetched, void* stream) {
  int st;
  void* ws = art_workspace(dims, workspace, workspace_bytes, &st);
  if (st) return st;
  if (!block_list || !n_list || max_list < 1) return ATTN_ERR_INVALID_ARG;
  return art_common(dims, q, k, v, seq_lens, block_list, max_list, n_list, tau, phi, patience, probe_dim, out,
                    stop_pos, blocks_fetched, stream, nullptr, ws, workspace_bytes);
}

int attn_decode_art_paged_ws(const attn_dims* dims, const void* q, const attn_paged_kv* kv,
                             const int32_t* seq_lens, const int32_t* order, float tau, float phi,
                             int32_t patience, int32_t probe_dim, void* workspace, size_t workspace_bytes,
                             float* out, int32_t* stop_pos, int32_t* blocks_fetched, void* stream) {
  int st;
  void* ws = art_workspace(dims, workspace, workspace_bytes, &st);
  if (st) return st;
  if ((st = check_paged(dims, kv, true))) return st;
  return art_common(dims, q, kv->k_pool, kv->v_pool, seq_lens, order, dims->max_blocks, nullptr, tau, phi,
                    patience, probe_dim, out, stop_pos, blocks_fetched, stream, kv, ws, workspace_bytes);
}

int attn_decode_art_list(const attn_dims* dims, const void* q, const void* k, const void* v,
                         const int32_t* seq_lens, const int32_t* block_list, const int32_t* n_list,
                         int32_t max_list, float tau, float phi, int32_t patience, int32_t probe_dim,
                         float* out, int32_t* stop_pos, int32_t* blocks_fetched, void* stream) {
  if (!block_list || !n_list || max_list < 1) return ATTN_ERR_INVALID_ARG;
  return art_common(dims, q, k, v, seq_lens, block_list, max_list, n_list, tau, phi, patience,
                    probe_dim, out, stop_pos, blocks_fetched, stream);
}

int attn_order_blocks(const attn_dims* dims, const float* scores, const int32_t* seq_lens,
                      int32_t* order, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!scores || !order) return ATTN_ERR_INVALID_ARG;
  if (dims->max_blocks - 1 > skv::kOrderMaxRest) return ATTN_ERR_UNSUPPORTED;
  if (dims->batch == 0) return ATTN_OK;
  return hip_status(skv::launch_order(scores, seq_lens, dims->batch, dims->num_kv_heads,
                                      dims->max_blocks, order, (hipStream_t)stream));
}

size_t attn_routed_workspace_bytes(const attn_dims* dims, int32_t n_shards, int32_t splits_per_shard,
                                   int32_t sa_splits) {
  if (check_dims(dims) != ATTN_OK || n_shards < 1 || splits_per_shard < 1 || sa_splits < 1) return 0;
  return routed_layout(dims, n_shards, splits_per_shard, sa_splits).total;
}

int attn_decode_routed(const attn_dims* dims, int32_t n_layers, const uint8_t* route_mask,
                       const void* const* q, const void* const* k, const void* const* v,
                       const int32_t* seq_lens, int32_t n_shards, int32_t splits_per_shard,
                       const int32_t* sa_block_idx, const int32_t* sa_n_sel, int32_t sa_max_sel,
                       int32_t sa_splits, void* workspace, size_t workspace_bytes,
                       float* const* out, void* stream) {
  int st = routed_check(dims, n_layers, route_mask, q, k, v, n_shards, splits_per_shard, sa_block_idx, sa_n_sel,
                        sa_max_sel, sa_splits, out);
  if (st) return st;
  if (!workspace) return ATTN_ERR_INVALID_ARG;
  if (workspace_bytes < routed_layout(dims, n_shards, splits_per_shard, sa_splits).total) return ATTN_ERR_WORKSPACE;
  return routed_run(dims, n_layers, route_mask, q, k, v, seq_lens, n_shards, splits_per_shard, sa_block_idx,
                    sa_n_sel, sa_max_sel, sa_splits, (char*)workspace, out, (hipStream_t)stream);
}

int attn_decode_routed_static(const attn_dims* dims, int32_t n_layers, const uint8_t* route_mask,
                              const void* const* q, const void* const* k, const void* const* v,
                              const int32_t* seq_lens, int32_t n_shards, int32_t splits_per_shard,
                              const int32_t* sa_block_idx, const int32_t* sa_n_sel, int32_t sa_max_sel,
                              int32_t sa_splits, float* const* out, void* stream) {
  int st = routed_check(dims, n_layers, route_mask, q, k, v, n_shards, splits_per_shard, sa_block_idx, sa_n_sel,
                        sa_max_sel, sa_splits, out);
  if (st) return st;
  if (routed_layout(dims, n_shards, splits_per_shard, sa_splits).total > ATTN_ROUTED_STATIC_BYTES)
    return ATTN_ERR_WORKSPACE;
  if (dims->batch == 0 || n_layers == 0) return ATTN_OK;
  char* ws = nullptr;
  if ((st = static_scratch((hipStream_t)stream, &ws))) return st;
  return routed_run(dims, n_layers, route_mask, q, k, v, seq_lens, n_shards, splits_per_shard, sa_block_idx,
                    sa_n_sel, sa_max_sel, sa_splits, ws, out, (hipStream_t)stream);
}

}  // extern "C"
