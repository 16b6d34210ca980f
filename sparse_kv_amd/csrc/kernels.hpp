// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;   // may be null: every row has NBmax * 64 tokens
  const int32_t* block_idx;  // sparse only
  const int32_t* n_sel;      // sparse only
  int32_t max_sel;           // sparse only
  float* m;
  float* l;
  float* o;
  int32_t B, Hq, Hkv, d, NBmax, S, block_begin, block_end, dtype;
  float scale;
  // paged cache: k, v are pools [pool_blocks, Hkv, 64, d] and table[b *
  // table_stride + j] is the pool block of logical block j (null: k, v are
  // contiguous [B, Hkv, NBmax * 64, d])
  const int32_t* table;
  int32_t table_stride;
  int64_t pool_blocks;
};

struct ArtArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* seq_lens;
  const int32_t* order;    // may be null: block 0, then the newest block backwards
  int32_t order_stride;    // elements per (b, kv head) row of order
  const int32_t* n_visit;  // may be null: visit every block of the sequence
  float tau, phi;
  int32_t patience, probe_dim;
  float* out;
  int32_t* stop_pos;
  int32_t* blocks_fetched;  // may be null
  int32_t B, Hq, Hkv, d, NBmax, dtype;
  float scale;
  const int32_t* table;  // paged cache, as in DecodeArgs
  int32_t table_stride;
  int64_t pool_blocks;
};

hipError_t launch_decode(const DecodeArgs& a, bool sparse, hipStream_t st);
hipError_t launch_merge(int32_t rows, int32_t S, int32_t d, const float* m, const float* l,
                        const float* o, float* out, float* m_out, float* l_out, hipStream_t st);
// Both levels of a shard merge in one launch (shards * inner <= 64): states
// [rows, shards, inner] merged per shard, then across shards.
hipError_t launch_merge2(int32_t rows, int32_t shards, int32_t inner, int32_t d, const float* m, const float* l,
                         const float* o, float* out, hipStream_t st);
// Paged K for the centroid kernels: null table = contiguous k.
struct PagedK {
  const int32_t* table;
  int32_t table_stride;
  int64_t pool_blocks;
};
hipError_t launch_build_centroids(const void* k, const int32_t* seq_lens, float* c, int32_t B,
                                  int32_t Hkv, int32_t d, int32_t NBmax, int32_t dtype,
                                  hipStream_t st, PagedK pg = PagedK{nullptr, 0, 0});
hipError_t launch_update_centroids(const void* k, const int32_t* seq_lens, const int32_t* prev_lens, float* c,
                                   int32_t B, int32_t Hkv, int32_t d, int32_t NBmax, int32_t dtype,
                                   int32_t span_hint, hipStream_t st, PagedK pg = PagedK{nullptr, 0, 0});
hipError_t launch_score(const void* q, const float* c, const int32_t* seq_lens, float* scores,
                        int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t NBmax,
                        int32_t dtype, float scale, hipStream_t st);
hipError_t launch_topk(const float* scores, const int32_t* seq_lens, int32_t B, int32_t Hkv,
                       int32_t NBmax, int32_t k, int32_t n_sink, int32_t n_recent,
                       int32_t max_sel, int32_t* idx, int32_t* n_sel, hipStream_t st);
// ART with several workgroups per (b, kv head) unit when the grid is small:
// needs a workspace of art_workspace_bytes (0 beyond kArtMcMaxUnits units);
// without one, or on a device with fewer than 2 CUs per unit, one workgroup
// per unit.
constexpr int kArtMcMaxUnits = 128;
constexpr int kArtMcMaxGroups = 4;
constexpr int kArtRingSlots = 128;
hipError_t launch_art(const ArtArgs& a, hipStream_t st, void* ws = nullptr, size_t ws_bytes = 0);
size_t art_workspace_bytes(int32_t units, int32_t G, int32_t d);
// Two-level selection capacities: super-blocks per sequence, and fine
// candidates (k_coarse * group) inside the opened super-blocks.
constexpr int32_t kTwoLevelMaxSuper = 4096;
constexpr int32_t kTwoLevelMaxCand = 8192;
hipError_t launch_super_centroids(const float* c, const int32_t* seq_lens, float* c2, int32_t B, int32_t Hkv,
                                  int32_t d, int32_t NBmax, int32_t group, hipStream_t st);
hipError_t launch_two_level(const void* q, const float* c, const float* c2, const int32_t* seq_lens, int32_t B,
                            int32_t Hq, int32_t Hkv, int32_t d, int32_t NBmax, int32_t dtype, float scale,
                            int32_t group, int32_t k_coarse, int32_t k, int32_t n_sink, int32_t n_recent,
                            int32_t max_sel, int32_t* idx, int32_t* n_sel, hipStream_t st);
// Largest number of non-sink blocks a sequence may have for launch_order.
constexpr int32_t kOrderMaxRest = 16384;
hipError_t launch_order(const float* scores, const int32_t* seq_lens, int32_t B, int32_t Hkv,
                        int32_t NBmax, int32_t* order, hipStream_t st);

}  // namespace skv
