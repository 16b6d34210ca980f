/*
 * sparse_kv -- long-context decode attention over a block-organised KV cache
 * for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer argument is a DEVICE pointer unless its comment says
 * "host".  The caller owns every buffer; the library never allocates, frees
 * or synchronises, and queues all work on `stream` (a hipStream_t passed as
 * void*; NULL = the default stream).  Its only global state is the scratch
 * array of attn_decode_routed_static.  Functions are reentrant and may be
 * called concurrently on different streams (attn_decode_routed_static: see
 * there).
 *
 * Errors: every function returns an attn_status.  Host-visible arguments
 * (pointers for NULL, sizes, dims) are checked before anything is queued;
 * on a check failure nothing is queued.  ATTN_ERR_HIP is returned when a
 * launch reports an error.  Values that live in device memory (seq_lens,
 * block lists, visit orders) are preconditions stated per function: kernels
 * clamp indices into range so that a violation cannot read outside the
 * buffers, but the result is then unspecified.
 *
 * Shapes (row-major, contiguous):
 *   q        [B, Hq, d]                       dtype
 *   k, v     [B, Hkv, max_blocks * 64, d]     dtype
 *   seq_lens int32 [B], 0 <= L_b <= max_blocks * 64; NULL means every L_b is
 *            max_blocks * 64.  Tokens at or beyond L_b are never read.
 * Query head h reads KV head h / (Hq / Hkv) (grouped-query attention).
 * A block is 64 consecutive tokens; block j of row b covers tokens
 * [64 j, min(64 j + 64, L_b)); nb(b) = ceil(L_b / 64).
 *
 * Softmax states (m, l, o): for a token set J and logits
 * s_t = scale * <q, k_t>:  m = max_J s_t (natural-log units),
 * l = sum_J exp(s_t - m), o = sum_J exp(s_t - m) v_t / l (normalised).
 * The empty set has the state (-inf, 0, 0).
 */
#ifndef SPARSE_KV_H
#define SPARSE_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbol visibility; the declarations below
 * are its whole exported interface. */
#pragma GCC visibility push(default)

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1, /* a NULL required pointer, a bad size or dim      */
  ATTN_ERR_UNSUPPORTED = -2, /* valid but not built: d not in {64,128}, G > 8,
                                a head's K slice above 2 GiB, and the per-
                                function limits stated below                  */
  ATTN_ERR_HIP = -3,         /* a launch or HIP runtime call failed             */
  ATTN_ERR_WORKSPACE = -4    /* the workspace given is too small                */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype; /* q, k, v share it */

typedef struct {
  int32_t batch;        /* B >= 0                                          */
  int32_t num_q_heads;  /* Hq >= 1, a multiple of Hkv                      */
  int32_t num_kv_heads; /* Hkv >= 1; G = Hq / Hkv must be <= 8             */
  int32_t head_dim;     /* d: 64 or 128                                     */
  int32_t block_size;   /* must be 64                                       */
  int32_t max_blocks;   /* NB_max >= 1: K/V hold NB_max * 64 rows per head;
                           one head's K (or V) slice must fit in 2 GiB       */
  int32_t dtype;        /* attn_dtype                                       */
  float scale;          /* logit scale, normally 1 / sqrt(d)                */
} attn_dims;

/*
 * Split-KV streaming decode attention (dense).
 * Defines: streaming tile-wise accumulation of the attention output over KV
 * blocks with an exposed running state -- "ART (Attention Run-time
 * Termination)" summary, §2.1; per-split states that merge exactly --
 * "Pulsar Attention" summary, Phase 2.
 *
 * For each (b, h) the block range [min(block_begin, e), e), with
 * e = nb(b) if block_end < 0 else min(block_end, nb(b)), is cut into
 * num_splits contiguous parts: part s holds n_s = floor((s+1) n / S) -
 * floor(s n / S) blocks starting at floor(s n / S) (n = blocks in range).
 * Writes the state of every part:
 *   m, l  float [B, Hq, S];  o  float [B, Hq, S, d]   (empty part: -inf, 0, 0)
 * Merging the parts with attn_merge_states gives attention over the range.
 * Requires block_begin >= 0, num_splits >= 1.
 */
int attn_decode_dense(const attn_dims* dims, const void* q, const void* k, const void* v,
                      const int32_t* seq_lens, int32_t block_begin, int32_t block_end,
                      int32_t num_splits, float* m, float* l, float* o, void* stream);

/*
 * Exact online-softmax merge of partial states.
 * Defines: "Pulsar Attention" summary, Phase 2 (per-shard attention results
 * combined by the online softmax merge): M = max_r m_r over non-empty
 * states, w_r = l_r exp(m_r - M), out = sum_r w_r o_r / sum_r w_r.
 *   m, l    float [rows, S];  o  float [rows, S, head_dim]
 *   out     float [rows, head_dim]   (all states empty: zeros)
 *   m_out, l_out  float [rows] or NULL: the merged state (M, sum_r w_r);
 *                 (-inf, 0) when every state is empty.
 * A state with l_r = 0 is empty: its m_r and o_r never reach the result.
 * Requires rows >= 0, S >= 1, head_dim in {64, 128}.
 */
int attn_merge_states(int32_t rows, int32_t num_splits, int32_t head_dim, const float* m,
                      const float* l, const float* o, float* out, float* m_out, float* l_out,
                      void* stream);

/*
 * Block centroids: the mean key of every 64-token block.
 * Defines: "Squeezed Attention" blog (jaehun.me), Q1 and Q2 step 1 -- one
 * centroid represents a group of keys; here the group is a block.
 *   centroids  float [B, Hkv, max_blocks, d]; block j < nb(b) holds the mean
 *              of its valid keys (a partial last block averages its L_b - 64 j
 *              tokens); blocks j >= nb(b) are written as zeros.
 */
int attn_build_centroids(const attn_dims* dims, const void* k, const int32_t* seq_lens,
                         float* centroids, void* stream);

/*
 * Incremental centroid refresh after tokens were appended to the cache.
 * Defines: "Squeezed Attention" blog, Q2 step 1 (the centroids stand for the
 * current keys) -- after the call, centroids equal what attn_build_centroids
 * would write for seq_lens, for every block of the refreshed range.
 *   prev_lens  int32 [B] or NULL: each row's length when its centroids were
 *              last built.  Refreshed blocks: [min(prev_len, L) / 64,
 *              max(nb, the previous block count)) -- the block that held the
 *              shorter end onwards; blocks past the new end are zeroed.  NULL refreshes
 *              only the last block of each row (one token appended).  Blocks
 *              outside the range are neither read nor written.
 *   span_hint  >= 1: expected blocks per row, sizes the launch (any span is
 *              handled; a small hint only means fewer waves per row).
 *   centroids  float [B, Hkv, max_blocks, d], updated in place.
 */
int attn_update_centroids(const attn_dims* dims, const void* k, const int32_t* seq_lens,
                          const int32_t* prev_lens, int32_t span_hint, float* centroids, void* stream);

/*
 * Query-versus-centroid block scores, one per KV head.
 * Defines: "Squeezed Attention" blog, Q1 and Q2 step 2 (compare the query
 * with the centroids to decide which keys to load); one score per GQA group
 * with no softmax -- "SparDA" summary, §2 (compact Forecast indexer).
 *   scores  float [B, Hkv, max_blocks]:
 *           scores[b,g,j] = scale * <sum_{h in group g} q[b,h], centroids[b,g,j]>
 *           for j < nb(b), -inf for j >= nb(b).
 */
int attn_score_centroids(const attn_dims* dims, const void* q, const float* centroids,
                         const int32_t* seq_lens, float* scores, void* stream);

/*
 * Top-k block choice with forced sink and recent blocks.
 * Defines: "Squeezed Attention" blog, Q1 / Q2 step 2 (keep the best-matching
 * groups); block 0 always kept -- "ART" summary §2.4 (attention sink) and
 * the 64-token sink prefix of the "Pulsar Attention" summary, Phase 1.
 * Per (b, g): F = [0, n_sink_blocks) u [nb - n_recent_blocks, nb) clipped to
 * [0, nb); the other blocks are candidates, ranked by descending score with
 * the lower index first among equal scores; the best min(k, #candidates)
 * are added to F.
 *   scores     float [B, Hkv, max_blocks]; may be NULL when k == 0.
 *   block_idx  int32 [B, Hkv, max_sel]: the chosen blocks ascending, then -1.
 *   n_sel      int32 [B, Hkv]: how many were chosen.
 * Requires k, n_sink_blocks, n_recent_blocks >= 0 and
 * max_sel >= min(max_blocks, n_sink_blocks + n_recent_blocks + k).
 */
int attn_select_topk(const attn_dims* dims, const float* scores, const int32_t* seq_lens,
                     int32_t k, int32_t n_sink_blocks, int32_t n_recent_blocks, int32_t max_sel,
                     int32_t* block_idx, int32_t* n_sel, void* stream);

/*
 * Super-block centroids for two-level selection.
 * Defines: "Squeezed Attention" blog, Q2 step 4 (optional hierarchical
 * clustering: a coarse level of groups above the fine one) -- here a coarse
 * group is `group` consecutive blocks and its centroid the mean of its valid
 * keys, computed from the block centroids weighted by their token counts.
 *   centroids        float [B, Hkv, max_blocks, d] (attn_build_centroids).
 *   super_centroids  float [B, Hkv, ceil(max_blocks / group), d] out; super-
 *                    blocks past the sequence's end are zeros.
 * Requires group >= 1.
 */
int attn_build_super_centroids(const attn_dims* dims, const float* centroids, const int32_t* seq_lens,
                               int32_t group, float* super_centroids, void* stream);

/*
 * Two-level block selection.
 * Defines: "Squeezed Attention" blog, Q2 step 4 and Q1 (search the coarse
 * groups first, then the fine groups inside the relevant ones; the search
 * cost falls from linear towards logarithmic in the context length), with
 * the one-level rules of attn_select_topk: forced sink [0, n_sink) and
 * window [nb - n_recent, nb) blocks, scores sigma = scale * <sum of the GQA
 * group's queries, centroid>, float32 ranking with the lower index first
 * among equal scores.  Per (b, g): the super-blocks holding a non-forced
 * block are ranked on their coarse score and the best k_coarse opened; the
 * non-forced blocks inside them are ranked on their fine score and the best
 * k taken.  Only the opened super-blocks' fine centroids are read.
 *   q                [B, Hq, d] (the scoring query; any query-shaped vector).
 *   block_idx, n_sel as attn_select_topk (ascending, -1 padded).
 * Requires group >= 1, k_coarse >= 0, k >= 0, max_sel >= min(n_sink +
 * n_recent + k, max_blocks); ceil(max_blocks / group) <= 4096 and
 * min(k_coarse, ceil(max_blocks / group)) * group <= 8192 (else
 * ATTN_ERR_UNSUPPORTED).
 */
int attn_select_two_level(const attn_dims* dims, const void* q, const float* centroids,
                          const float* super_centroids, const int32_t* seq_lens, int32_t group,
                          int32_t k_coarse, int32_t k, int32_t n_sink_blocks, int32_t n_recent_blocks,
                          int32_t max_sel, int32_t* block_idx, int32_t* n_sel, void* stream);

/*
 * Split-KV decode attention restricted to listed blocks.
 * Defines: attention computed over the keys of the selected groups only --
 * "Squeezed Attention" blog, Q2 step 3 ("Sparse FlashAttention").
 *   block_idx  int32 [B, Hkv, max_sel], n_sel int32 [B, Hkv]: per (b, g) a
 *              list of n_sel <= max_sel distinct blocks < nb(b) (attn_select_topk
 *              output; precondition).  Blocks not listed are never read.
 * The list positions [0, n_sel) are cut into num_splits parts as in
 * attn_decode_dense; m, l [B, Hq, S], o [B, Hq, S, d] as there.
 */
int attn_decode_sparse(const attn_dims* dims, const void* q, const void* k, const void* v,
                       const int32_t* seq_lens, const int32_t* block_idx, const int32_t* n_sel,
                       int32_t max_sel, int32_t num_splits, float* m, float* l, float* o,
                       void* stream);

/*
 * A paged KV cache.  Every (block, kv head) run of 64 tokens is contiguous in
 * a pool shared by the batch rows; a block table maps each row's logical
 * blocks to pool blocks (rows may share pool blocks, e.g. a common prefix).
 * The pages organise the cache in 64-token blocks ("ART" summary, §2.1) and
 * move whole blocks ("SparDA" summary, offloaded KV blocks); the layout is
 * this library's.
 *   k_pool, v_pool  [pool_blocks, Hkv, 64, d] in the dims' dtype (v_pool may
 *                   be NULL where only K is read).
 *   block_table     int32 [B, table_stride], device memory: entry j of row b
 *                   is the pool block of logical block j, for j < nb(b)
 *                   (precondition: in [0, pool_blocks); entries are clamped).
 *   table_stride    >= max_blocks.
 * The paged entry points compute exactly what their contiguous namesakes
 * compute on the cache the table describes; dims.max_blocks is the logical
 * block capacity of a row.  Invalid descriptors give ATTN_ERR_INVALID_ARG.
 */
typedef struct {
  const void* k_pool;
  const void* v_pool;
  int64_t pool_blocks;
  const int32_t* block_table;
  int32_t table_stride;
} attn_paged_kv;

int attn_decode_dense_paged(const attn_dims* dims, const void* q, const attn_paged_kv* kv, const int32_t* seq_lens,
                            int32_t block_begin, int32_t block_end, int32_t num_splits, float* m, float* l,
                            float* o, void* stream);
int attn_decode_sparse_paged(const attn_dims* dims, const void* q, const attn_paged_kv* kv,
                             const int32_t* seq_lens, const int32_t* block_idx, const int32_t* n_sel,
                             int32_t max_sel, int32_t num_splits, float* m, float* l, float* o, void* stream);
int attn_build_centroids_paged(const attn_dims* dims, const attn_paged_kv* kv, const int32_t* seq_lens,
                               float* centroids, void* stream);
int attn_update_centroids_paged(const attn_dims* dims, const attn_paged_kv* kv, const int32_t* seq_lens,
                                const int32_t* prev_lens, int32_t span_hint, float* centroids, void* stream);
int attn_decode_art_paged(const attn_dims* dims, const void* q, const attn_paged_kv* kv, const int32_t* seq_lens,
                          const int32_t* order, float tau, float phi, int32_t patience, int32_t probe_dim,
                          float* out, int32_t* stop_pos, int32_t* blocks_fetched, void* stream);

/*
 * Decode attention with ART run-time termination.
 * Defines: "ART (Attention Run-time Termination)" summary, §2.1-2.4.  Blocks
 * are folded into the running state in a visit order; after folding the
 * block at visit position t >= 1 the probe x_t = the first probe_dim channels
 * of the normalised partial output is compared with x_{t-1}:
 *   d_scale = | ||x_t|| - ||x_{t-1}|| |,  d_dir = 1 - cos(x_t, x_{t-1})
 *   (not stable if a norm is 0); stable iff d_scale < tau and d_dir < phi.
 * The stop T is the first t with p = patience consecutive stable steps; with
 * no stop T = nb - 1.  Decisions are per query head; a KV head's blocks are
 * fetched until every query head of its group has stopped.
 *   order           int32 [B, Hkv, max_blocks] or NULL.  Row (b,g) starts with
 *                   block 0 and its first nb(b) entries are a permutation of
 *                   [0, nb(b)) (precondition).  NULL: (0, nb-1, nb-2, ..., 1).
 *   out             float [B, Hq, d]: the partial output after position T
 *                   (zeros when nb = 0).
 *   stop_pos        int32 [B, Hq]: T (-1 when nb = 0).
 *   blocks_fetched  int32 [B, Hkv] or NULL: blocks read from memory per KV head
 *                   (>= max over the group of T + 1; speculative read-ahead
 *                   beyond the stop is counted).
 * probe_dim = 0 turns the detector off (dense result, T = nb - 1).
 * Requires patience >= 1, probe_dim >= 0, tau, phi not NaN (else
 * ATTN_ERR_INVALID_ARG); probe_dim > min(d, 16) is ATTN_ERR_UNSUPPORTED.
 */
int attn_decode_art(const attn_dims* dims, const void* q, const void* k, const void* v,
                    const int32_t* seq_lens, const int32_t* order, float tau, float phi,
                    int32_t patience, int32_t probe_dim, float* out, int32_t* stop_pos,
                    int32_t* blocks_fetched, void* stream);

/*
 * attn_decode_art with a workspace, for batches too small to fill the chip.
 * Defines: as attn_decode_art ("ART (Attention Run-time Termination)"
 * summary, §2.1-2.4); same arguments, results and errors.  With
 * B * Hkv <= 128 and at least 2 CUs per (b, kv head) on the device of
 * `stream`, each (b, kv head) is streamed by up to 4 workgroups on different
 * CUs that hand block states to folding waves through the workspace, and as
 * CUs free up further workgroups join the (b, kv heads) still running;
 * read-ahead past the stop is then at most max(64, T + 1) blocks, and at
 * most 128, per KV head.  Otherwise it runs as attn_decode_art and the
 * workspace is not touched.
 *   workspace        device memory of at least attn_art_workspace_bytes(dims)
 *                    bytes (may be NULL when that is 0), used only by this
 *                    call until it completes on `stream`; no initial contents.
 * ATTN_ERR_INVALID_ARG for a NULL workspace that is needed,
 * ATTN_ERR_WORKSPACE when workspace_bytes is too small.
 */
int attn_decode_art_ws(const attn_dims* dims, const void* q, const void* k, const void* v,
                       const int32_t* seq_lens, const int32_t* order, float tau, float phi,
                       int32_t patience, int32_t probe_dim, void* workspace, size_t workspace_bytes,
                       float* out, int32_t* stop_pos, int32_t* blocks_fetched, void* stream);

/*
 * attn_decode_art_list and attn_decode_art_paged across workgroups.
 * Defines: as attn_decode_art_list and attn_decode_art_paged ("ART (Attention
 * Run-time Termination)" summary, §2.1-2.4); same arguments, results and
 * errors, plus the workspace, its size and its use as in attn_decode_art_ws.
 */
int attn_decode_art_list_ws(const attn_dims* dims, const void* q, const void* k, const void* v,
                            const int32_t* seq_lens, const int32_t* block_list, const int32_t* n_list,
                            int32_t max_list, float tau, float phi, int32_t patience, int32_t probe_dim,
                            void* workspace, size_t workspace_bytes, float* out, int32_t* stop_pos,
                            int32_t* blocks_fetched, void* stream);
int attn_decode_art_paged_ws(const attn_dims* dims, const void* q, const attn_paged_kv* kv,
                             const int32_t* seq_lens, const int32_t* order, float tau, float phi,
                             int32_t patience, int32_t probe_dim, void* workspace, size_t workspace_bytes,
                             float* out, int32_t* stop_pos, int32_t* blocks_fetched, void* stream);

/* Workspace bytes attn_decode_art_ws needs for these dims: 0 when
 * B * Hkv > 128 or on invalid dims, else 261 KiB (G <= 4) or 521 KiB
 * (G > 4) per (b, kv head) at d = 128, about half that at d = 64. */
size_t attn_art_workspace_bytes(const attn_dims* dims);

/*
 * ART over a listed subset of blocks.
 * Defines: "ART (Attention Run-time Termination)" summary, §2.4 -- the stop
 * rule is a control layer that composes with KV selection: the visit order
 * is the list, and attention is over the listed blocks folded so far.
 *   block_list  int32 [B, Hkv, max_list], n_list int32 [B, Hkv]: per (b, g)
 *               the first n = clamp(n_list, 0, min(max_list, nb(b))) entries
 *               are visited in list order; they must be distinct blocks
 *               < nb(b), block 0 first when the sink is kept (precondition;
 *               entries are clamped into [0, nb)).  An attn_select_topk result
 *               (ascending, sink first) or a prefix of attn_order_blocks
 *               output with max_list = max_blocks both qualify.
 * Stop rule, out, stop_pos and blocks_fetched as in attn_decode_art with nb
 * replaced by n: with no stop T = n - 1; n = 0 gives zeros and T = -1.
 */
int attn_decode_art_list(const attn_dims* dims, const void* q, const void* k, const void* v,
                         const int32_t* seq_lens, const int32_t* block_list, const int32_t* n_list,
                         int32_t max_list, float tau, float phi, int32_t patience, int32_t probe_dim,
                         float* out, int32_t* stop_pos, int32_t* blocks_fetched, void* stream);

/*
 * Importance-first visit order from block scores.
 * Defines: "ART (Attention Run-time Termination)" summary, §2.4 (the visit
 * order may put the most important blocks first; the first block is always
 * evaluated first), with importance = the centroid score of
 * attn_score_centroids ("Squeezed Attention" blog, Q2 step 2).
 *   scores  float [B, Hkv, max_blocks] (finite for blocks < nb(b)).
 *   order   int32 [B, Hkv, max_blocks] out: 0, then blocks 1 .. nb-1 by
 *           descending float32 score, lower index first among equal scores
 *           (-0 equals +0); -1 from position nb on.  Usable as the order of
 *           attn_decode_art.
 * Supports max_blocks - 1 <= 16384 (1M tokens at 64 per block), else
 * ATTN_ERR_UNSUPPORTED.
 */
int attn_order_blocks(const attn_dims* dims, const float* scores, const int32_t* seq_lens,
                      int32_t* order, void* stream);

/*
 * One decode step of a layer stack under a per-layer hard route.
 * Defines: "Flux Attention" summary, §2 -- every layer runs either full
 * attention (FA) or sparse attention (SA), fixed once at prefill; SA layers
 * skip loading the historical KV.  FA layers are computed as n_shards
 * context shards of splits_per_shard splits each and merged twice (inner
 * splits -> shard states -> output), the one-device form of the
 * "Pulsar Attention" Phase 2 merge.  SA layers attend to the listed blocks
 * (normally the sink and recent window from attn_select_topk with k = 0).
 *   route_mask      host uint8 [n_layers]: 1 = FA, 0 = SA.
 *   q, k, v         host arrays [n_layers] of device pointers (shapes above).
 *   sa_block_idx    int32 [B, Hkv, sa_max_sel], sa_n_sel int32 [B, Hkv]: the
 *                   block list shared by all SA layers (may be NULL if no layer
 *                   is SA).
 *   workspace       device memory of at least attn_routed_workspace_bytes().
 *   out             host array [n_layers] of device pointers to float [B, Hq, d].
 * The layers are queued in order on `stream`.
 */
int attn_decode_routed(const attn_dims* dims, int32_t n_layers, const uint8_t* route_mask,
                       const void* const* q, const void* const* k, const void* const* v,
                       const int32_t* seq_lens, int32_t n_shards, int32_t splits_per_shard,
                       const int32_t* sa_block_idx, const int32_t* sa_n_sel, int32_t sa_max_sel,
                       int32_t sa_splits, void* workspace, size_t workspace_bytes,
                       float* const* out, void* stream);

/* Workspace bytes attn_decode_routed needs for these dims and split counts
 * (0 on invalid arguments). */
size_t attn_routed_workspace_bytes(const attn_dims* dims, int32_t n_shards,
                                   int32_t splits_per_shard, int32_t sa_splits);

/*
 * attn_decode_routed for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, arguments, results and errors, without
 * the workspace.  The split and shard states live in a scratch array of
 * ATTN_ROUTED_STATIC_BYTES that the library holds on every device it runs on
 * until the process ends; the call allocates nothing.
 * ATTN_ERR_WORKSPACE when attn_routed_workspace_bytes() for the same
 * arguments exceeds ATTN_ROUTED_STATIC_BYTES (nothing is queued).
 * Every call on one device uses that device's one array, and the array keeps
 * the last call's contents (no call reads a state it has not written): calls
 * that overlap on one device -- other streams, other threads -- race.
 * The first call on a device takes the array's address with that device made
 * current for the duration (ATTN_ERR_HIP if that fails).
 */
#define ATTN_ROUTED_STATIC_BYTES (8u << 20)
int attn_decode_routed_static(const attn_dims* dims, int32_t n_layers, const uint8_t* route_mask,
                              const void* const* q, const void* const* k, const void* const* v,
                              const int32_t* seq_lens, int32_t n_shards, int32_t splits_per_shard,
                              const int32_t* sa_block_idx, const int32_t* sa_n_sel, int32_t sa_max_sel,
                              int32_t sa_splits, float* const* out, void* stream);

/* Static description of a status code (never NULL). */
const char* attn_status_string(int status);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_KV_H */
