/* Drives the C-ABI layer (argument checks, workspace layouts, the routed
 * layer loop, the static scratch of attn_decode_routed_static) against the
 * recording launchers of launch_stubs.cpp, under the host address and
 * undefined-behaviour sanitizers.  No GPU: nothing here reaches a kernel.
 * Prints "ok" and exits 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sparse_kv.h"

extern int stub_launches;
extern const void* stub_last_ptr[4];
extern int stub_last_S;
extern int stub_device_count;
void stub_reset(void);
int hipSetDevice(int);

static int fails = 0;
#define CHECK(cond)                                                       \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__);   \
      ++fails;                                                            \
    }                                                                     \
  } while (0)

static attn_dims dims(int B, int Hq, int Hkv, int d, int nb) {
  attn_dims x;
  memset(&x, 0, sizeof x);
  x.batch = B;
  x.num_q_heads = Hq;
  x.num_kv_heads = Hkv;
  x.head_dim = d;
  x.block_size = 64;
  x.max_blocks = nb;
  x.dtype = ATTN_BF16;
  x.scale = 0.125f;
  return x;
}

static int inside(const void* p, const char* base, size_t bytes) {
  return (const char*)p >= base && (const char*)p < base + bytes;
}

int main(void) {
  attn_dims d = dims(2, 8, 2, 128, 4);
  char* fake = (char*)malloc(64);
  float* ff = (float*)fake;
  int32_t* fi = (int32_t*)fake;

  /* every entry point: a valid call queues its launches, a bad one nothing */
  stub_reset();
  CHECK(attn_decode_dense(&d, fake, fake, fake, NULL, 0, -1, 4, ff, ff, ff, NULL) == ATTN_OK);
  CHECK(attn_decode_sparse(&d, fake, fake, fake, NULL, fi, fi, 4, 2, ff, ff, ff, NULL) == ATTN_OK);
  CHECK(attn_merge_states(16, 4, 128, ff, ff, ff, ff, NULL, NULL, NULL) == ATTN_OK);
  CHECK(attn_build_centroids(&d, fake, NULL, ff, NULL) == ATTN_OK);
  CHECK(attn_update_centroids(&d, fake, NULL, NULL, 1, ff, NULL) == ATTN_OK);
  CHECK(attn_score_centroids(&d, fake, ff, NULL, ff, NULL) == ATTN_OK);
  CHECK(attn_select_topk(&d, ff, NULL, 1, 1, 1, 3, fi, fi, NULL) == ATTN_OK);
  CHECK(attn_build_super_centroids(&d, ff, NULL, 2, ff, NULL) == ATTN_OK);
  CHECK(attn_select_two_level(&d, fake, ff, ff, NULL, 2, 1, 1, 1, 1, 3, fi, fi, NULL) == ATTN_OK);
  CHECK(attn_order_blocks(&d, ff, NULL, fi, NULL) == ATTN_OK);
  CHECK(attn_decode_art(&d, fake, fake, fake, NULL, NULL, 1e-3f, 1e-4f, 2, 8, ff, fi, fi, NULL) == ATTN_OK);
  CHECK(attn_decode_art_list(&d, fake, fake, fake, NULL, fi, fi, 4, 1e-3f, 1e-4f, 2, 8, ff, fi, NULL, NULL) ==
        ATTN_OK);
  CHECK(stub_launches == 12);
  stub_reset();
  CHECK(attn_decode_dense(&d, fake, fake, fake, NULL, 0, -1, 0, ff, ff, ff, NULL) == ATTN_ERR_INVALID_ARG);
  CHECK(attn_decode_sparse(&d, fake, fake, fake, NULL, NULL, fi, 4, 2, ff, ff, ff, NULL) == ATTN_ERR_INVALID_ARG);
  CHECK(attn_merge_states(16, 4, 96, ff, ff, ff, ff, NULL, NULL, NULL) == ATTN_ERR_UNSUPPORTED);
  CHECK(attn_select_topk(&d, ff, NULL, 2, 1, 1, 3, fi, fi, NULL) == ATTN_ERR_INVALID_ARG);
  CHECK(attn_decode_art(&d, fake, fake, fake, NULL, NULL, 1e-3f, 1e-4f, 2, 17, ff, fi, fi, NULL) ==
        ATTN_ERR_UNSUPPORTED);
  CHECK(stub_launches == 0);

  /* paged twins */
  {
    attn_paged_kv kv;
    kv.k_pool = fake;
    kv.v_pool = fake;
    kv.pool_blocks = 8;
    kv.block_table = fi;
    kv.table_stride = 4;
    stub_reset();
    CHECK(attn_decode_dense_paged(&d, fake, &kv, NULL, 0, -1, 2, ff, ff, ff, NULL) == ATTN_OK);
    CHECK(attn_decode_sparse_paged(&d, fake, &kv, NULL, fi, fi, 4, 2, ff, ff, ff, NULL) == ATTN_OK);
    CHECK(attn_build_centroids_paged(&d, &kv, NULL, ff, NULL) == ATTN_OK);
    CHECK(attn_update_centroids_paged(&d, &kv, NULL, NULL, 2, ff, NULL) == ATTN_OK);
    CHECK(attn_decode_art_paged(&d, fake, &kv, NULL, NULL, 1e-3f, 1e-4f, 2, 8, ff, fi, NULL, NULL) == ATTN_OK);
    CHECK(stub_launches == 5);
    kv.table_stride = 3;
    CHECK(attn_decode_dense_paged(&d, fake, &kv, NULL, 0, -1, 2, ff, ff, ff, NULL) == ATTN_ERR_INVALID_ARG);
  }

  /* ART workspaces: the size the library asks for is accepted, one byte less is not */
  {
    const size_t need = attn_art_workspace_bytes(&d);
    char* ws = (char*)malloc(need);
    CHECK(need > 0);
    stub_reset();
    CHECK(attn_decode_art_ws(&d, fake, fake, fake, NULL, NULL, 1e-3f, 1e-4f, 2, 8, ws, need, ff, fi, NULL, NULL) ==
          ATTN_OK);
    CHECK(attn_decode_art_list_ws(&d, fake, fake, fake, NULL, fi, fi, 4, 1e-3f, 1e-4f, 2, 8, ws, need, ff, fi, NULL,
                                  NULL) == ATTN_OK);
    CHECK(attn_decode_art_ws(&d, fake, fake, fake, NULL, NULL, 1e-3f, 1e-4f, 2, 8, ws, need - 1, ff, fi, NULL,
                             NULL) == ATTN_ERR_WORKSPACE);
    CHECK(stub_launches == 2);
    free(ws);
  }

  /* the routed stack: 2 launches per layer (decode, then both merge levels or the split
     merge), every state pointer inside the workspace; 3 per full layer when a row's
     shard-by-split states exceed one wave (9 shards x 8 splits) */
  {
    const uint8_t mask[3] = {1, 0, 1};
    const void* ptrs[3] = {fake, fake, fake};
    float* outs[3] = {ff, ff, ff};
    const size_t need = attn_routed_workspace_bytes(&d, 8, 2, 4);
    char* ws = (char*)malloc(need);
    int i;
    stub_reset();
    CHECK(attn_decode_routed(&d, 3, mask, ptrs, ptrs, ptrs, NULL, 8, 2, fi, fi, 4, 4, ws, need, outs, NULL) ==
          ATTN_OK);
    CHECK(stub_launches == 6);
    for (i = 0; i < 3; ++i) CHECK(inside(stub_last_ptr[i], ws, need));
    {
      const size_t need72 = attn_routed_workspace_bytes(&d, 9, 8, 4);
      char* ws72 = (char*)malloc(need72);
      stub_reset();
      CHECK(attn_decode_routed(&d, 3, mask, ptrs, ptrs, ptrs, NULL, 9, 8, fi, fi, 4, 4, ws72, need72, outs, NULL) ==
            ATTN_OK);
      CHECK(stub_launches == 8);
      for (i = 0; i < 3; ++i) CHECK(inside(stub_last_ptr[i], ws72, need72));
      free(ws72);
    }
    CHECK(attn_decode_routed(&d, 3, mask, ptrs, ptrs, ptrs, NULL, 8, 2, fi, fi, 4, 4, ws, need - 1, outs, NULL) ==
          ATTN_ERR_WORKSPACE);
    free(ws);

    /* the same without a workspace: one static scratch, the same on every call;
       the first call on a second device takes that device's address */
    {
      const void* first[3];
      stub_reset();
      CHECK(attn_decode_routed_static(&d, 3, mask, ptrs, ptrs, ptrs, NULL, 8, 2, fi, fi, 4, 4, outs, NULL) ==
            ATTN_OK);
      CHECK(stub_launches == 6);
      for (i = 0; i < 3; ++i) {
        first[i] = stub_last_ptr[i];
        CHECK(first[i] != NULL && ((uintptr_t)first[i] & 255) == 0);
      }
      stub_device_count = 2;
      CHECK(hipSetDevice(1) == 0);
      stub_reset();
      CHECK(attn_decode_routed_static(&d, 3, mask, ptrs, ptrs, ptrs, NULL, 8, 2, fi, fi, 4, 4, outs, NULL) ==
            ATTN_OK);
      for (i = 0; i < 3; ++i) CHECK(stub_last_ptr[i] == first[i]);
      CHECK(hipSetDevice(0) == 0);
      /* states beyond the scratch: refused before anything is queued */
      {
        attn_dims big = dims(64, 32, 8, 128, 4);
        CHECK(attn_routed_workspace_bytes(&big, 8, 4, 4) > ATTN_ROUTED_STATIC_BYTES);
        stub_reset();
        CHECK(attn_decode_routed_static(&big, 3, mask, ptrs, ptrs, ptrs, NULL, 8, 4, fi, fi, 4, 4, outs, NULL) ==
              ATTN_ERR_WORKSPACE);
        CHECK(stub_launches == 0);
      }
      CHECK(attn_decode_routed_static(&d, 3, mask, ptrs, ptrs, ptrs, NULL, 8, 2, NULL, fi, 4, 4, outs, NULL) ==
            ATTN_ERR_INVALID_ARG);
    }
  }
  free(fake);
  if (fails == 0) printf("ok\n");
  return fails != 0;
}
