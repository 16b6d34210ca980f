/* Calls the library from plain C through include/sparse_kv.h: status strings
 * and argument validation only (no call reaches a kernel launch, so no GPU is
 * needed).  Exits 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "sparse_kv.h"

static int fails = 0;
#define CHECK(cond)                                            \
  do {                                                         \
    if (!(cond)) {                                             \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      ++fails;                                                 \
    }                                                          \
  } while (0)

int main(void) {
  attn_dims d;
  attn_paged_kv kv;
  void* fake = (void*)0x1000;
  float* ff = (float*)0x1000;
  int32_t* fi = (int32_t*)0x1000;
  memset(&d, 0, sizeof d);
  d.batch = 2;
  d.num_q_heads = 8;
  d.num_kv_heads = 2;
  d.head_dim = 128;
  d.block_size = 64;
  d.max_blocks = 4;
  d.dtype = ATTN_BF16;
  d.scale = 0.125f;

  CHECK(strcmp(attn_status_string(ATTN_OK), "ok") == 0);
  CHECK(attn_status_string(ATTN_ERR_UNSUPPORTED)[0] != '\0');
  CHECK(attn_decode_dense(NULL, fake, fake, fake, NULL, 0, -1, 4, ff, ff, ff, NULL) == ATTN_ERR_INVALID_ARG);
  CHECK(attn_decode_dense(&d, fake, fake, fake, NULL, 0, -1, 0, ff, ff, ff, NULL) == ATTN_ERR_INVALID_ARG);
  d.head_dim = 96;
  CHECK(attn_decode_dense(&d, fake, fake, fake, NULL, 0, -1, 4, ff, ff, ff, NULL) == ATTN_ERR_UNSUPPORTED);
  d.head_dim = 128;
  CHECK(attn_merge_states(4, 0, 128, ff, ff, ff, ff, NULL, NULL, NULL) == ATTN_ERR_INVALID_ARG);
  CHECK(attn_select_topk(&d, NULL, NULL, 2, 1, 1, 4, fi, fi, NULL) == ATTN_ERR_INVALID_ARG);
  CHECK(attn_decode_art(&d, fake, fake, fake, NULL, NULL, 1e-3f, 1e-4f, 0, 8, ff, fi, NULL, NULL) ==
        ATTN_ERR_INVALID_ARG);
  CHECK(attn_select_two_level(&d, fake, ff, ff, NULL, 0, 2, 2, 1, 1, 4, fi, fi, NULL) == ATTN_ERR_INVALID_ARG);
  kv.k_pool = fake;
  kv.v_pool = fake;
  kv.pool_blocks = 0;
  kv.block_table = fi;
  kv.table_stride = 4;
  CHECK(attn_decode_dense_paged(&d, fake, &kv, NULL, 0, -1, 4, ff, ff, ff, NULL) == ATTN_ERR_INVALID_ARG);
  CHECK(attn_routed_workspace_bytes(&d, 8, 4, 32) > 0);
  CHECK(attn_routed_workspace_bytes(&d, 0, 4, 32) == 0);
  {
    const size_t art_ws = attn_art_workspace_bytes(&d);
    CHECK(art_ws > 0);
    CHECK(attn_decode_art_ws(&d, fake, fake, fake, NULL, NULL, 1e-3f, 1e-4f, 2, 8, NULL, art_ws, ff, fi, NULL,
                             NULL) == ATTN_ERR_INVALID_ARG);
    CHECK(attn_decode_art_ws(&d, fake, fake, fake, NULL, NULL, 1e-3f, 1e-4f, 2, 8, fake, art_ws - 1, ff, fi, NULL,
                             NULL) == ATTN_ERR_WORKSPACE);
  }
  d.batch = 0;
  CHECK(attn_decode_dense(&d, fake, fake, fake, NULL, 0, -1, 4, ff, ff, ff, NULL) == ATTN_OK);
  if (fails == 0) printf("ok\n");
  return fails != 0;
}
