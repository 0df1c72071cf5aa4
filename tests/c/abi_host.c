/* A plain C program against include/pkv.h and libpkv.so: the pool, sequence
 * and page-table calls on a metadata-only pool (no GPU), checked against the
 * known answers of "nx_paged_kv_gate.nx source" (KAT part: ids 0, 1, 2, then
 * -1 on a pool of 3; a released id is handed out again; fork shares pages by
 * reference count).  Prints "ok" and exits 0 on success. */
#include <stdio.h>
#include <stdlib.h>

#include "pkv.h"

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      return 1;                                                      \
    }                                                                \
  } while (0)

int main(void) {
  /* block ids in order, exhaustion, reuse of a released id */
  pkv_pool *p = pkv_pool_new(3, 4, 1, 1, 4, 4, NULL, 0);
  CHECK(p != NULL);
  CHECK(pkv_alloc_block(p) == 0);
  CHECK(pkv_alloc_block(p) == 1);
  CHECK(pkv_alloc_block(p) == 2);
  CHECK(pkv_alloc_block(p) == -1);
  CHECK(pkv_unref_block(p, 1) == PKV_OK);
  CHECK(pkv_alloc_block(p) == 1);
  CHECK(pkv_unref_block(p, 7) == PKV_ERR_BAD_ARG);
  pkv_pool_free(p);

  /* sequences: 5 rows, fork, divergent appends copy the shared tail */
  p = pkv_pool_new(16, 4, 2, 2, 8, 8, NULL, 0);
  CHECK(p != NULL);
  int32_t a = pkv_seq_new(p, 64);
  CHECK(a >= 0);
  CHECK(pkv_ensure_append(p, &a, 1, 5, NULL) == PKV_OK);
  CHECK(pkv_advance(p, &a, 1, 5) == PKV_OK);
  CHECK(pkv_seq_len(p, a) == 5);
  int32_t b = pkv_seq_fork(p, a);
  CHECK(b >= 0 && b != a);
  int64_t pa[4], pb[4];
  CHECK(pkv_seq_pages(p, a, pa, 4) == 2);
  CHECK(pkv_seq_pages(p, b, pb, 4) == 2);
  CHECK(pa[0] == pb[0] && pa[1] == pb[1]);
  int32_t rc[16];
  CHECK(pkv_pool_refcounts(p, rc) == 16);
  CHECK(rc[pa[0]] == 2 && rc[pa[1]] == 2);
  int32_t both[2] = {a, b};
  CHECK(pkv_ensure_append(p, both, 2, 2, NULL) == PKV_OK);
  CHECK(pkv_advance(p, both, 2, 2) == PKV_OK);
  CHECK(pkv_seq_pages(p, a, pa, 4) == 2);
  CHECK(pkv_seq_pages(p, b, pb, 4) == 2);
  CHECK(pa[0] == pb[0]);  /* full first page stays shared */
  CHECK(pa[1] != pb[1]);  /* the partial tail was copied on append */
  CHECK(pkv_pool_refcounts(p, rc) == 16);
  CHECK(rc[pa[0]] == 2 && rc[pa[1]] == 1 && rc[pb[1]] == 1);
  /* rewind b to the fork point, errors leave the pool untouched */
  CHECK(pkv_seq_truncate(p, b, 5) == PKV_OK);
  CHECK(pkv_seq_truncate(p, b, 9) == PKV_ERR_BAD_ARG);
  CHECK(pkv_seq_len(p, b) == 5);
  /* a holds 7 rows in two 4-row pages: advancing past row 8 needs an ensure */
  CHECK(pkv_advance(p, &a, 1, 2) == PKV_ERR_SEQ);
  CHECK(pkv_seq_len(p, a) == 7);
  /* attention on a metadata-only pool is refused */
  CHECK(pkv_attn_paged_decode(p, &a, 1, 0, 4, 2, 8, NULL, 0.5f, NULL, NULL, 0,
                              NULL) == PKV_ERR_BAD_ARG);
  CHECK(pkv_seq_free(p, a) == PKV_OK);
  CHECK(pkv_seq_free(p, b) == PKV_OK);
  pkv_pool_free(p);
  printf("ok\n");
  return 0;
}
