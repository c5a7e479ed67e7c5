/* A plain C99 caller of libpf: the header must compile as C (no C++ in the
 * declarations) and the host allocator must behave as documented when called
 * from C.  Host-only calls: runs without a GPU.  Prints "c abi ok" on success;
 * any mismatch prints where and exits 1. */
#include <stdio.h>
#include <stdlib.h>

#include "pf.h"

static int fails = 0;
#define EXPECT(cond)                                           \
  do {                                                         \
    if (!(cond)) {                                             \
      printf("FAIL line %d: %s\n", __LINE__, #cond);           \
      ++fails;                                                 \
    }                                                          \
  } while (0)

int main(void) {
  pf_geometry g;
  pf_pool* pool = NULL;
  int32_t bt[2 * 4], lens[2], got = 0;
  uint64_t ids[2] = {1, 2};
  int32_t new_lens[2] = {35, 17};
  int i;

  g.num_pages = 8;
  g.block_size = 16;
  g.num_layers = 2;
  g.num_kv_heads = 3;
  g.head_dim = 64;
  g.dtype = PF_F16;
  EXPECT(pf_pool_create(&g, NULL, &pool) == PF_OK && pool != NULL);
  /* page = 2 layers x 3 heads x K,V x 16 slots x 64 dims x 2 bytes */
  EXPECT(pf_page_bytes(pool) == (size_t)2 * 3 * 2 * 16 * 64 * 2);
  EXPECT(pf_pool_bytes(pool) == 8 * pf_page_bytes(pool));
  EXPECT(pf_free_pages(pool) == 8);

  /* 35 tokens take ceil(35/16) = 3 pages, 17 tokens 2; a fresh pool pops 0 first */
  EXPECT(pf_alloc_for_seqs(pool, ids, new_lens, 2, NULL) == PF_OK);
  EXPECT(pf_free_pages(pool) == 3);
  EXPECT(pf_block_tables(pool, ids, 2, 4, bt, lens) == PF_OK);
  EXPECT(bt[0] == 0 && bt[1] == 1 && bt[2] == 2 && bt[3] == -1);
  EXPECT(bt[4] == 3 && bt[5] == 4 && bt[6] == -1 && bt[7] == -1);
  EXPECT(lens[0] == 35 && lens[1] == 17);

  /* all or nothing: 4 more pages do not fit in 3, nothing changes */
  EXPECT(pf_alloc_for_seq(pool, 2, 17 + 4 * 16, &got) == PF_ERR_OOM);
  EXPECT(pf_seq_len(pool, 2, &got) == PF_OK && got == 17 && pf_free_pages(pool) == 3);
  EXPECT(pf_alloc_for_seq(pool, 2, 16, NULL) == PF_ERR_INVALID);  /* below the current length */

  /* free pushes the table back last page first: the first page ends on top */
  EXPECT(pf_free_seq(pool, 1) == PF_OK);
  EXPECT(pf_free_seq(pool, 1) == PF_ERR_UNKNOWN_SEQ);              /* double free */
  EXPECT(pf_alloc_for_seq(pool, 7, 1, &got) == PF_OK && got == 1);
  EXPECT(pf_block_tables(pool, ids + 1, 1, 4, bt, NULL) == PF_OK && bt[0] == 3 && bt[1] == 4);
  {
    uint64_t seven = 7;
    int32_t row[4];
    EXPECT(pf_block_tables(pool, &seven, 1, 4, row, NULL) == PF_OK && row[0] == 0 && row[1] == -1);
  }
  EXPECT(pf_num_seqs(pool) == 2 && pf_pool_peak_pages(pool) == 5);

  /* kernel entry points before a device pool is bound report it, launching nothing */
  EXPECT(pf_scatter_kv(pool, 0, NULL, NULL, NULL, NULL, 0, NULL, 0, 1, NULL) == PF_ERR_UNBOUND);

  for (i = 0; i < 2; ++i) EXPECT(pf_free_seq(pool, i == 0 ? 2 : 7) == PF_OK);
  EXPECT(pf_free_pages(pool) == 8 && pf_num_seqs(pool) == 0);
  pf_pool_destroy(pool);
  pf_pool_destroy(NULL);
  EXPECT(pf_free_pages(NULL) == -1);

  if (fails) return 1;
  printf("c abi ok\n");
  return 0;
}
