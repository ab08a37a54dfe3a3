/* A C99 caller of the library's host-side entry points: status strings,
 * workspace sizes, argument errors (returned before anything touches a
 * device; the pointers below are never dereferenced) and the host block
 * manager with its prefix cache.  Prints one line per check and "all ok". */
#include <stdio.h>
#include <string.h>

#include "pagedkv.h"

static int failures = 0;

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      printf("FAILED line %d: %s\n", __LINE__, #cond);           \
      ++failures;                                                \
    }                                                            \
  } while (0)

int main(void) {
  void* fake = (void*)0x1000;                  /* never dereferenced */

  CHECK(strcmp(pkv_status_string(PKV_OK), "ok") == 0);
  CHECK(paged_attention_decode_workspace_bytes(2, 4, 128, 128, 16, 0) == 0);   /* 1 partition */
  /* 2 sequences x 4 heads x 2 partitions (4096 tokens / 2048) x (128 + 2) floats */
  CHECK(paged_attention_decode_workspace_bytes(2, 4, 128, 256, 16, 0) == 2 * 4 * 2 * 130 * 4);

  /* argument errors */
  CHECK(reshape_and_cache(NULL, fake, fake, fake, (const int64_t*)fake, 4, 2, 64, 16, 8,
                          PKV_F16, PKV_F16, 1.f, 1.f, NULL) == PKV_ERR_NULL);
  CHECK(reshape_and_cache(fake, fake, fake, fake, (const int64_t*)fake, 4, 2, 64, 12, 8,
                          PKV_F16, PKV_F16, 1.f, 1.f, NULL) == PKV_ERR_UNSUPPORTED);
  CHECK(paged_attention_decode(fake, fake, fake, fake, (const int32_t*)fake,
                               (const int32_t*)fake, 2, 6, 4, 128, 16, 4, 16, 0.1f, PKV_F16,
                               PKV_F16, 1.f, 1.f, 0, NULL, 0, NULL) == PKV_ERR_SHAPE);
  CHECK(paged_attention_decode(fake, fake, fake, fake, (const int32_t*)fake,
                               (const int32_t*)fake, 2, 4, 2, 48, 16, 4, 16, 0.1f, PKV_F16,
                               PKV_F16, 1.f, 1.f, 0, NULL, 0, NULL) == PKV_ERR_UNSUPPORTED);
  CHECK(paged_attention_decode(fake, fake, fake, fake, (const int32_t*)fake,
                               (const int32_t*)fake, 2, 4, 2, 128, 16, 256, 16, 0.1f, PKV_F16,
                               PKV_F16, 1.f, 1.f, 0, NULL, 0, NULL) == PKV_ERR_WORKSPACE);
  CHECK(paged_attention_decode_strided(fake, fake, fake, fake, (const int32_t*)fake,
                                       (const int32_t*)fake, 2, 4, 2, 128, 16, 4, 16, 1024,
                                       100, 0.1f, PKV_F16, PKV_F16, 1.f, 1.f, 0, NULL, 0,
                                       NULL) == PKV_ERR_SHAPE);
  CHECK(paged_attention_decode(fake, fake, fake, fake, (const int32_t*)fake,
                               (const int32_t*)fake, 0, 4, 2, 128, 16, 4, 16, 0.1f, PKV_BF16,
                               PKV_FP8_E4M3, 0.5f, 0.5f, 0, NULL, 0, NULL) == PKV_OK);

  /* host block manager: prompt, fork, copy-on-write append, tables */
  pkv_block_manager* bm = NULL;
  CHECK(pkv_bm_create(8, 4, &bm) == PKV_OK && bm != NULL);
  CHECK(pkv_bm_add_sequence(bm, 1, 6) == PKV_OK);               /* blocks 0, 1 */
  CHECK(pkv_bm_fork(bm, 1, 2) == PKV_OK);
  int64_t ids[2] = {1, 2}, slots[2], pairs[4];
  int32_t ncopy = -1, ndone = -1;
  CHECK(pkv_bm_append_tokens(bm, ids, 2, slots, pairs, &ncopy, &ndone) == PKV_OK);
  CHECK(ndone == 2 && ncopy == 1 && pairs[0] == 1 && pairs[1] == 2);  /* seq 1 copies block 1 */
  CHECK(slots[0] == 2 * 4 + 2 && slots[1] == 1 * 4 + 2);
  int32_t tables[2 * 3], lens[2];
  CHECK(pkv_bm_build_block_tables(bm, ids, 2, 3, tables, lens) == PKV_OK);
  CHECK(tables[0] == 0 && tables[1] == 2 && tables[2] == -1 && lens[0] == 7);
  CHECK(tables[3] == 0 && tables[4] == 1 && lens[1] == 7);
  CHECK(pkv_bm_num_free_blocks(bm) == 5);
  CHECK(pkv_bm_free_sequence(bm, 2) == PKV_OK && pkv_bm_free_sequence(bm, 2) == PKV_ERR_SEQUENCE);

  /* prefix cache: a freed prompt's full blocks serve the next identical prompt */
  int64_t prompt[9] = {5, 6, 7, 8, 9, 10, 11, 12, 13}, cached = -1;
  CHECK(pkv_bm_add_sequence_cached(bm, 3, prompt, 9, &cached) == PKV_OK && cached == 0);
  int32_t t3[3], nb3 = 0;
  int64_t ntok = 0;
  CHECK(pkv_bm_get_block_table(bm, 3, t3, 3, &nb3, &ntok) == PKV_OK && nb3 == 3 && ntok == 9);
  CHECK(pkv_bm_free_sequence(bm, 3) == PKV_OK && pkv_bm_num_cached_blocks(bm) == 2);
  CHECK(pkv_bm_add_sequence_cached(bm, 4, prompt, 9, &cached) == PKV_OK && cached == 8);
  int32_t t4[3], nb4 = 0;
  CHECK(pkv_bm_get_block_table(bm, 4, t4, 3, &nb4, &ntok) == PKV_OK);
  CHECK(t4[0] == t3[0] && t4[1] == t3[1]);
  CHECK(pkv_bm_add_sequence_cached(bm, 5, NULL, 3, &cached) == PKV_ERR_NULL);
  pkv_bm_destroy(bm);
  pkv_bm_destroy(NULL);

  if (failures == 0) printf("all ok\n");
  return failures == 0 ? 0 : 1;
}
