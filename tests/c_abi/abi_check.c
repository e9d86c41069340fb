/*
 * Plain C client of libsp24.so: includes only include/sp24.h, links the
 * library, and calls the entry points that need no device (the pattern
 * table, status strings, version) plus argument validation with fake,
 * never-dereferenced pointers.  Prints "ok" and exits 0 when every check
 * holds; prints the failing check and exits 1 otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sp24.h"

static int failures = 0;
#define CHECK(cond)                                            \
  do {                                                         \
    if (!(cond)) {                                             \
      printf("FAILED line %d: %s\n", __LINE__, #cond);         \
      ++failures;                                              \
    }                                                          \
  } while (0)

int main(void) {
  void* fake = (void*)(uintptr_t)0x1000;   /* 16-byte aligned, never used */
  void* mis = (void*)(uintptr_t)0x1008;    /* 8-byte aligned only */
  uint16_t table[90];
  unsigned key[90];
  int p, ones, r, c;

  CHECK(sp24_abi_version() == 8);
  CHECK(sp24_pattern_table(NULL) == SP24_ERR_NULL);
  CHECK(sp24_pattern_table(table) == SP24_OK);
  /* every pattern keeps two entries in each row and each column */
  for (p = 0; p < 90; ++p) {
    for (r = 0; r < 4; ++r) {
      ones = 0;
      for (c = 0; c < 4; ++c) ones += (table[p] >> (4 * r + c)) & 1;
      CHECK(ones == 2);
    }
    for (c = 0; c < 4; ++c) {
      ones = 0;
      for (r = 0; r < 4; ++r) ones += (table[p] >> (4 * r + c)) & 1;
      CHECK(ones == 2);
    }
    /* the row-major bit string, row 0 column 0 first (most significant) */
    key[p] = 0;
    for (r = 0; r < 4; ++r)
      for (c = 0; c < 4; ++c) key[p] = (key[p] << 1) | ((table[p] >> (4 * r + c)) & 1u);
    if (p > 0) CHECK(key[p] < key[p - 1]);   /* patterns in descending bit-string order */
  }
  CHECK(table[0] == 0xCC33 && table[89] == 0x33CC);
  CHECK(strcmp(sp24_status_str(SP24_OK), "ok") == 0);
  CHECK(strcmp(sp24_status_str(12345), "unknown status") == 0);

  /* validation happens on the host, before any device call */
  CHECK(sp24_mask_search(fake, 6, 8, (uint8_t*)fake, NULL) == SP24_ERR_SHAPE);
  CHECK(sp24_mask_search(mis, 8, 8, (uint8_t*)fake, NULL) == SP24_ERR_ALIGN);
  CHECK(sp24_mask_search(NULL, 0, 8, NULL, NULL) == SP24_OK);
  CHECK(sp24_compress(fake, NULL, 16, 16, fake, (uint16_t*)fake, NULL, NULL, NULL) == SP24_ERR_NULL);
  CHECK(sp24_spmm_fwd(fake, fake, (uint16_t*)fake, 8, 16, 20, fake, NULL) == SP24_ERR_SHAPE);
  CHECK(sp24_spmm_bwd_input(fake, fake, (uint16_t*)fake, -1, 16, 16, fake, NULL) == SP24_ERR_SHAPE);
  CHECK(sp24_search_compress_batch(NULL, 1, NULL) == SP24_ERR_NULL);
  CHECK(sp24_flip_count((uint8_t*)fake, (uint8_t*)fake, -1, (uint64_t*)fake, NULL) == SP24_ERR_SHAPE);
  CHECK(sp24_weight_grad(fake, fake, fake, NULL, 0.5f, 8, 16, 16, (float*)fake, NULL) == SP24_ERR_NULL);
  CHECK(sp24_geglu_fwd(fake, 4, 24, 16, fake, NULL) == SP24_ERR_SHAPE);
  CHECK(sp24_geglu_bwd(fake, fake, 4, 16, 8, mis, NULL) == SP24_ERR_ALIGN);
  CHECK(sp24_spmm_fwd_geglu(fake, fake, (uint16_t*)fake, 8, 48, 64, NULL, fake, NULL) == SP24_ERR_SHAPE);
  CHECK(sp24_mvue(fake, (const float*)fake, 4, 24, fake, (uint16_t*)fake, NULL) == SP24_ERR_SHAPE);
  {
    sp24_sc_job job;
    memset(&job, 0, sizeof(job));
    job.W = fake;
    job.R = 16;
    job.C = 16;
    job.vals_row = fake;
    job.meta_row = (uint16_t*)fake;
    job.idx_prev = (const uint8_t*)fake;   /* without a counter */
    CHECK(sp24_search_compress_batch(&job, 1, NULL) == SP24_ERR_NULL);
    CHECK(sp24_search_compress_batch(&job, 0, NULL) == SP24_ERR_SHAPE);
  }
  {
    sp24_gemm g[2];
    memset(g, 0, sizeof(g));
    g[0].A = fake;
    g[0].vals = fake;
    g[0].meta = (const uint16_t*)fake;
    g[0].out = fake;
    g[0].T = 300;
    g[0].N = 256;
    g[0].K = 1600;
    g[1] = g[0];
    g[1].K = 20;   /* not a multiple of 16 */
    CHECK(sp24_spmm_group(g, 2, fake, NULL) == SP24_ERR_SHAPE);
    CHECK(sp24_spmm_group(g, 1, NULL, NULL) == SP24_ERR_NULL);
    CHECK(sp24_spmm_group(g, SP24_MAX_GROUP + 1, fake, NULL) == SP24_ERR_SHAPE);
    CHECK(sp24_spmm_group_noalloc(g, SP24_MAX_GROUP + 1, NULL) == SP24_ERR_SHAPE);
    CHECK(sp24_spmm_group_noalloc(g, 2, NULL) == SP24_ERR_SHAPE);
    CHECK(sp24_spmm_group_noalloc(NULL, 1, NULL) == SP24_ERR_NULL);
    CHECK(SP24_GROUP_WORKSPACE_BYTES >= 64);
  }
  if (failures == 0) printf("ok\n");
  return failures == 0 ? 0 : 1;
}
