/* A C client of the library: argument validation of every entry point and
 * the host block manager (no device memory is touched).  Prints "ok" and
 * exits 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pagedattn.h"
#include "pagedattn_blocks.h"
#include "pagedattn_bench.h"

static int failures = 0;

#define EXPECT(cond)                                               \
  do {                                                             \
    if (!(cond)) {                                                 \
      fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                  \
    }                                                              \
  } while (0)

int main(void) {
  void* fake = (void*)0x1000; /* never dereferenced: every call below fails validation first */
  int32_t* ifake = (int32_t*)0x1000;

  EXPECT(strcmp(paged_attn_status_string(PA_OK), "ok") == 0);
  for (int c = PA_ERR_SCRATCH; c < 0; ++c) EXPECT(strcmp(paged_attn_status_string(c), "unknown status") != 0);

  /* kv_append */
  EXPECT(kv_append(fake, fake, fake, fake, ifake, 4, 8, 96, 16, 10, PA_BF16, NULL) == PA_ERR_HEAD_DIM);
  EXPECT(kv_append(fake, fake, fake, fake, ifake, 4, 8, 128, 24, 10, PA_BF16, NULL) == PA_ERR_BLOCK_SIZE);
  EXPECT(kv_append(fake, fake, (char*)fake + 2, fake, ifake, 4, 8, 128, 16, 10, PA_BF16, NULL) == PA_ERR_ALIGN);
  EXPECT(kv_append(NULL, NULL, NULL, NULL, NULL, 0, 8, 128, 16, 10, PA_BF16, NULL) == PA_OK);

  /* decode */
  EXPECT(paged_attn_decode(fake, fake, fake, fake, ifake, 4, ifake, 2, 30, 8, 128, 16, 100, 64, 0.1f, 0, NULL,
                           fake, (size_t)1 << 40, PA_BF16, NULL) == PA_ERR_HEADS);
  EXPECT(paged_attn_decode(fake, fake, fake, fake, ifake, 4, ifake, 2, 32, 8, 128, 16, 100, 4096, 0.1f, 0, NULL,
                           NULL, 0, PA_BF16, NULL) == PA_ERR_WORKSPACE);
  pa_score_mods bad = {-1, 0.f, NULL, NULL, NULL};
  EXPECT(paged_attn_decode(fake, fake, fake, fake, ifake, 4, ifake, 2, 32, 8, 128, 16, 100, 64, 0.1f, 0, &bad,
                           fake, (size_t)1 << 40, PA_BF16, NULL) == PA_ERR_MODS);
  EXPECT(paged_attn_decode_noalloc(fake, fake, fake, fake, ifake, 2048, ifake, 4000, 64, 8, 128, 16, 100, 32768,
                                   0.1f, 0, NULL, PA_BF16, NULL) == PA_ERR_SCRATCH);
  EXPECT(paged_attn_decode_workspace_size(64, 64, 8, 128, 32768, 0) <= PA_DECODE_SCRATCH_BYTES);
  EXPECT(paged_attn_decode_workspace_size(8, 32, 8, 128, 256, 0) == 0);   /* short rows: unsplit */
  EXPECT(paged_attn_decode_split_tokens(64, 8, 32768, 512) == 512);

  /* prefill */
  EXPECT(paged_attn_prefill(fake, fake, ifake, fake, fake, ifake, 4, ifake, 2, 16, 32, 8, 128, 16, 100, 0.1f, 2,
                            NULL, PA_BF16, NULL) == PA_ERR_FLAG);

  /* two-phase decode */
  pa_prefix_level lv = {ifake, NULL, ifake, 0, 4, 512};
  EXPECT(paged_attn_decode_cascade(fake, fake, fake, fake, ifake, 4, ifake, 8, &lv, 1, 32, 8, 128, 16, 100, 1024,
                                   0.1f, NULL, fake, (size_t)1 << 40, PA_BF16, NULL) == PA_ERR_SIZE);
  lv.num_groups = 1;
  EXPECT(paged_attn_decode_cascade_workspace_size(64, &lv, 1, 64, 8, 128, 17408) > 0);
  EXPECT(paged_attn_decode_cascade(fake, fake, fake, fake, ifake, 4, ifake, 8, &lv, 1, 32, 8, 128, 16, 100, 1024,
                                   0.1f, NULL, fake, (size_t)1 << 40, PA_F32, NULL) == PA_ERR_DTYPE);

  /* block copies and the measurement kernels */
  EXPECT(kv_copy_blocks(fake, fake, ifake, ifake, -1, 8, 128, 16, 10, PA_BF16, NULL) == PA_ERR_SIZE);
  EXPECT(pa_bench_fill(NULL, 64, 0, NULL) == PA_ERR_NULL);

  /* block manager: a prompt, two forks, copy-on-write, prefix levels */
  pa_block_manager* bm = NULL;
  EXPECT(pa_bm_create(64, 16, &bm) == PA_OK && bm != NULL);
  int32_t a, b, c, slots[64], src[4], dst[4], ncopy = -1;
  EXPECT(pa_bm_new_sequence(bm, &a) == PA_OK);
  EXPECT(pa_bm_append(bm, a, 40, slots, src, dst, 4, &ncopy) == PA_OK && ncopy == 0);
  EXPECT(pa_bm_fork(bm, a, &b) == PA_OK && pa_bm_fork(bm, a, &c) == PA_OK);
  EXPECT(pa_bm_append(bm, b, 3, slots, src, dst, 4, &ncopy) == PA_OK && ncopy == 1); /* shared 3rd block */
  int32_t seqs[3] = {a, b, c}, gs[8 * 4], ps[8 * 3], pe[8 * 3], ng[8], nl = -1;
  EXPECT(pa_bm_prefix_levels(bm, seqs, 3, 8, gs, ps, pe, ng, &nl) == PA_OK);
  /* a, b, c share the two full blocks (32 tokens); a and c also their 8-token third block, not counted */
  EXPECT(nl == 1 && ng[0] == 1 && gs[0] == 0 && gs[1] == 3 && ps[0] == 0 && pe[0] == 32);
  int64_t fr, used, waste;
  EXPECT(pa_bm_stats(bm, &fr, &used, &waste) == PA_OK && used == 4 && fr == 60);
  EXPECT(pa_bm_free_sequence(bm, b) == PA_OK && pa_bm_free_sequence(bm, b) == PA_ERR_SEQ);
  pa_bm_destroy(bm);

  /* pages of several blocks: 1, 2, 4 blocks along a sequence, 4-block pages for its fork */
  EXPECT(pa_bm_create_paged(64, 16, 3, &bm) == PA_ERR_SIZE && bm == NULL);
  EXPECT(pa_bm_create_paged(64, 16, 4, &bm) == PA_OK && bm != NULL);
  EXPECT(pa_bm_new_sequence_paged(bm, 1, 8, &a) == PA_ERR_SIZE);
  EXPECT(pa_bm_new_sequence_paged(bm, 1, 4, &a) == PA_OK);
  int32_t pslots[128];
  EXPECT(pa_bm_append(bm, a, 100, pslots, src, dst, 4, &ncopy) == PA_OK && ncopy == 0);
  int32_t pst[8], pnb[8], np = -1;
  EXPECT(pa_bm_pages(bm, a, pst, pnb, 8, &np) == PA_OK && np == 3 && pnb[0] == 1 && pnb[1] == 2 && pnb[2] == 4);
  EXPECT(pst[1] % 2 == 0 && pst[2] % 4 == 0);
  EXPECT(pa_bm_fork(bm, a, &b) == PA_OK);
  /* 100 tokens: 48 in the first two pages, 52 in the shared 4-block last page, whose 4 blocks
     all hold tokens and are copied (room for 2 pairs is too little) */
  EXPECT(pa_bm_append(bm, b, 1, pslots, src, dst, 2, &ncopy) == PA_ERR_SIZE);
  EXPECT(pa_bm_append(bm, b, 1, pslots, src, dst, 4, &ncopy) == PA_OK && ncopy == 4 && src[0] == pst[2]);
  EXPECT(pa_bm_stats(bm, &fr, &used, &waste) == PA_OK && used == 11 && fr == 53);
  pa_bm_destroy(bm);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
