/* The C ABI used from plain C99: include/pa.h compiles as C and libpa.so
 * links into a C program.  Only host-side calls run here (no GPU needed):
 * the block-layout helper, the status strings and one block-manager
 * lifecycle (admit, fork, append with copy-on-write, release).  Exit status 0
 * when every check holds, else the number of the first failed check. */
#include <stdio.h>
#include <string.h>

#include "pa.h"

#define CHECK(n, cond)                              \
  do {                                              \
    if (!(cond)) {                                  \
      fprintf(stderr, "check %d failed\n", (n));    \
      return (n);                                   \
    }                                               \
  } while (0)

int main(void) {
  int64_t blocks = -1, unused = -1;
  CHECK(1, pa_abi_version() == 2);
  CHECK(2, pa_block_layout(10, 4, &blocks, &unused) == PA_OK && blocks == 3 && unused == 2);
  CHECK(3, pa_block_layout(-1, 4, &blocks, &unused) == PA_ERR_INVALID_ARG);
  CHECK(4, strcmp(pa_status_string(PA_OK), "ok") == 0);

  /* 8 blocks of 4 tokens, no watermark, no host pool */
  pa_block_manager* bm = NULL;
  CHECK(5, pa_bm_create(8, 4, 0, 0, &bm) == PA_OK && bm != NULL);
  CHECK(6, pa_bm_admit(bm, 0, 6) == PA_OK);           /* 2 blocks, the last half full */
  CHECK(7, pa_bm_fork(bm, 0, 1) == PA_OK);            /* child shares both blocks */
  int64_t seqs[2] = {0, 1}, slots[2], pairs[4];
  int32_t ncow = -1;
  CHECK(8, pa_bm_append_slots(bm, seqs, 2, slots, pairs, &ncow) == PA_OK);
  /* the first writer into the shared, partly filled block copies it */
  CHECK(9, ncow == 1 && pairs[0] != pairs[1]);
  int64_t free_blocks = -1, free_host = -1, nseq = -1;
  CHECK(10, pa_bm_stats(bm, &free_blocks, &free_host, &nseq) == PA_OK);
  CHECK(11, free_blocks == 5 && nseq == 2);
  CHECK(12, pa_bm_release(bm, 0) == PA_OK && pa_bm_release(bm, 1) == PA_OK);
  CHECK(13, pa_bm_stats(bm, &free_blocks, &free_host, &nseq) == PA_OK && free_blocks == 8);
  CHECK(14, pa_bm_destroy(bm) == PA_OK);
  return 0;
}
