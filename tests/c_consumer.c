/* A C99 consumer of include/sp.h: compiled with gcc -std=c99 -Wall -Werror
 * and linked against libspattn.so by tests/test_abi.py, then run on the host.
 * It calls only the host-only entry points (no device is needed) and exits
 * non-zero on the first mismatch. */
#include <stdio.h>
#include <string.h>

#include "sp.h"

static int fails = 0;
#define CHECK(cond)                                               \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++fails;                                                    \
    }                                                             \
  } while (0)

int main(void) {
  int64_t off[4], len[4];
  int32_t sh = 0, sw = 0;
  int r;
  CHECK(sp_version() > 0);
  CHECK(sp_status_string(SP_OK) != NULL && strlen(sp_status_string(SP_OK)) > 0);
  CHECK(sp_status_string(SP_ERR_NOT_DIVISIBLE) != NULL);
  /* 52 tokens over 4 ranks: shards of 13 at 0, 13, 26, 39; 50 tokens do not divide */
  CHECK(sp_partition(52, 4, off, len) == SP_OK);
  for (r = 0; r < 4; ++r) {
    CHECK(off[r] == 13 * r);
    CHECK(len[r] == 13);
  }
  CHECK(sp_partition(50, 4, off, len) == SP_ERR_NOT_DIVISIBLE);
  CHECK(sp_partition(8, 0, NULL, NULL) == SP_ERR_INVALID_ARG);
  /* the near-square rank grid of 8 ranks over a 16 x 24 latent */
  CHECK(sp_optimal_split(8, 16, 24, &sh, &sw) == SP_OK);
  CHECK(sh == 2 && sw == 4);
  CHECK(sp_optimal_split(8, 7, 7, &sh, &sw) == SP_ERR_NOT_DIVISIBLE);
  /* argument checks happen on the host before anything touches a device */
  {
    sp_shard_strides st;
    st.rank = 0;
    st.batch = 0;
    CHECK(sp_relayout_heads(NULL, NULL, 1, 4, 1, 50, 8, 16, SP_F32, SP_TOKENS_TO_HEADS, st, st, NULL) ==
          SP_ERR_NOT_DIVISIBLE);
  }
  CHECK(sp_masked_attention_workspace_size(1, 1, 6144, 6144, 4, 128, SP_BF16, 0, 0) > 0);
  if (fails == 0) printf("c consumer ok\n");
  return fails == 0 ? 0 : 1;
}
