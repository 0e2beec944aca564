/* Host-only use of the C ABI (include/moe_shuffle.h) from plain C: the
 * partition, plan creation and its checks, sizes and status strings.  Makes
 * no GPU call.  Exit status 0 on success; prints the first failed check. */
#include <stdio.h>
#include <string.h>

#include "moe_shuffle.h"

#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c); \
      return 1;                                                   \
    }                                                             \
  } while (0)

static moe_status make(int64_t T, int32_t H, int32_t E, int32_t k, int32_t R, int32_t G,
                       uint32_t flags, int32_t band, moe_plan** out) {
  moe_config c;
  memset(&c, 0, sizeof c);
  c.num_tokens = T;
  c.hidden = H;
  c.num_experts = E;
  c.top_k = k;
  c.num_ranks = R;
  c.ranks_per_node = G;
  c.flags = flags;
  c.band_tokens = band;
  return moe_plan_create(&c, out);
}

int main(void) {
  /* 256 experts over 7 ranks: the first 4 ranks hold 37, the rest 36. */
  int32_t lo[8];
  CHECK(moe_expert_partition(256, 7, lo) == MOE_OK);
  const int32_t want[8] = {0, 37, 74, 111, 148, 184, 220, 256};
  for (int d = 0; d < 8; ++d) CHECK(lo[d] == want[d]);
  CHECK(moe_expert_partition(2, 8, lo) == MOE_ERR_EXPERTS_LT_RANKS);

  moe_plan* p = NULL;
  CHECK(make(4096, 2048, 64, 8, 4, 4, 0, 0, &p) == MOE_OK);
  CHECK(moe_plan_recv_rows(p) == 4096 * 8);
  CHECK(moe_plan_staging_rows_max(p) == 0);
  CHECK(moe_plan_workspace_bytes(p) % 256 == 0 && moe_plan_workspace_bytes(p) > 0);
  CHECK(moe_plan_bands(p) == 1);
  CHECK(moe_plan_scale_blocks(p) == 16);
  moe_plan_destroy(p);

  CHECK(make(16384, 7168, 256, 8, 64, 8, MOE_FLAG_NODE_DEDUP, 0, &p) == MOE_OK);
  CHECK(moe_plan_staging_rows_max(p) == 16384 * 8);
  moe_plan_destroy(p);

  CHECK(make(4096, 2048, 64, 8, 4, 4, 0, 512, &p) == MOE_OK);
  CHECK(moe_plan_bands(p) == 8);
  moe_plan_destroy(p);

  p = NULL;
  CHECK(make(128, 12, 8, 2, 2, 2, 0, 0, &p) == MOE_ERR_INVALID_ARGUMENT && p == NULL);
  CHECK(make(128, 256, 8, 2, 16, 16, 0, 0, &p) == MOE_ERR_EXPERTS_LT_RANKS);
  CHECK(make(128, 256, 2048, 2, 8, 8, 0, 0, &p) == MOE_ERR_UNSUPPORTED);
  CHECK(make(128, 256, 8, 2, 2, 2, MOE_FLAG_NODE_DEDUP, 0, &p) == MOE_ERR_INVALID_ARGUMENT);
  moe_plan_destroy(NULL);

  for (int s = MOE_OK; s <= MOE_ERR_PIPELINE_STALL; ++s)
    CHECK(moe_status_str((moe_status)s) && strlen(moe_status_str((moe_status)s)) > 0);
  printf("abi_host ok\n");
  return 0;
}
