/* End-to-end use of the C ABI from plain C with the HIP C runtime: route
 * plan, dispatch and combine of a small deterministic batch, single hop and
 * node-deduplicated, checked against properties that fix the results:
 *   - counts sum to T*k and the expert offsets are their exclusive scan;
 *   - receive row r holds x[row_src[r]] bit for bit, and row_src inverts
 *     slot_of;
 *   - rows are in (expert, token) order;
 *   - with one-hot combine weights the float32 combine is the token's own
 *     row (exactly: one product by 1.0, no rounding).
 * Exit status 0 on success; prints the first failed check. */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_shuffle.h"

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #c);   \
      return 1;                                                               \
    }                                                                         \
  } while (0)
#define HIPCHECK(c) CHECK((c) == hipSuccess)

enum { T = 1000, H = 64, E = 32, K = 4, R = 8, G = 2 };

static uint16_t bf16_of_small_int(int v) {  /* exact for |v| < 256 */
  float f = (float)v;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static int run(uint32_t flags) {
  static int32_t idx[T * K], slot_of[T * K], row_src[T * K], counts[E], eoff[E + 1];
  static uint16_t x[T * H], recv[T * K * H];
  static float w[T * K], out[T * H];
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < K; ++j) {
      idx[t * K + j] = (t * 7 + j * 5) % E;          /* distinct in a row: steps of 5 mod 32 */
      w[t * K + j] = (j == t % K) ? 1.0f : 0.0f;     /* one-hot */
    }
  for (int t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h) x[t * H + h] = bf16_of_small_int((t * 3 + h) % 200 - 100);

  moe_config c;
  memset(&c, 0, sizeof c);
  c.num_tokens = T; c.hidden = H; c.num_experts = E; c.top_k = K;
  c.num_ranks = R; c.ranks_per_node = G; c.flags = flags;
  moe_plan* p = NULL;
  CHECK(moe_plan_create(&c, &p) == MOE_OK);
  void *d_idx, *d_x, *d_recv, *d_stage = NULL, *d_w, *d_out, *d_ws;
  HIPCHECK(hipMalloc(&d_idx, sizeof idx));
  HIPCHECK(hipMalloc(&d_x, sizeof x));
  HIPCHECK(hipMalloc(&d_recv, sizeof recv));
  HIPCHECK(hipMalloc(&d_w, sizeof w));
  HIPCHECK(hipMalloc(&d_out, sizeof out));
  HIPCHECK(hipMalloc(&d_ws, moe_plan_workspace_bytes(p)));
  if (moe_plan_staging_rows_max(p) > 0)
    HIPCHECK(hipMalloc(&d_stage, (size_t)moe_plan_staging_rows_max(p) * H * 2));
  HIPCHECK(hipMemcpy(d_idx, idx, sizeof idx, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(d_w, w, sizeof w, hipMemcpyHostToDevice));

  CHECK(moe_route_plan(p, (const int32_t*)d_idx, d_ws, NULL) == MOE_OK);
  CHECK(moe_dispatch(p, (const uint16_t*)d_x, (uint16_t*)d_recv, (uint16_t*)d_stage, NULL) == MOE_OK);
  CHECK(moe_combine(p, (const uint16_t*)d_recv, (const float*)d_w, d_out, MOE_OUT_F32, NULL) == MOE_OK);
  int32_t status = -1;
  CHECK(moe_plan_read(p, MOE_ITEM_STATUS, &status, sizeof status, NULL) == MOE_OK);
  CHECK(status == MOE_OK);
  CHECK(moe_plan_read(p, MOE_ITEM_COUNTS, counts, sizeof counts, NULL) == MOE_OK);
  CHECK(moe_plan_read(p, MOE_ITEM_EXPERT_OFFSETS, eoff, sizeof eoff, NULL) == MOE_OK);
  CHECK(moe_plan_read(p, MOE_ITEM_SLOT_OF, slot_of, sizeof slot_of, NULL) == MOE_OK);
  CHECK(moe_plan_read(p, MOE_ITEM_ROW_SRC, row_src, sizeof row_src, NULL) == MOE_OK);
  HIPCHECK(hipMemcpy(recv, d_recv, sizeof recv, hipMemcpyDeviceToHost));
  HIPCHECK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));

  int64_t sum = 0;
  CHECK(eoff[0] == 0);
  for (int e = 0; e < E; ++e) {
    sum += counts[e];
    CHECK(eoff[e + 1] == eoff[e] + counts[e]);
  }
  CHECK(sum == T * K && eoff[E] == T * K);
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < K; ++j) {
      const int r = slot_of[t * K + j];
      CHECK(r >= 0 && r < T * K && row_src[r] == t);
      CHECK(r >= eoff[idx[t * K + j]] && r < eoff[idx[t * K + j] + 1]);  /* in its expert's segment */
    }
  for (int r = 0; r < T * K; ++r) {
    CHECK(memcmp(&recv[(size_t)r * H], &x[(size_t)row_src[r] * H], H * 2) == 0);
    if (r > 0) {
      int e0 = 0, e1 = 0;  /* experts of rows r-1 and r */
      while (eoff[e0 + 1] <= r - 1) ++e0;
      while (eoff[e1 + 1] <= r) ++e1;
      CHECK(e1 > e0 || (e1 == e0 && row_src[r] > row_src[r - 1]));
    }
  }
  for (int t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h) {
      uint32_t u = (uint32_t)x[t * H + h] << 16;
      float v;
      memcpy(&v, &u, 4);
      CHECK(out[t * H + h] == v);
    }
  hipFree(d_idx); hipFree(d_x); hipFree(d_recv); hipFree(d_w); hipFree(d_out); hipFree(d_ws);
  if (d_stage) hipFree(d_stage);
  moe_plan_destroy(p);
  return 0;
}

int main(void) {
  if (run(0)) return 1;
  if (run(MOE_FLAG_NODE_DEDUP)) return 1;
  printf("abi_gpu ok (single hop and node-deduplicated)\n");
  return 0;
}
