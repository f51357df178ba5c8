/*
 * A plain C11 caller of liblcsa.so through include/lcsa.h: the boundary needs
 * no C++ and no torch on the caller's side. Only host-side calls run here
 * (ring metadata, the k rule, workspace sizes, validation errors), with
 * device pointers that are aligned but never dereferenced: every call below
 * returns before any device work.
 *
 * stdin: lines "k num den scale out_h out_w topk_fixed n_allowed k" of the
 * hand k table ("How FlashVSR works", section 2.2 step 3: the topk_ratio
 * rule), checked against lcsa_topk_count.
 * Exit status 0 and a last line "c consumer ok" on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lcsa.h"

#define CHECK(cond, ...)                                          \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "FAIL line %d: ", __LINE__);                \
      fprintf(stderr, __VA_ARGS__);                               \
      fprintf(stderr, " (last error: %s)\n", lcsa_last_error()); \
      return 1;                                                   \
    }                                                             \
  } while (0)

static void* fake(uintptr_t a) { return (void*)a; }

int main(void) {
  /* the 768x1408 streaming step's ring: 12 heads, d128, 6 x 11 blocks per
   * TB, 4 slots; K and V rings of 128 x D bf16 per block, pooled K float64 */
  const int32_t heads = 12, D = 128, nby = 6, nbx = 11, n_slots = 4;
  const size_t blocks = (size_t)heads * n_slots * nby * nbx;
  const size_t bytes_kv = blocks * 128 * D * 2, bytes_pool = blocks * D * 8;
  lcsa_kv_cache c;
  lcsa_status st;

  st = lcsa_kv_cache_init(&c, 1, heads, D, nby, nbx, LCSA_BF16, n_slots, fake(0x10000),
                          fake(0x20000), (double*)fake(0x30000), bytes_kv - 1, bytes_kv,
                          bytes_pool);
  CHECK(st == LCSA_ERR_CAPACITY, "undersized K ring: status %d", (int)st);
  CHECK(strlen(lcsa_last_error()) > 0, "no error text");
  st = lcsa_kv_cache_init(&c, 1, heads, D, nby, nbx, LCSA_BF16, n_slots, fake(0x10008),
                          fake(0x20000), (double*)fake(0x30000), bytes_kv, bytes_kv, bytes_pool);
  CHECK(st == LCSA_ERR_ALIGN, "misaligned K ring: status %d", (int)st);
  st = lcsa_kv_cache_init(&c, 1, heads, D, nby, nbx, LCSA_BF16, n_slots, fake(0x10000),
                          fake(0x20000), (double*)fake(0x30000), bytes_kv, bytes_kv, bytes_pool);
  CHECK(st == LCSA_OK, "init: status %d", (int)st);

  /* append 3 cached TBs, then the chunk's TB; a fifth does not fit */
  int32_t slot = -1;
  st = lcsa_kv_cache_append(&c, 3, 0, &slot);
  CHECK(st == LCSA_OK && slot == 0, "append 3: status %d slot %d", (int)st, slot);
  st = lcsa_kv_cache_append(&c, 1, 3, &slot);
  CHECK(st == LCSA_OK && slot == 3 && c.count == 4, "append 1: slot %d count %d", slot, c.count);
  st = lcsa_kv_cache_append(&c, 1, 4, &slot);
  CHECK(st == LCSA_ERR_CAPACITY, "append beyond capacity: status %d", (int)st);

  /* the k rule through the library: the 768x1408 step keeps 52 of 264 */
  lcsa_geom g = {1, heads, D, 2, 8 * nby, 8 * nbx, LCSA_BF16};
  lcsa_select_params p = {11, LCSA_BORDER_PRESERVED, 0, 1, 5, 0, 768, 1280, 768, 1280, 0};
  int32_t kmax = 0;
  st = lcsa_max_topk(&g, 3, &c, &p, &kmax);
  CHECK(st == LCSA_OK && kmax == 52, "max_topk: status %d kmax %d", (int)st, kmax);
  size_t ws = 1;
  st = lcsa_draft_workspace_size(&g, &c, &p, &ws);
  CHECK(st == LCSA_OK && ws == 0, "draft workspace at 264 candidates: %zu", ws);
  st = lcsa_attn_bwd_workspace_size(&g, &ws);
  CHECK(st == LCSA_OK && ws > 0, "backward workspace: status %d bytes %zu", (int)st, ws);

  /* evict to the 3 newest, wrap the ring, read the view back */
  st = lcsa_kv_cache_evict(&c, 3);
  CHECK(st == LCSA_OK && c.count == 3 && c.head == 1, "evict: count %d head %d", c.count, c.head);
  st = lcsa_kv_cache_append(&c, 1, 4, &slot);
  CHECK(st == LCSA_OK && slot == 0, "wrapped append: slot %d", slot);
  int32_t n = 0, slots[LCSA_MAX_SLOTS];
  int64_t tbs[LCSA_MAX_SLOTS];
  st = lcsa_kv_cache_view(&c, &n, slots, tbs);
  CHECK(st == LCSA_OK && n == 4, "view: status %d n %d", (int)st, n);
  for (int i = 0; i < 4; ++i)
    CHECK(slots[i] == (1 + i) % 4 && tbs[i] == 1 + i, "view %d: slot %d tb %lld", i, slots[i],
          (long long)tbs[i]);

  /* validation before any device work */
  st = lcsa_max_topk(NULL, 3, &c, &p, &kmax);
  CHECK(st == LCSA_ERR_NULL, "NULL geometry: status %d", (int)st);
  lcsa_select_params bad = p;
  bad.ratio_den = 0;
  int32_t k = 0;
  st = lcsa_topk_count(&bad, 10, 10, &k);
  CHECK(st == LCSA_ERR_PARAM, "zero ratio denominator: status %d", (int)st);

  /* the hand k table */
  char line[256];
  int rows = 0;
  while (fgets(line, sizeof line, stdin)) {
    int num, den, scale, oh, ow, fixed, na, want;
    if (sscanf(line, "k %d %d %d %d %d %d %d %d", &num, &den, &scale, &oh, &ow, &fixed, &na,
               &want) != 8)
      continue;
    lcsa_select_params q = {11, 0, fixed, num, den, scale, oh, ow, 768, 1280, 0};
    st = lcsa_topk_count(&q, na, na, &k);
    CHECK(st == LCSA_OK && k == want, "k table: %d allowed, ratio %d/%d, out %dx%d: k %d, want %d",
          na, num, den, oh, ow, k, want);
    ++rows;
  }
  printf("k table rows %d\n", rows);
  printf("c consumer ok\n");
  return 0;
}
