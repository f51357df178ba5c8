// CPU-only driver for the host half of the C-ABI (lcsa_host.cpp: argument
// validation, the k rule, window bounds, the ring metadata), built with the
// address and undefined-behaviour sanitizers by tests/test_host_sanitized.py.
// It calls the extern "C" entry points the way a C caller would, and exits
// non-zero on the first check that fails. No HIP, no device.
//
// stdin: lines "k <ratio_num> <ratio_den> <scale> <out_h> <out_w> <topk_fixed>
// <n_allowed> <expected_k>", the k table of the topk_ratio rule ("How
// FlashVSR works", section 2.2 step 3).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/lcsa.h"

static int failures = 0;
#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "check failed at line %d: %s (%s)\n", __LINE__, #cond, \
                   lcsa_last_error());                                           \
      ++failures;                                                                \
    }                                                                            \
  } while (0)

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

static lcsa_status init(lcsa_kv_cache* c, int heads, int D, int nby, int nbx, int dtype, int slots,
                        size_t shrink_k = 0, size_t shrink_pool = 0) {
  const size_t blocks = (size_t)heads * slots * nby * nbx;
  const size_t kv = blocks * 128 * D * (dtype == LCSA_BF16 ? 2 : 4);
  const size_t pool = blocks * D * sizeof(double);
  return lcsa_kv_cache_init(c, 1, heads, D, nby, nbx, dtype, slots, fake(0x10000), fake(0x20000),
                            (double*)fake(0x30000), kv - shrink_k, kv, pool - shrink_pool);
}

int main() {
  // ---- ring metadata: wrap-around over many steps, capacity and order
  lcsa_kv_cache c;
  CHECK(init(&c, 12, 128, 6, 11, LCSA_BF16, 4) == LCSA_OK);
  int32_t first = -1, n = -1, slots[LCSA_MAX_SLOTS];
  int64_t tbs[LCSA_MAX_SLOTS];
  CHECK(lcsa_kv_cache_append(&c, 3, 0, &first) == LCSA_OK && first == 0);
  for (int64_t step = 3; step < 200; ++step) {
    CHECK(lcsa_kv_cache_append(&c, 1, step, &first) == LCSA_OK);
    CHECK(first == (int32_t)(step % 4));
    CHECK(lcsa_kv_cache_view(&c, &n, slots, tbs) == LCSA_OK && n == 4);
    for (int i = 0; i < n; ++i) CHECK(tbs[i] == step - 3 + i && slots[i] == (step - 3 + i) % 4);
    CHECK(lcsa_kv_cache_evict(&c, 3) == LCSA_OK);
  }
  CHECK(lcsa_kv_cache_append(&c, 2, 500, &first) == LCSA_ERR_CAPACITY);   // 3 + 2 > 4
  CHECK(lcsa_kv_cache_append(&c, 1, 10, &first) == LCSA_ERR_PARAM);       // not newer
  CHECK(lcsa_kv_cache_append(&c, -1, 600, &first) == LCSA_ERR_PARAM);
  CHECK(lcsa_kv_cache_append(&c, 1, 600, nullptr) == LCSA_ERR_NULL);
  CHECK(lcsa_kv_cache_evict(&c, -1) == LCSA_ERR_PARAM);
  CHECK(lcsa_kv_cache_evict(&c, 0) == LCSA_OK);
  CHECK(lcsa_kv_cache_view(&c, &n, nullptr, nullptr) == LCSA_OK && n == 0);
  CHECK(lcsa_kv_cache_evict(&c, 0) == LCSA_OK);                           // underflow: no-op
  // corrupt metadata is refused, never indexed
  lcsa_kv_cache bad = c;
  bad.head = 99;
  CHECK(lcsa_kv_cache_view(&bad, &n, slots, tbs) == LCSA_ERR_CAPACITY);
  bad = c;
  bad.count = -3;
  CHECK(lcsa_kv_cache_append(&bad, 1, 700, &first) == LCSA_ERR_CAPACITY);
  bad = c;
  bad.n_slots = LCSA_MAX_SLOTS + 1;
  CHECK(lcsa_kv_cache_evict(&bad, 0) == LCSA_ERR_CAPACITY);

  // ---- ring init: sizes, slots, geometry
  lcsa_kv_cache d;
  CHECK(init(&d, 2, 64, 2, 3, LCSA_F32, 4, 1, 0) == LCSA_ERR_CAPACITY);
  CHECK(init(&d, 2, 64, 2, 3, LCSA_F32, 4, 0, 8) == LCSA_ERR_CAPACITY);
  CHECK(init(&d, 2, 64, 2, 3, LCSA_F32, 0) == LCSA_ERR_CAPACITY);
  CHECK(init(&d, 2, 64, 2, 3, LCSA_F32, LCSA_MAX_SLOTS + 1) == LCSA_ERR_CAPACITY);
  CHECK(init(&d, 2, 96, 2, 3, LCSA_BF16, 4) == LCSA_ERR_SHAPE);
  CHECK(init(&d, 2, 64, 2, 3, 5, 4) == LCSA_ERR_DTYPE);
  CHECK(init(&d, 2, 64, 0, 3, LCSA_BF16, 4) == LCSA_ERR_SHAPE);
  CHECK(lcsa_kv_cache_init(nullptr, 1, 1, 64, 1, 1, LCSA_BF16, 1, fake(16), fake(16),
                           (double*)fake(16), 1 << 20, 1 << 20, 1 << 20) == LCSA_ERR_NULL);
  CHECK(lcsa_kv_cache_init(&d, 1, 1, 64, 1, 1, LCSA_BF16, 1, fake(17), fake(16),
                           (double*)fake(16), 1 << 20, 1 << 20, 1 << 20) == LCSA_ERR_ALIGN);
  CHECK(init(&d, 2, 64, 2, 3, LCSA_F32, 4) == LCSA_OK);

  // ---- selection parameters and the kmax of a chunk
  lcsa_select_params p{11, LCSA_BORDER_PRESERVED, 0, 1, 5, 0, 768, 1280, 768, 1280, 0};
  int32_t k = -1;
  CHECK(lcsa_topk_count(&p, 0, 10, &k) == LCSA_OK && k == 0);
  CHECK(lcsa_topk_count(&p, 11, 10, &k) == LCSA_ERR_PARAM);
  CHECK(lcsa_topk_count(&p, -1, 10, &k) == LCSA_ERR_PARAM);
  CHECK(lcsa_topk_count(&p, 3, 10, &k) == LCSA_OK && k == 1);   // floor(3/5) = 0, clamped to 1
  CHECK(lcsa_topk_count(&p, 2147483647, 2147483647, &k) == LCSA_OK && k == 429496729);
  lcsa_select_params q = p;
  q.local_range = 10;
  CHECK(lcsa_topk_count(&q, 5, 10, &k) == LCSA_ERR_PARAM);
  q = p;
  q.ratio_den = 0;
  CHECK(lcsa_topk_count(&q, 5, 10, &k) == LCSA_ERR_PARAM);
  q = p;
  q.scale_by_resolution = 1;
  q.out_h = 0;
  CHECK(lcsa_topk_count(&q, 5, 10, &k) == LCSA_ERR_PARAM);
  q = p;
  q.ratio_base = 2;
  CHECK(lcsa_topk_count(&q, 5, 10, &k) == LCSA_ERR_PARAM);
  q = p;
  q.topk_fixed = 7;
  CHECK(lcsa_topk_count(&q, 5, 10, &k) == LCSA_OK && k == 5);
  // 768x1408 step: 4 TBs held, 264 candidates per row, k = 52
  lcsa_kv_cache e;
  CHECK(init(&e, 12, 128, 6, 11, LCSA_BF16, 4) == LCSA_OK);
  CHECK(lcsa_kv_cache_append(&e, 4, 0, &first) == LCSA_OK);
  const lcsa_geom gq{1, 12, 128, 2, 48, 88, LCSA_BF16};
  int32_t kmax = -1, cand = -1;
  CHECK(lcsa_max_topk(&gq, 3, &e, &p, &kmax) == LCSA_OK && kmax == 52);
  CHECK(lcsa_max_candidates(&gq, 3, &e, &p, &cand) == LCSA_OK && cand == 264);
  // the query TB 1 sees only TBs 0, 1: 132 candidates, k 26
  CHECK(lcsa_max_topk(&gq, 1, &e, &p, &kmax) == LCSA_OK && kmax == 26);
  const lcsa_geom gbad{1, 8, 128, 2, 48, 88, LCSA_BF16};
  CHECK(lcsa_max_topk(&gbad, 3, &e, &p, &kmax) == LCSA_ERR_SHAPE);
  CHECK(lcsa_max_topk(&gq, 3, &e, &p, nullptr) == LCSA_ERR_NULL);

  // ---- the hand k table, from stdin
  char line[256];
  int rows = 0;
  while (std::fgets(line, sizeof line, stdin)) {
    int num, den, scale, oh, ow, fixed, na, expect;
    if (std::sscanf(line, "k %d %d %d %d %d %d %d %d", &num, &den, &scale, &oh, &ow, &fixed, &na,
                    &expect) != 8)
      continue;
    lcsa_select_params r{11, LCSA_BORDER_PRESERVED, fixed, num, den, scale, oh, ow, 768, 1280, 0};
    CHECK(lcsa_topk_count(&r, na, 1000000, &k) == LCSA_OK);
    if (k != expect) std::fprintf(stderr, "k table: n_allowed %d gave %d, expected %d\n", na, k, expect);
    CHECK(k == expect);
    ++rows;
  }
  CHECK(rows >= 10);
  std::printf("host driver: %d k-table rows, %d failures\n", rows, failures);
  return failures == 0 ? 0 : 1;
}
