// Host-only part of the C-ABI: validation, the k rule, window bounds and the
// streaming ring's metadata ([HW] "How FlashVSR works" 2.3). No HIP calls.
#include "lcsa_host.h"
#include "lcsa_window.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>

namespace lcsa {

namespace {
thread_local char g_err[512] = "";
}

lcsa_status fail(lcsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

lcsa_status ok() {
  g_err[0] = '\0';
  return LCSA_OK;
}

void window_bounds(int32_t i, int32_t n, int32_t r, int32_t border, int32_t* lo,
                   int32_t* hi) {
  window_range(i, n, r, border, lo, hi);
}

int32_t topk_rule(const lcsa_select_params& p, int64_t n_allowed, int64_t n_keys) {
  if (n_allowed <= 0) return 0;
  if (p.topk_fixed > 0) return (int32_t)(p.topk_fixed < n_allowed ? p.topk_fixed : n_allowed);
  const int64_t base = p.ratio_base == 0 ? n_allowed : n_keys;
  // 128-bit products keep the rule exact for any int32 inputs.
  __int128 num = (__int128)p.ratio_num * (p.scale_by_resolution ? (int64_t)p.ref_h * p.ref_w : 1);
  __int128 den = (__int128)p.ratio_den * (p.scale_by_resolution ? (int64_t)p.out_h * p.out_w : 1);
  __int128 k = ((__int128)base * num) / den;
  if (k < 1) k = 1;
  if (k > n_allowed) k = n_allowed;
  return (int32_t)k;
}

lcsa_status check_geom(const lcsa_geom* g, const char* what) {
  if (!g) return fail(LCSA_ERR_NULL, "%s: geometry is NULL", what);
  if (g->batch < 1 || g->heads < 1)
    return fail(LCSA_ERR_SHAPE, "%s: batch (%d) and heads (%d) must be >= 1", what,
                g->batch, g->heads);
  if (g->head_dim != 64 && g->head_dim != 128)
    return fail(LCSA_ERR_SHAPE, "%s: head_dim %d unsupported (64 or 128)", what, g->head_dim);
  if (g->frames < 0 || g->frames % 2)
    return fail(LCSA_ERR_SHAPE, "%s: frames %d is not a whole number of 2-frame windows",
                what, g->frames);
  if (g->height < 8 || g->height % 8 || g->width < 8 || g->width % 8)
    return fail(LCSA_ERR_SHAPE, "%s: token grid %dx%d is not a whole number of 8x8 windows",
                what, g->height, g->width);
  if (g->dtype != LCSA_BF16 && g->dtype != LCSA_F32)
    return fail(LCSA_ERR_DTYPE, "%s: unknown dtype %d", what, g->dtype);
  const int64_t nS = (int64_t)(g->height / 8) * (g->width / 8);
  const int64_t tokens = (int64_t)g->frames * g->height * g->width;
  if (nS > (1 << 20) || tokens * g->heads * g->head_dim * g->batch > ((int64_t)1 << 40))
    return fail(LCSA_ERR_SHAPE, "%s: problem too large", what);
  return LCSA_OK;
}

lcsa_status check_params(const lcsa_select_params* p) {
  if (!p) return fail(LCSA_ERR_NULL, "selection parameters are NULL");
  if (p->local_range < 1 || p->local_range % 2 == 0)
    return fail(LCSA_ERR_PARAM, "local_range %d must be odd and >= 1", p->local_range);
  if (p->border != LCSA_BORDER_PRESERVED && p->border != LCSA_BORDER_TRUNCATED)
    return fail(LCSA_ERR_PARAM, "unknown border rule %d", p->border);
  if (p->topk_fixed < 0) return fail(LCSA_ERR_PARAM, "topk_fixed %d < 0", p->topk_fixed);
  if (p->topk_fixed == 0) {
    if (p->ratio_num <= 0 || p->ratio_den <= 0)
      return fail(LCSA_ERR_PARAM, "ratio %d/%d must be positive", p->ratio_num, p->ratio_den);
    if (p->scale_by_resolution &&
        (p->out_h <= 0 || p->out_w <= 0 || p->ref_h <= 0 || p->ref_w <= 0))
      return fail(LCSA_ERR_PARAM, "resolutions must be positive (out %dx%d, ref %dx%d)",
                  p->out_h, p->out_w, p->ref_h, p->ref_w);
    if (p->ratio_base != 0 && p->ratio_base != 1)
      return fail(LCSA_ERR_PARAM, "ratio_base %d must be 0 or 1", p->ratio_base);
  }
  return LCSA_OK;
}

lcsa_status check_ptr(const void* p, const char* name, bool allow_null) {
  if (!p) return allow_null ? LCSA_OK : fail(LCSA_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16)
    return fail(LCSA_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return LCSA_OK;
}

lcsa_status check_cache(const lcsa_kv_cache* c) {
  if (!c) return fail(LCSA_ERR_NULL, "cache is NULL");
  if (c->n_slots < 1 || c->n_slots > LCSA_MAX_SLOTS || c->count < 0 || c->count > c->n_slots ||
      c->head < 0 || c->head >= c->n_slots)
    return fail(LCSA_ERR_CAPACITY, "cache metadata is corrupt (n_slots %d, head %d, count %d)",
                c->n_slots, c->head, c->count);
  return LCSA_OK;
}

lcsa_status check_matches_cache(const lcsa_geom* g, const lcsa_kv_cache* c) {
  if (g->batch != c->batch || g->heads != c->heads || g->head_dim != c->head_dim ||
      g->height / 8 != c->nby || g->width / 8 != c->nbx)
    return fail(LCSA_ERR_SHAPE,
                "geometry (B %d, NH %d, D %d, %dx%d blocks) disagrees with the cache "
                "(B %d, NH %d, D %d, %dx%d blocks)",
                g->batch, g->heads, g->head_dim, g->height / 8, g->width / 8, c->batch,
                c->heads, c->head_dim, c->nby, c->nbx);
  if (g->dtype != c->dtype)
    return fail(LCSA_ERR_DTYPE, "dtype %d disagrees with the cache's %d", g->dtype, c->dtype);
  return LCSA_OK;
}

int32_t visible_tbs(const lcsa_kv_cache& c, int64_t tb) {
  int32_t n = 0;
  for (int32_t i = 0; i < c.count; ++i)
    if (c.abs_tb[(c.head + i) % c.n_slots] <= tb) n = i + 1;
  return n;
}

int32_t max_topk(const lcsa_geom& gq, int64_t q_first_abs_tb, const lcsa_kv_cache& c,
                 const lcsa_select_params& p, int64_t* n_allowed_max) {
  const int32_t nby = gq.height / 8, nbx = gq.width / 8, ntb = gq.frames / 2;
  const int64_t n_keys = (int64_t)c.count * nby * nbx;
  int32_t kmax = 0;
  int64_t amax = 0;
  for (int32_t t = 0; t < ntb; ++t) {
    const int32_t vis = visible_tbs(c, q_first_abs_tb + t);
    for (int32_t by = 0; by < nby; ++by) {
      int32_t ylo, yhi;
      window_bounds(by, nby, p.local_range, p.border, &ylo, &yhi);
      for (int32_t bx = 0; bx < nbx; ++bx) {
        int32_t xlo, xhi;
        window_bounds(bx, nbx, p.local_range, p.border, &xlo, &xhi);
        const int64_t na = (int64_t)vis * (yhi - ylo + 1) * (xhi - xlo + 1);
        const int32_t k = topk_rule(p, na, n_keys);
        if (k > kmax) kmax = k;
        if (na > amax) amax = na;
      }
    }
  }
  if (n_allowed_max) *n_allowed_max = amax;
  return kmax;
}

}  // namespace lcsa

using namespace lcsa;

extern "C" {

lcsa_status lcsa_kv_cache_init(lcsa_kv_cache* cache, int32_t batch, int32_t heads,
                               int32_t head_dim, int32_t nby, int32_t nbx, int32_t dtype,
                               int32_t n_slots, void* k_ring, void* v_ring,
                               double* kpool_ring, size_t bytes_k, size_t bytes_v,
                               size_t bytes_kpool) {
  if (!cache) return fail(LCSA_ERR_NULL, "cache is NULL");
  lcsa_geom g{batch, heads, head_dim, 0, nby * 8, nbx * 8, dtype};
  if (nby < 1 || nbx < 1) return fail(LCSA_ERR_SHAPE, "cache grid %dx%d blocks", nby, nbx);
  lcsa_status st = check_geom(&g, "lcsa_kv_cache_init");
  if (st) return st;
  if (n_slots < 1 || n_slots > LCSA_MAX_SLOTS)
    return fail(LCSA_ERR_CAPACITY, "n_slots %d outside [1, %d]", n_slots, LCSA_MAX_SLOTS);
  if ((st = check_ptr(k_ring, "k_ring")) || (st = check_ptr(v_ring, "v_ring")) ||
      (st = check_ptr(kpool_ring, "kpool_ring")))
    return st;
  // every block of every slot the kernels may touch must lie inside the
  // caller's buffers (sizes of at most 2^40 elements, so no overflow)
  const uint64_t blocks = (uint64_t)batch * heads * n_slots * nby * nbx;
  const uint64_t esize = dtype == LCSA_BF16 ? 2 : 4;
  const uint64_t need_kv = blocks * 128 * head_dim * esize;
  const uint64_t need_pool = blocks * head_dim * sizeof(double);
  if ((uint64_t)bytes_k < need_kv || (uint64_t)bytes_v < need_kv ||
      (uint64_t)bytes_kpool < need_pool)
    return fail(LCSA_ERR_CAPACITY,
                "ring buffers too small for %d slots: k %zu, v %zu, kpool %zu bytes given; "
                "%llu, %llu, %llu needed",
                n_slots, bytes_k, bytes_v, bytes_kpool, (unsigned long long)need_kv,
                (unsigned long long)need_kv, (unsigned long long)need_pool);
  std::memset(cache, 0, sizeof(*cache));
  cache->batch = batch;
  cache->heads = heads;
  cache->head_dim = head_dim;
  cache->nby = nby;
  cache->nbx = nbx;
  cache->dtype = dtype;
  cache->n_slots = n_slots;
  cache->k_ring = k_ring;
  cache->v_ring = v_ring;
  cache->kpool_ring = kpool_ring;
  for (int i = 0; i < LCSA_MAX_SLOTS; ++i) cache->abs_tb[i] = -1;
  return ok();
}

lcsa_status lcsa_kv_cache_append(lcsa_kv_cache* cache, int32_t n_tb, int64_t first_abs_tb,
                                 int32_t* first_slot_out) {
  lcsa_status st = check_cache(cache);
  if (st) return st;
  if (!first_slot_out) return fail(LCSA_ERR_NULL, "first_slot_out is NULL");
  if (n_tb < 0) return fail(LCSA_ERR_PARAM, "n_tb %d < 0", n_tb);
  if (first_abs_tb < 0) return fail(LCSA_ERR_PARAM, "first_abs_tb %lld < 0", (long long)first_abs_tb);
  if (cache->count + n_tb > cache->n_slots)
    return fail(LCSA_ERR_CAPACITY, "ring holds %d of %d TBs; cannot append %d", cache->count,
                cache->n_slots, n_tb);
  if (cache->count > 0) {
    const int64_t newest = cache->abs_tb[(cache->head + cache->count - 1) % cache->n_slots];
    if (first_abs_tb <= newest)
      return fail(LCSA_ERR_PARAM, "TB %lld is not newer than the newest held TB %lld",
                  (long long)first_abs_tb, (long long)newest);
  }
  const int32_t first = (cache->head + cache->count) % cache->n_slots;
  for (int32_t t = 0; t < n_tb; ++t) cache->abs_tb[(first + t) % cache->n_slots] = first_abs_tb + t;
  cache->count += n_tb;
  *first_slot_out = first;
  return ok();
}

lcsa_status lcsa_kv_cache_evict(lcsa_kv_cache* cache, int32_t keep_tb) {
  lcsa_status st = check_cache(cache);
  if (st) return st;
  if (keep_tb < 0) return fail(LCSA_ERR_PARAM, "keep_tb %d < 0", keep_tb);
  while (cache->count > keep_tb) {
    cache->abs_tb[cache->head] = -1;
    cache->head = (cache->head + 1) % cache->n_slots;
    --cache->count;
  }
  return ok();
}

lcsa_status lcsa_kv_cache_view(const lcsa_kv_cache* cache, int32_t* n_out, int32_t* slots,
                               int64_t* abs_tb) {
  lcsa_status st = check_cache(cache);
  if (st) return st;
  if (!n_out) return fail(LCSA_ERR_NULL, "n_out is NULL");
  *n_out = cache->count;
  for (int32_t i = 0; i < cache->count; ++i) {
    const int32_t s = (cache->head + i) % cache->n_slots;
    if (slots) slots[i] = s;
    if (abs_tb) abs_tb[i] = cache->abs_tb[s];
  }
  return ok();
}

lcsa_status lcsa_topk_count(const lcsa_select_params* params, int32_t n_allowed, int32_t n_keys,
                            int32_t* k_out) {
  lcsa_status st = check_params(params);
  if (st) return st;
  if (!k_out) return fail(LCSA_ERR_NULL, "k_out is NULL");
  if (n_allowed < 0 || n_keys < n_allowed)
    return fail(LCSA_ERR_PARAM, "need 0 <= n_allowed (%d) <= n_keys (%d)", n_allowed, n_keys);
  *k_out = topk_rule(*params, n_allowed, n_keys);
  return ok();
}

lcsa_status lcsa_max_topk(const lcsa_geom* gq, int64_t q_first_abs_tb, const lcsa_kv_cache* cache,
                          const lcsa_select_params* params, int32_t* kmax_out) {
  lcsa_status st;
  if ((st = check_geom(gq, "lcsa_max_topk")) || (st = check_params(params)) ||
      (st = check_cache(cache)) || (st = check_matches_cache(gq, cache)))
    return st;
  if (!kmax_out) return fail(LCSA_ERR_NULL, "kmax_out is NULL");
  *kmax_out = max_topk(*gq, q_first_abs_tb, *cache, *params, nullptr);
  return ok();
}

const char* lcsa_last_error(void) { return g_err; }

lcsa_status lcsa_max_candidates(const lcsa_geom* gq, int64_t q_first_abs_tb,
                                const lcsa_kv_cache* cache, const lcsa_select_params* params,
                                int32_t* n_out) {
  lcsa_status st;
  if ((st = check_geom(gq, "lcsa_max_candidates")) || (st = check_params(params)) ||
      (st = check_cache(cache)) || (st = check_matches_cache(gq, cache)))
    return st;
  if (!n_out) return fail(LCSA_ERR_NULL, "n_out is NULL");
  int64_t amax = 0;
  max_topk(*gq, q_first_abs_tb, *cache, *params, &amax);
  if (amax > INT32_MAX) return fail(LCSA_ERR_CAPACITY, "more than 2^31 candidates in a row");
  *n_out = (int32_t)amax;
  return ok();
}

int32_t lcsa_abi_version(void) { return 5; }

}  // extern "C"
