// C-ABI entry points that enqueue device work. Every argument is validated
// on the host (lcsa_host.cpp) before the first HIP call; on any failure
// nothing is enqueued.
#include <cmath>
#include <mutex>
#include <numeric>

#include "lcsa_host.h"
#include "lcsa_kernels.h"

using namespace lcsa;

namespace {

// Scratch of the allocation-free backward (lcsa_block_sparse_attn_bwd_noalloc):
// a file-scope device array, one copy on every GPU the library runs on, held
// until the process ends. Its host-side name is only a stand-in; the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept per device.
constexpr size_t kNoAllocScratchBytes = LCSA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, or nullptr (with the error recorded).
void* noalloc_scratch(const char* fn) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(LCSA_ERR_DEVICE, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(LCSA_ERR_DEVICE, "%s: device %d beyond the %d the scratch table covers", fn, dev,
         kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      fail(LCSA_ERR_DEVICE, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

RingView make_view(const lcsa_kv_cache& c) {
  RingView v{};
  v.n = c.count;
  for (int32_t i = 0; i < c.count; ++i) {
    const int32_t s = (c.head + i) % c.n_slots;
    v.slot[i] = s;
    v.abs_tb[i] = c.abs_tb[s];
  }
  return v;
}

lcsa_status device_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(LCSA_ERR_DEVICE, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return ok();
}

// Stage-1 segment tables from a host array of per-frame segment ids:
// key TBs of the chunk listed for each query TB (any frame pair shares a
// segment) and, per (query TB, key TB), which of the four frame pairs do.
lcsa_status segment_tables(const lcsa_geom* gq, const int32_t* frame_seg, const char* fn,
                           int32_t n_tb[LCSA_MAX_SLOTS], int8_t tb[LCSA_MAX_SLOTS][LCSA_MAX_SLOTS],
                           uint8_t qmask[LCSA_MAX_SLOTS][LCSA_MAX_SLOTS], int32_t* maxlen) {
  if (!frame_seg) return fail(LCSA_ERR_NULL, "%s: frame_seg is NULL", fn);
  const int32_t n = gq->frames / 2;
  if (n > LCSA_MAX_SLOTS)
    return fail(LCSA_ERR_CAPACITY, "%s: %d frames; segment attention takes at most %d", fn,
                gq->frames, 2 * LCSA_MAX_SLOTS);
  const int32_t nS = (gq->height / 8) * (gq->width / 8);
  int32_t most = 0;
  for (int32_t a = 0; a < n; ++a) {
    n_tb[a] = 0;
    for (int32_t p = 0; p < n; ++p) {
      uint8_t m = 0;
      for (int dq = 0; dq < 2; ++dq)
        for (int dk = 0; dk < 2; ++dk)
          if (frame_seg[2 * a + dq] == frame_seg[2 * p + dk]) m |= (uint8_t)(1u << (2 * dq + dk));
      qmask[a][p] = m;
      if (m) tb[a][n_tb[a]++] = (int8_t)p;
    }
    most = n_tb[a] > most ? n_tb[a] : most;
  }
  *maxlen = most * nS;
  return ok();
}

// The segment calls take the chunk as a cold start: the cache view must be
// exactly the chunk's temporal blocks, oldest first.
lcsa_status check_cold_view(const lcsa_geom* gq, int64_t q_first_abs_tb,
                            const lcsa_kv_cache* cache, const char* fn) {
  const int32_t n = gq->frames / 2;
  if (q_first_abs_tb < 0) return fail(LCSA_ERR_PARAM, "%s: q_first_abs_tb < 0", fn);
  bool same = cache->count == n;
  for (int32_t p = 0; same && p < n; ++p)
    same = cache->abs_tb[(cache->head + p) % cache->n_slots] == q_first_abs_tb + p;
  if (!same)
    return fail(LCSA_ERR_PARAM,
                "%s: the cache must hold exactly the chunk's %d temporal blocks from %lld", fn, n,
                (long long)q_first_abs_tb);
  return ok();
}

// Validation and argument setup shared by the attention entry points; q is
// q_blk (block layout) or, with tokens set, q in token layout.
lcsa_status attn_args(const lcsa_geom* gq, const void* q, bool tokens,
                      const lcsa_kv_cache* cache, const int32_t* sel_idx,
                      const int32_t* sel_cnt, int32_t kmax, float scale, void* out, float* lse,
                      const char* fn, AttnArgs* a) {
  lcsa_status st;
  if ((st = check_geom(gq, fn)) || (st = check_cache(cache)) ||
      (st = check_matches_cache(gq, cache)) || (st = check_ptr(q, tokens ? "q" : "q_blk")) ||
      (st = check_ptr(sel_idx, "sel_idx")) || (st = check_ptr(sel_cnt, "sel_cnt")) ||
      (st = check_ptr(out, "out")) || (st = check_ptr(lse, "lse", true)))
    return st;
  if (kmax < 1) return fail(LCSA_ERR_CAPACITY, "kmax %d < 1", kmax);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(LCSA_ERR_PARAM, "scale must be finite and >= 0 (0 = 1/sqrt(D))");
  if (gq->frames > 0 && cache->count == 0)
    return fail(LCSA_ERR_CAPACITY, "the cache holds no key blocks");
  *a = AttnArgs{};
  (tokens ? a->q_tok : a->q_blk) = q;
  a->k_ring = cache->k_ring;
  a->v_ring = cache->v_ring;
  a->sel_idx = sel_idx;
  a->sel_cnt = sel_cnt;
  a->out = out;
  a->lse = lse;
  a->B = gq->batch;
  a->NH = gq->heads;
  a->D = gq->head_dim;
  a->T = gq->frames;
  a->H = gq->height;
  a->W = gq->width;
  a->n_slots = cache->n_slots;
  a->kmax = kmax;
  a->view = make_view(*cache);
  a->scale = scale == 0.f ? 1.f / std::sqrt((float)gq->head_dim) : scale;
  return ok();
}

// Workspace sections of the backward, each rounded up to 256 bytes.
struct BwdLayout {
  size_t delta, inv_cnt, inv_idx, total;
};

BwdLayout bwd_layout(const lcsa_geom& g) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t nq = (size_t)(g.frames / 2) * (g.height / 8) * (g.width / 8);
  const size_t rows = (size_t)g.batch * g.heads * nq;
  BwdLayout L{};
  L.delta = 0;
  L.inv_cnt = L.delta + up(rows * 256 * 4);
  L.inv_idx = L.inv_cnt + up(rows * 4);
  L.total = L.inv_idx + up(rows * nq * 4);
  return L;
}

}  // namespace

extern "C" {

lcsa_status lcsa_partition_pool(const lcsa_geom* g, const void* q, const void* k, const void* v,
                                void* q_blk, double* q_pool, lcsa_kv_cache* cache,
                                int32_t first_slot, void* stream) {
  const char* fn = "lcsa_partition_pool";
  lcsa_status st;
  if ((st = check_geom(g, fn)) || (st = check_cache(cache)) ||
      (st = check_matches_cache(g, cache)))
    return st;
  const bool has_q = q || q_blk || q_pool;
  if (has_q && !(q && q_pool))
    return fail(LCSA_ERR_NULL, "q and q_pool must be both NULL or both non-NULL (q_blk needs q)");
  if ((st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (has_q && ((st = check_ptr(q, "q")) || (st = check_ptr(q_blk, "q_blk", true)) ||
                 (st = check_ptr(q_pool, "q_pool")))))
    return st;
  const int32_t ntb = g->frames / 2;
  if (ntb == 0) return ok();
  if (first_slot < 0 || first_slot >= cache->n_slots)
    return fail(LCSA_ERR_PARAM, "first_slot %d outside [0, %d)", first_slot, cache->n_slots);
  if (ntb > cache->count)
    return fail(LCSA_ERR_CAPACITY, "%s: a chunk of %d TBs but the cache holds %d; append first",
                fn, ntb, cache->count);
  // the chunk's TBs are the newest ones held, in order: the slots the last
  // append returned (any other first_slot would overwrite older cached TBs)
  const int32_t pos = (first_slot - cache->head + cache->n_slots) % cache->n_slots;
  if (pos + ntb != cache->count)
    return fail(LCSA_ERR_PARAM,
                "%s: first_slot %d is view position %d of %d held TBs; the chunk's %d TBs must "
                "be the newest (position %d)", fn, first_slot, pos, cache->count, ntb,
                cache->count - ntb);
  PartitionArgs a{};
  a.q = has_q ? q : nullptr;
  a.k = k;
  a.v = v;
  a.q_blk = has_q ? q_blk : nullptr;
  a.q_pool = q_pool;
  a.k_ring = cache->k_ring;
  a.v_ring = cache->v_ring;
  a.kpool_ring = cache->kpool_ring;
  a.B = g->batch;
  a.NH = g->heads;
  a.D = g->head_dim;
  a.T = g->frames;
  a.H = g->height;
  a.W = g->width;
  a.n_slots = cache->n_slots;
  a.first_slot = first_slot;
  a.dtype = g->dtype;
  return device_status(launch_partition_pool(a, (hipStream_t)stream), fn);
}

lcsa_status lcsa_kv_cache_copy(lcsa_kv_cache* dst, const lcsa_kv_cache* src, void* stream) {
  const char* fn = "lcsa_kv_cache_copy";
  lcsa_status st;
  if ((st = check_cache(src)) || (st = check_cache(dst))) return st;
  if (dst == src) return fail(LCSA_ERR_PARAM, "%s: dst and src are the same cache", fn);
  if (dst->batch != src->batch || dst->heads != src->heads || dst->head_dim != src->head_dim ||
      dst->nby != src->nby || dst->nbx != src->nbx || dst->n_slots != src->n_slots)
    return fail(LCSA_ERR_SHAPE,
                "%s: dst (B %d, NH %d, D %d, %dx%d blocks, %d slots) and src (B %d, NH %d, "
                "D %d, %dx%d blocks, %d slots) differ", fn, dst->batch, dst->heads,
                dst->head_dim, dst->nby, dst->nbx, dst->n_slots, src->batch, src->heads,
                src->head_dim, src->nby, src->nbx, src->n_slots);
  if (dst->dtype != src->dtype)
    return fail(LCSA_ERR_DTYPE, "%s: dst dtype %d, src dtype %d", fn, dst->dtype, src->dtype);
  if ((st = check_ptr(dst->k_ring, "dst k_ring")) || (st = check_ptr(dst->v_ring, "dst v_ring")) ||
      (st = check_ptr(dst->kpool_ring, "dst kpool_ring")) ||
      (st = check_ptr(src->k_ring, "src k_ring")) || (st = check_ptr(src->v_ring, "src v_ring")) ||
      (st = check_ptr(src->kpool_ring, "src kpool_ring")))
    return st;
  // per (batch, head): n_slots slots of nS blocks (rings [B][NH][n_slots]...)
  const size_t esize = src->dtype == LCSA_BF16 ? 2 : 4;
  const size_t nS = (size_t)src->nby * src->nbx;
  const size_t rows = (size_t)src->batch * src->heads;
  const size_t slot_kv = nS * 128 * src->head_dim * esize;
  const size_t slot_kp = nS * src->head_dim * sizeof(double);
  const size_t pitch_kv = slot_kv * src->n_slots, pitch_kp = slot_kp * src->n_slots;
  const uintptr_t d_ptr[3] = {(uintptr_t)dst->k_ring, (uintptr_t)dst->v_ring,
                              (uintptr_t)dst->kpool_ring};
  const uintptr_t s_ptr[3] = {(uintptr_t)src->k_ring, (uintptr_t)src->v_ring,
                              (uintptr_t)src->kpool_ring};
  const size_t len[3] = {rows * pitch_kv, rows * pitch_kv, rows * pitch_kp};
  for (int x = 0; x < 3; ++x)
    for (int y = 0; y < 3; ++y)
      if (d_ptr[x] < s_ptr[y] + len[y] && s_ptr[y] < d_ptr[x] + len[x])
        return fail(LCSA_ERR_PARAM, "%s: a dst ring overlaps a src ring", fn);
  const hipStream_t s = (hipStream_t)stream;
  for (int32_t i = 0; i < src->count; ++i) {
    const size_t slot = (size_t)((src->head + i) % src->n_slots);
    const size_t skv = slot * slot_kv, skp = slot * slot_kp;
    hipError_t e = hipMemcpy2DAsync((char*)dst->k_ring + skv, pitch_kv,
                                    (const char*)src->k_ring + skv, pitch_kv, slot_kv, rows,
                                    hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync((char*)dst->v_ring + skv, pitch_kv, (const char*)src->v_ring + skv,
                           pitch_kv, slot_kv, rows, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync((char*)dst->kpool_ring + skp, pitch_kp,
                           (const char*)src->kpool_ring + skp, pitch_kp, slot_kp, rows,
                           hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return device_status(e, fn);
  }
  dst->head = src->head;
  dst->count = src->count;
  for (int32_t i = 0; i < LCSA_MAX_SLOTS; ++i) dst->abs_tb[i] = src->abs_tb[i];
  return ok();
}

lcsa_status lcsa_draft_workspace_size(const lcsa_geom* gq, const lcsa_kv_cache* cache,
                                      const lcsa_select_params* params, size_t* bytes_out) {
  lcsa_status st;
  if ((st = check_geom(gq, "lcsa_draft_workspace_size")) || (st = check_params(params)) ||
      (st = check_cache(cache)) || (st = check_matches_cache(gq, cache)))
    return st;
  if (!bytes_out) return fail(LCSA_ERR_NULL, "bytes_out is NULL");
  DraftArgs a{};
  a.B = gq->batch;
  a.NH = gq->heads;
  a.D = gq->head_dim;
  a.ntb_q = gq->frames / 2;
  a.nby = gq->height / 8;
  a.nbx = gq->width / 8;
  a.local_range = params->local_range;
  a.border = params->border;
  size_t most = 0;  // over every occupancy of the cache
  for (int32_t nv = 1; nv <= cache->n_slots; ++nv) {
    a.view.n = nv;
    const size_t b = draft_workspace_bytes(a);
    most = b > most ? b : most;
  }
  *bytes_out = most;
  return ok();
}

lcsa_status lcsa_draft_mask(const lcsa_geom* gq, const double* q_pool, int64_t q_first_abs_tb,
                            const lcsa_kv_cache* cache, const lcsa_select_params* params,
                            int32_t kmax, int32_t* sel_idx, int32_t* sel_cnt, double* probs,
                            size_t probs_bytes, void* workspace, size_t workspace_bytes,
                            void* stream) {
  lcsa_status st;
  if ((st = check_geom(gq, "lcsa_draft_mask")) || (st = check_params(params)) ||
      (st = check_cache(cache)) || (st = check_matches_cache(gq, cache)) ||
      (st = check_ptr(q_pool, "q_pool")) || (st = check_ptr(sel_idx, "sel_idx")) ||
      (st = check_ptr(sel_cnt, "sel_cnt")) || (st = check_ptr(probs, "probs", true)))
    return st;
  if (q_first_abs_tb < 0) return fail(LCSA_ERR_PARAM, "q_first_abs_tb < 0");
  const int32_t ntb = gq->frames / 2;
  if (ntb == 0) return ok();
  int64_t amax = 0;
  const int32_t need = max_topk(*gq, q_first_abs_tb, *cache, *params, &amax);
  if (kmax < need || kmax < 1)
    return fail(LCSA_ERR_CAPACITY, "kmax %d is smaller than the largest k %d", kmax, need);
  if (amax > LCSA_MAX_CANDIDATES)
    return fail(LCSA_ERR_CAPACITY, "a row has %lld candidates; at most %d are supported",
                (long long)amax, LCSA_MAX_CANDIDATES);
  if (probs) {
    const uint64_t nq = (uint64_t)ntb * (gq->height / 8) * (gq->width / 8);
    const uint64_t n_keys = (uint64_t)cache->count * (gq->height / 8) * (gq->width / 8);
    const uint64_t need = (uint64_t)gq->batch * gq->heads * nq * n_keys * sizeof(double);
    if ((uint64_t)probs_bytes < need)
      return fail(LCSA_ERR_CAPACITY, "probs of %zu bytes; %llu needed for %llu keys", probs_bytes,
                  (unsigned long long)need, (unsigned long long)n_keys);
  }

  DraftArgs a{};
  a.q_pool = q_pool;
  a.kpool_ring = cache->kpool_ring;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.probs = probs;
  a.B = gq->batch;
  a.NH = gq->heads;
  a.D = gq->head_dim;
  a.ntb_q = ntb;
  a.nby = gq->height / 8;
  a.nbx = gq->width / 8;
  a.n_slots = cache->n_slots;
  a.kmax = kmax;
  a.q_first_abs_tb = q_first_abs_tb;
  a.view = make_view(*cache);
  a.local_range = params->local_range;
  a.border = params->border;
  a.topk_fixed = params->topk_fixed;
  a.ratio_base = params->ratio_base;
  if (params->topk_fixed == 0) {
    __int128 num = (__int128)params->ratio_num *
                   (params->scale_by_resolution ? (int64_t)params->ref_h * params->ref_w : 1);
    __int128 den = (__int128)params->ratio_den *
                   (params->scale_by_resolution ? (int64_t)params->out_h * params->out_w : 1);
    // reduce the fraction so the device's 64 x 64-bit product is exact
    __int128 x = num, y = den;
    while (y) {
      const __int128 t = x % y;
      x = y;
      y = t;
    }
    num /= x;
    den /= x;
    if (num > UINT32_MAX || den > INT64_MAX)
      return fail(LCSA_ERR_PARAM,
                  "ratio rule does not reduce to a 32-bit numerator and 64-bit denominator");
    a.ratio_num = (int64_t)num;
    a.ratio_den = (int64_t)den;
  } else {
    a.ratio_num = 1;
    a.ratio_den = 1;
  }
  a.row_stride = (int32_t)((amax + 1) / 2 * 2);
  if (a.row_stride < 2) a.row_stride = 2;
  // Rows per workgroup: the most that still leave >= 2 workgroups per CU
  // (but at least 2 rows, so a pooled key row serves two queries), then
  // fewer if the scores would not fit in 64 KB of LDS.
  const int64_t rows_per_col = (int64_t)a.B * a.NH * a.ntb_q * a.nby;
  int gx = 8;
  while (gx > 2 && rows_per_col * ((a.nbx + gx - 1) / gx) < 512) gx /= 2;
  while (gx > 1 && (int64_t)gx * a.row_stride * 8 > 64 * 1024) gx /= 2;
  a.gx = gx;
  if (workspace) {
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(LCSA_ERR_ALIGN, "lcsa_draft_mask: workspace is not 256-byte aligned");
    const size_t need = draft_workspace_bytes(a);
    if (need > workspace_bytes)
      return fail(LCSA_ERR_CAPACITY, "lcsa_draft_mask: workspace of %zu bytes; %zu needed",
                  workspace_bytes, need);
    if (need) a.scores = static_cast<float*>(workspace);
  }
  return device_status(launch_draft_mask(a, (hipStream_t)stream), "lcsa_draft_mask");
}

static lcsa_status sparse_attn(const lcsa_geom* gq, const void* q, bool tokens,
                               const lcsa_kv_cache* cache, const int32_t* sel_idx,
                               const int32_t* sel_cnt, int32_t kmax, float scale, void* out,
                               float* lse, void* stream, const char* fn) {
  AttnArgs a;
  lcsa_status st = attn_args(gq, q, tokens, cache, sel_idx, sel_cnt, kmax, scale, out, lse, fn, &a);
  if (st || gq->frames == 0) return st;
  return device_status(launch_block_sparse_attn(a, gq->dtype, false, (hipStream_t)stream), fn);
}

lcsa_status lcsa_block_sparse_attn(const lcsa_geom* gq, const void* q_blk,
                                   const lcsa_kv_cache* cache, const int32_t* sel_idx,
                                   const int32_t* sel_cnt, int32_t kmax, float scale, void* out,
                                   float* lse, void* stream) {
  return sparse_attn(gq, q_blk, false, cache, sel_idx, sel_cnt, kmax, scale, out, lse, stream,
                     "lcsa_block_sparse_attn");
}

lcsa_status lcsa_block_sparse_attn_tok(const lcsa_geom* gq, const void* q,
                                       const lcsa_kv_cache* cache, const int32_t* sel_idx,
                                       const int32_t* sel_cnt, int32_t kmax, float scale,
                                       void* out, float* lse, void* stream) {
  return sparse_attn(gq, q, true, cache, sel_idx, sel_cnt, kmax, scale, out, lse, stream,
                     "lcsa_block_sparse_attn_tok");
}

lcsa_status lcsa_local_lists(const lcsa_geom* gq, int64_t q_first_abs_tb,
                             const lcsa_kv_cache* cache, const lcsa_select_params* params,
                             int32_t kmax, int32_t* sel_idx, int32_t* sel_cnt, void* stream) {
  const char* fn = "lcsa_local_lists";
  lcsa_status st;
  if ((st = check_geom(gq, fn)) || (st = check_params(params)) || (st = check_cache(cache)) ||
      (st = check_matches_cache(gq, cache)) || (st = check_ptr(sel_idx, "sel_idx")) ||
      (st = check_ptr(sel_cnt, "sel_cnt")))
    return st;
  if (q_first_abs_tb < 0) return fail(LCSA_ERR_PARAM, "q_first_abs_tb < 0");
  const int32_t ntb = gq->frames / 2;
  if (ntb == 0) return ok();
  if (ntb > LCSA_MAX_SLOTS)
    return fail(LCSA_ERR_CAPACITY, "%s: a chunk of %d TBs; at most %d", fn, ntb, LCSA_MAX_SLOTS);
  int64_t amax = 0;
  max_topk(*gq, q_first_abs_tb, *cache, *params, &amax);
  if (kmax < amax)
    return fail(LCSA_ERR_CAPACITY, "%s: kmax %d is smaller than the largest list %lld", fn,
                kmax, (long long)amax);
  LocalListArgs a{};
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.nby = gq->height / 8;
  a.nbx = gq->width / 8;
  a.nq = ntb * a.nby * a.nbx;
  a.rows = gq->batch * gq->heads * a.nq;
  a.kmax = kmax;
  a.local_range = params->local_range;
  a.border = params->border;
  for (int32_t t = 0; t < ntb; ++t) a.n_vis[t] = visible_tbs(*cache, q_first_abs_tb + t);
  return device_status(launch_local_lists(a, (hipStream_t)stream), fn);
}

lcsa_status lcsa_attn_bwd_workspace_size(const lcsa_geom* g, size_t* bytes_out) {
  lcsa_status st;
  if ((st = check_geom(g, "lcsa_attn_bwd_workspace_size"))) return st;
  if (!bytes_out) return fail(LCSA_ERR_NULL, "bytes_out is NULL");
  *bytes_out = bwd_layout(*g).total;
  return ok();
}

// Validation and launch of the backward, shared by the entry point that
// takes a caller workspace and the one that uses the library's scratch.
// check_ws: whether workspace / workspace_bytes come from the caller.
static lcsa_status attn_bwd(const lcsa_geom* g, const void* q, const void* k, const void* v,
                            const void* out, const void* dout, const float* lse,
                            const int32_t* sel_idx, const int32_t* sel_cnt, int32_t kmax,
                            float scale, void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, void* stream, const char* fn,
                            bool check_ws) {
  lcsa_status st;
  if ((st = check_geom(g, fn)) || (st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) ||
      (st = check_ptr(v, "v")) || (st = check_ptr(out, "out")) ||
      (st = check_ptr(dout, "dout")) || (st = check_ptr(lse, "lse")) ||
      (st = check_ptr(sel_idx, "sel_idx")) || (st = check_ptr(sel_cnt, "sel_cnt")) ||
      (st = check_ptr(dq, "dq")) || (st = check_ptr(dk, "dk")) || (st = check_ptr(dv, "dv")) ||
      (check_ws && (st = check_ptr(workspace, "workspace"))))
    return st;
  if (g->dtype != LCSA_BF16) return fail(LCSA_ERR_DTYPE, "%s: bf16 only", fn);
  if (kmax < 1) return fail(LCSA_ERR_CAPACITY, "kmax %d < 1", kmax);
  if (!std::isfinite(scale) || scale < 0.f)
    return fail(LCSA_ERR_PARAM, "scale must be finite and >= 0 (0 = 1/sqrt(D))");
  // a 32-row quarter of a block spans 4 token rows; its tiles are read with
  // 32-bit offsets from the quarter's first token
  if ((int64_t)(3 * (int64_t)g->width + 8) * g->heads * g->head_dim * 2 >= ((int64_t)1 << 31))
    return fail(LCSA_ERR_CAPACITY, "%s: token rows of %d x %d x %d are too wide", fn, g->width,
                g->heads, g->head_dim);
  const BwdLayout lay = bwd_layout(*g);
  if (check_ws) {
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
      return fail(LCSA_ERR_ALIGN, "%s: workspace is not 256-byte aligned", fn);
    if (workspace_bytes < lay.total)
      return fail(LCSA_ERR_CAPACITY, "%s: workspace of %zu bytes, %zu needed", fn,
                  workspace_bytes, lay.total);
  } else if (lay.total > workspace_bytes) {
    return fail(LCSA_ERR_CAPACITY,
                "%s: this chunk needs %zu bytes of scratch; the library's scratch holds %zu "
                "(use lcsa_block_sparse_attn_bwd with a caller workspace)",
                fn, lay.total, workspace_bytes);
  }
  if (g->frames == 0) return ok();
  if (!check_ws && !(workspace = noalloc_scratch(fn))) return LCSA_ERR_DEVICE;
  char* ws = (char*)workspace;
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.ld2 = (float*)(ws + lay.delta);
  a.inv_cnt = (int32_t*)(ws + lay.inv_cnt);
  a.inv_idx = (int32_t*)(ws + lay.inv_idx);
  a.B = g->batch;
  a.NH = g->heads;
  a.D = g->head_dim;
  a.T = g->frames;
  a.H = g->height;
  a.W = g->width;
  a.kmax = kmax;
  a.scale = scale == 0.f ? 1.f / std::sqrt((float)g->head_dim) : scale;
  return device_status(launch_attn_bwd(a, (hipStream_t)stream), fn);
}

lcsa_status lcsa_block_sparse_attn_bwd(const lcsa_geom* g, const void* q, const void* k,
                                       const void* v, const void* out, const void* dout,
                                       const float* lse, const int32_t* sel_idx,
                                       const int32_t* sel_cnt, int32_t kmax, float scale,
                                       void* dq, void* dk, void* dv, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return attn_bwd(g, q, k, v, out, dout, lse, sel_idx, sel_cnt, kmax, scale, dq, dk, dv,
                  workspace, workspace_bytes, stream, "lcsa_block_sparse_attn_bwd", true);
}

lcsa_status lcsa_block_sparse_attn_bwd_noalloc(const lcsa_geom* g, const void* q, const void* k,
                                               const void* v, const void* out, const void* dout,
                                               const float* lse, const int32_t* sel_idx,
                                               const int32_t* sel_cnt, int32_t kmax, float scale,
                                               void* dq, void* dk, void* dv, void* stream) {
  return attn_bwd(g, q, k, v, out, dout, lse, sel_idx, sel_cnt, kmax, scale, dq, dk, dv, nullptr,
                  kNoAllocScratchBytes, stream, "lcsa_block_sparse_attn_bwd_noalloc", false);
}

lcsa_status lcsa_segment_max_list(const lcsa_geom* gq, const int32_t* frame_seg,
                                  int32_t* kmax_out) {
  lcsa_status st;
  if ((st = check_geom(gq, "lcsa_segment_max_list"))) return st;
  if (!kmax_out) return fail(LCSA_ERR_NULL, "kmax_out is NULL");
  int32_t n_tb[LCSA_MAX_SLOTS];
  int8_t tb[LCSA_MAX_SLOTS][LCSA_MAX_SLOTS];
  uint8_t qmask[LCSA_MAX_SLOTS][LCSA_MAX_SLOTS];
  int32_t most = 0;
  if ((st = segment_tables(gq, frame_seg, "lcsa_segment_max_list", n_tb, tb, qmask, &most)))
    return st;
  *kmax_out = most;
  return ok();
}

lcsa_status lcsa_segment_lists(const lcsa_geom* gq, int64_t q_first_abs_tb,
                               const lcsa_kv_cache* cache, const int32_t* frame_seg,
                               int32_t kmax, int32_t* sel_idx, int32_t* sel_cnt, void* stream) {
  const char* fn = "lcsa_segment_lists";
  lcsa_status st;
  if ((st = check_geom(gq, fn)) || (st = check_cache(cache)) ||
      (st = check_matches_cache(gq, cache)) || (st = check_ptr(sel_idx, "sel_idx")) ||
      (st = check_ptr(sel_cnt, "sel_cnt")))
    return st;
  if (gq->frames == 0) return ok();
  SegListArgs a{};
  uint8_t qmask[LCSA_MAX_SLOTS][LCSA_MAX_SLOTS];
  int32_t most = 0;
  if ((st = segment_tables(gq, frame_seg, fn, a.n_tb, a.tb, qmask, &most)) ||
      (st = check_cold_view(gq, q_first_abs_tb, cache, fn)))
    return st;
  if (kmax < most)
    return fail(LCSA_ERR_CAPACITY, "%s: kmax %d is smaller than the longest list %d", fn, kmax,
                most);
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.nS = (gq->height / 8) * (gq->width / 8);
  a.nq = (gq->frames / 2) * a.nS;
  a.rows = gq->batch * gq->heads * a.nq;
  a.kmax = kmax;
  return device_status(launch_segment_lists(a, (hipStream_t)stream), fn);
}

static lcsa_status segment_attn(const lcsa_geom* gq, const void* q, bool tokens,
                                int64_t q_first_abs_tb, const lcsa_kv_cache* cache,
                                const int32_t* frame_seg, const int32_t* sel_idx,
                                const int32_t* sel_cnt, int32_t kmax, float scale, void* out,
                                float* lse, void* stream, const char* fn) {
  AttnArgs a;
  lcsa_status st = attn_args(gq, q, tokens, cache, sel_idx, sel_cnt, kmax, scale, out, lse, fn, &a);
  if (st || gq->frames == 0) return st;
  int32_t n_tb[LCSA_MAX_SLOTS];
  int8_t tb[LCSA_MAX_SLOTS][LCSA_MAX_SLOTS];
  int32_t most = 0;
  if ((st = segment_tables(gq, frame_seg, fn, n_tb, tb, a.qmask, &most)) ||
      (st = check_cold_view(gq, q_first_abs_tb, cache, fn)))
    return st;
  return device_status(launch_block_sparse_attn(a, gq->dtype, true, (hipStream_t)stream), fn);
}

lcsa_status lcsa_segment_attn(const lcsa_geom* gq, const void* q_blk, int64_t q_first_abs_tb,
                              const lcsa_kv_cache* cache, const int32_t* frame_seg,
                              const int32_t* sel_idx, const int32_t* sel_cnt, int32_t kmax,
                              float scale, void* out, float* lse, void* stream) {
  return segment_attn(gq, q_blk, false, q_first_abs_tb, cache, frame_seg, sel_idx, sel_cnt, kmax,
                      scale, out, lse, stream, "lcsa_segment_attn");
}

lcsa_status lcsa_segment_attn_tok(const lcsa_geom* gq, const void* q, int64_t q_first_abs_tb,
                                  const lcsa_kv_cache* cache, const int32_t* frame_seg,
                                  const int32_t* sel_idx, const int32_t* sel_cnt, int32_t kmax,
                                  float scale, void* out, float* lse, void* stream) {
  return segment_attn(gq, q, true, q_first_abs_tb, cache, frame_seg, sel_idx, sel_cnt, kmax,
                      scale, out, lse, stream, "lcsa_segment_attn_tok");
}

}  // extern "C"
