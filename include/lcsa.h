/*
 * lcsa.h -- locality-constrained block-sparse causal attention (LCSA) on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (sources):
 *   [FN] "FlashVSR: Towards Real-time Diffusion-Based Streaming Video Super
 *        Resolution" (papernotes.org CVPR 2026 note): Key design 1 (Stage 2
 *        causal mask: each latent sees only the current and past), Key design
 *        2 (block-sparse causal attention: (2,8,8) blocks of 128 tokens,
 *        block-mean pooling, a coarse block-to-block map, full 128x128
 *        attention only on the top-k block pairs), Key design 3 (local
 *        window constraint with a Boundary-Preserved and a
 *        Boundary-Truncated rule).
 *   [HW] "How FlashVSR works" (vsr-hover-compare learn page): section 2.2
 *        steps 1-3 (window partition, the local_range x local_range block
 *        mask, the draft scores / softmax / top-k, the topk_ratio rule that
 *        scales k inversely with resolution against 768x1280), section 2.3
 *        (streaming with a KV cache trimmed by dropping the oldest segment),
 *        section 5.3 (one block = 8x8 tokens of 2 latent frames).
 *
 * A streaming step is:
 *   lcsa_kv_cache_append   reserve ring slots for the chunk's temporal blocks
 *   lcsa_partition_pool    partition q/k/v into blocks, mean-pool q and k,
 *                          write k/v blocks straight into the ring slots
 *                          (q's blocks only when q_blk is given)
 *   lcsa_draft_mask        masked draft scores, row softmax, per-row top-k
 *                          (with an optional workspace of
 *                          lcsa_draft_workspace_size bytes for whole-grid
 *                          windows)
 *   lcsa_block_sparse_attn exact attention over the selected block pairs,
 *                          q read from q_blk (lcsa_block_sparse_attn_tok: q
 *                          read in token layout, so q_blk is never written)
 *   lcsa_kv_cache_evict    drop the oldest temporal blocks beyond capacity
 * and, between steps, lcsa_kv_cache_copy saves a stream's ring into a spare
 * one (a checkpoint) or restores it.
 *
 * Conventions shared by every entry point:
 *   - All buffers are allocated and owned by the caller, workspaces
 *     included. The library never allocates or frees memory. Its only state is the thread-local text of
 *     the last error and, for lcsa_block_sparse_attn_bwd_noalloc alone, a
 *     fixed scratch array on each GPU (see there).
 *   - Device pointers must be 16-byte aligned (LCSA_ERR_ALIGN otherwise).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued asynchronously; nothing synchronises.
 *   - Every argument is validated on the host before any HIP call. Nothing
 *     is padded, clamped or reshaped silently: an input the method does not
 *     define is refused with a status code. On failure nothing is enqueued
 *     and lcsa_last_error() describes the problem.
 *   - No function throws or aborts across this interface.
 *
 * Layouts (row-major, innermost last; B batch, NH heads, D head_dim):
 *   token layout  q, k, v, out:  [B][T][H][W][NH][D], tokens (t, y, x)
 *   query blocks  q_blk:         [B][NH][nq][128][D]
 *   pooled query  q_pool:        [B][NH][nq][D]               float64
 *   ring K        k_ring:        [B][NH][n_slots][nS][128][D]
 *   ring V        v_ring:        [B][NH][n_slots][nS][D][128] (block transposed)
 *   ring pooled K kpool_ring:    [B][NH][n_slots][D][nS]      float64 (d-major)
 *   selections    sel_idx:       [B][NH][nq][kmax] int32, sel_cnt [B][NH][nq]
 * with nby = H/8, nbx = W/8, nS = nby*nbx blocks per temporal block (TB),
 * nq = (T/2)*nS. Block n = (bt*nby + by)*nbx + bx holds the tokens
 * (2bt+dt, 8by+dy, 8bx+dx) at in-block position (dt*8 + dy)*8 + dx.
 * A key block's logical id is (its TB's position in the cache, oldest = 0)
 * * nS + by*nbx + bx.
 */
#ifndef LCSA_H
#define LCSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LCSA_OK = 0,
  LCSA_ERR_NULL = 1,      /* a required pointer is NULL */
  LCSA_ERR_SHAPE = 2,     /* sizes not a whole number of 2x8x8 windows, head_dim
                             unsupported, or geometry disagrees with the cache */
  LCSA_ERR_DTYPE = 3,     /* unknown dtype, or dtype disagrees with the cache */
  LCSA_ERR_PARAM = 4,     /* selection parameters out of their domain */
  LCSA_ERR_ALIGN = 5,     /* a device pointer is not 16-byte aligned */
  LCSA_ERR_CAPACITY = 6,  /* ring full, evicting more than held, kmax too
                             small, or a row with more candidates than the
                             draft kernel holds (LCSA_MAX_CANDIDATES) */
  LCSA_ERR_DEVICE = 7     /* a HIP call or kernel launch failed */
} lcsa_status;

typedef enum { LCSA_BF16 = 0, LCSA_F32 = 1 } lcsa_dtype;
typedef enum { LCSA_BORDER_PRESERVED = 0, LCSA_BORDER_TRUNCATED = 1 } lcsa_border;

#define LCSA_MAX_SLOTS 16          /* ring capacity limit, in temporal blocks */
#define LCSA_MAX_CANDIDATES 4096   /* allowed key blocks per query row */

/* Token grid of one chunk of new latent frames ([FN] Key design 2: blocks
 * of (2,8,8) tokens). frames even, height and width multiples of 8,
 * head_dim 64 or 128, batch and heads >= 1. frames == 0 is an empty chunk:
 * entry points accept it and do nothing. */
typedef struct {
  int32_t batch, heads, head_dim;
  int32_t frames, height, width;   /* latent frames x token rows x token cols */
  int32_t dtype;                   /* lcsa_dtype of q, k, v, q_blk, rings, out */
} lcsa_geom;

/* Selection knobs ([HW] 2.2 steps 2-3).
 *   local_range  odd, >= 1: each query block may see a local_range x
 *                local_range neighbourhood of key blocks (11 on the pages);
 *                a value >= the grid makes an axis unbounded.
 *   border       LCSA_BORDER_PRESERVED: a window of fixed size shifted to
 *                stay inside the grid; LCSA_BORDER_TRUNCATED: the centred
 *                window clipped at the grid edge ([FN] Key design 3).
 *   topk_fixed   > 0: keep min(topk_fixed, allowed) blocks per row.
 *   otherwise the ratio rule: k = floor(base * ratio_num/ratio_den
 *                * (scale_by_resolution ? ref_h*ref_w/(out_h*out_w) : 1))
 *                in exact integer arithmetic, clamped to [1, allowed];
 *                base = the row's allowed count (ratio_base 0) or every key
 *                block in the cache view (ratio_base 1). */
typedef struct {
  int32_t local_range;
  int32_t border;
  int32_t topk_fixed;
  int32_t ratio_num, ratio_den;
  int32_t scale_by_resolution;
  int32_t out_h, out_w;            /* output resolution in pixels */
  int32_t ref_h, ref_w;            /* base resolution of the ratio (768x1280) */
  int32_t ratio_base;
} lcsa_select_params;

/* Host-side metadata of one layer's streaming K/V cache ([HW] 2.3): a ring
 * of n_slots temporal-block slots in caller-owned device buffers. The
 * struct itself is caller-owned host memory; fill it with
 * lcsa_kv_cache_init and treat the fields as read-only. */
typedef struct {
  int32_t batch, heads, head_dim, nby, nbx, dtype;
  int32_t n_slots;                 /* ring capacity in temporal blocks */
  int32_t head;                    /* slot of the oldest held TB */
  int32_t count;                   /* TBs held (appended, not yet evicted) */
  int32_t reserved;
  int64_t abs_tb[LCSA_MAX_SLOTS];  /* absolute TB index held by each slot */
  void* k_ring;                    /* device, see layouts above */
  void* v_ring;
  double* kpool_ring;
} lcsa_kv_cache;

/* ---- cache metadata (host only, O(1), no HIP calls) -------------------- */

/* [HW] 2.3: the streaming KV cache that keeps the newest temporal blocks.
 * Set up an empty ring over caller-allocated device buffers: k_ring and
 * v_ring of B*NH*n_slots*nS*128*D elements in `dtype` (bytes_k, bytes_v
 * their sizes in bytes), kpool_ring of B*NH*n_slots*D*nS doubles
 * (bytes_kpool), nS = nby*nbx. 1 <= n_slots <= LCSA_MAX_SLOTS. A buffer
 * smaller than that is LCSA_ERR_CAPACITY: every later call writes and reads
 * the rings only inside those sizes. */
lcsa_status lcsa_kv_cache_init(lcsa_kv_cache* cache, int32_t batch, int32_t heads,
                               int32_t head_dim, int32_t nby, int32_t nbx,
                               int32_t dtype, int32_t n_slots, void* k_ring,
                               void* v_ring, double* kpool_ring, size_t bytes_k,
                               size_t bytes_v, size_t bytes_kpool);

/* Reserve slots for n_tb new temporal blocks numbered first_abs_tb,
 * first_abs_tb+1, ... (must be greater than every TB held). The slot of the
 * first is written to *first_slot_out; the others follow it modulo n_slots.
 * LCSA_ERR_CAPACITY if count + n_tb > n_slots. */
lcsa_status lcsa_kv_cache_append(lcsa_kv_cache* cache, int32_t n_tb,
                                 int64_t first_abs_tb, int32_t* first_slot_out);

/* Drop the oldest TBs until at most keep_tb remain ([HW] 2.3: the oldest
 * segment is discarded). keep_tb >= 0. O(1); no bytes move. */
lcsa_status lcsa_kv_cache_evict(lcsa_kv_cache* cache, int32_t keep_tb);

/* [HW] 2.3: the keys a streaming step attends are the cached segments
 * followed by the new one. The held TBs oldest -> newest: slots[i] and
 * abs_tb[i] for i < *n_out (at most LCSA_MAX_SLOTS entries each). Either
 * output array may be NULL. */
lcsa_status lcsa_kv_cache_view(const lcsa_kv_cache* cache, int32_t* n_out,
                               int32_t* slots, int64_t* abs_tb);

/* Checkpoint and resume of a stream ([HW] 2.3: the ring of cached segments
 * is the only state a streaming layer carries from one step to the next).
 * Copies what src holds into dst, slot for slot: for each held temporal
 * block its K, V^T and pooled-K slots of every (batch, head), then src's
 * head, count and abs_tb, so that dst continues the stream exactly where
 * src stood (bitwise: the next steps on dst give the results they would
 * have given on src). dst keeps its own buffers; slots src does not hold
 * are left as they were. dst and src must come from lcsa_kv_cache_init
 * with the same batch, heads, head_dim, grid and n_slots
 * (LCSA_ERR_SHAPE), and dtype (LCSA_ERR_DTYPE); dst == src, or a dst ring
 * overlapping any src ring, is LCSA_ERR_PARAM. The device copies are
 * enqueued on `stream` (device to device, no host staging) and dst's
 * metadata is updated when the call returns, so work that reads dst or
 * writes src goes on the same stream after it. A device error is
 * LCSA_ERR_DEVICE with dst's metadata unchanged (its ring may be partly
 * written). Save a checkpoint by copying the live cache into a spare one
 * of the same shape; resume by copying it back. */
lcsa_status lcsa_kv_cache_copy(lcsa_kv_cache* dst, const lcsa_kv_cache* src, void* stream);

/* ---- selection helpers (host only) ------------------------------------ */

/* [HW] 2.2 step 3, the topk_ratio rule (k shrinks as the output grows
 * past the 768x1280 base). k for a row with n_allowed candidates out of
 * n_keys key blocks, by the rule in lcsa_select_params; 0 when n_allowed
 * == 0. LCSA_ERR_PARAM unless 0 <= n_allowed <= n_keys. */
lcsa_status lcsa_topk_count(const lcsa_select_params* params, int32_t n_allowed,
                            int32_t n_keys, int32_t* k_out);

/* [HW] 2.2 steps 2-3 (the local window and causal TBs give each row its
 * candidates; the topk_ratio rule its k). Largest k over the query rows of
 * a chunk (geometry gq, first temporal block q_first_abs_tb) against the
 * TBs currently held by `cache`: the smallest kmax lcsa_draft_mask accepts. */
lcsa_status lcsa_max_topk(const lcsa_geom* gq, int64_t q_first_abs_tb,
                          const lcsa_kv_cache* cache,
                          const lcsa_select_params* params, int32_t* kmax_out);

/* ---- device steps ------------------------------------------------------ */

/* Steps 1-2 ([HW] 2.2 step 1 and step 3's pooling; [FN] Key design 2).
 * Partition the chunk's q, k, v (token layout, geometry g) into 128-token
 * blocks. q goes to q_blk with its block means in q_pool (float64); k and v
 * of temporal block t of the chunk go to ring slot (first_slot + t) %
 * n_slots, with the block means of k in kpool_ring. Those slots must be
 * the cache's newest TBs, in order: first_slot is the slot that
 * lcsa_kv_cache_append returned for this chunk (LCSA_ERR_PARAM otherwise;
 * LCSA_ERR_CAPACITY if the chunk has more TBs than the cache holds). q and
 * q_pool are both NULL (fill the cache only) or both non-NULL; q_blk may be
 * NULL with them, and then only q's block means are written (for the _tok
 * attention entry points, which read q in token layout). q_blk without q is
 * LCSA_ERR_NULL. */
lcsa_status lcsa_partition_pool(const lcsa_geom* g, const void* q, const void* k,
                                const void* v, void* q_blk, double* q_pool,
                                lcsa_kv_cache* cache, int32_t first_slot,
                                void* stream);

/* Steps 3-4 ([HW] 2.2 steps 2-3; [FN] Key designs 1-3). For each query
 * block of the chunk (geometry gq, first temporal block q_first_abs_tb) and
 * every key block held by the cache: candidate iff the key's TB is not
 * later than the query's and it lies in the local window; score =
 * q_pool . kpool / sqrt(D) (float64); softmax over the candidates (written to
 * probs, [B][NH][nq][n_keys] float64 with 0 off the candidates, when probs is
 * non-NULL; n_keys = cache count * nS; probs_bytes is its size in bytes and
 * a smaller buffer is LCSA_ERR_CAPACITY); keep the k candidates of largest
 * score, equal scores ordered by lower logical id. sel_idx receives the kept
 * logical ids in ascending order, padded with -1 up to kmax; sel_cnt the
 * count. kmax >= lcsa_max_topk() (LCSA_ERR_CAPACITY otherwise).
 * workspace (nullable): device memory, 256-byte aligned (LCSA_ERR_ALIGN),
 * of workspace_bytes bytes. With a window covering the whole grid and about
 * a thousand to 2,304 candidates per row (and probs NULL), the call then
 * writes each row's float32 scores there and selects from them with one
 * wave per row, instead of one fused kernel; the selections are the same.
 * It needs lcsa_draft_workspace_size() bytes (LCSA_ERR_CAPACITY if
 * smaller); other calls leave it untouched. The caller owns it; calls that
 * share one workspace must be ordered on one stream. */
lcsa_status lcsa_draft_mask(const lcsa_geom* gq, const double* q_pool,
                            int64_t q_first_abs_tb, const lcsa_kv_cache* cache,
                            const lcsa_select_params* params, int32_t kmax,
                            int32_t* sel_idx, int32_t* sel_cnt, double* probs,
                            size_t probs_bytes, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Bytes of workspace lcsa_draft_mask can use for a chunk of geometry gq and
 * the draft rule params, at any occupancy of `cache` (the float32 scores of
 * every query block against the cache's key blocks; [HW] 2.2 step 3 scores
 * every block pair of the coarse map). 0 when no occupancy takes the split
 * path. */
lcsa_status lcsa_draft_workspace_size(const lcsa_geom* gq, const lcsa_kv_cache* cache,
                                      const lcsa_select_params* params, size_t* bytes_out);

/* Step 5 ([FN] Key design 2: full 128x128 attention with the original Q, K,
 * V on the selected block pairs only; [HW] 2.2: unselected blocks are
 * skipped, not multiplied by zero). For every query token of block i:
 * out = softmax(scale * q . k_b) v_b over the tokens b of the blocks listed
 * in sel_idx[i][0 .. sel_cnt[i]) (logical ids into the cache as it is now).
 * scale == 0 means 1/sqrt(D). bf16 runs on MFMA with float32 accumulation;
 * f32 runs on the vector ALU. out is in token layout; lse (nullable,
 * [B][NH][nq][128] float32) receives the natural log-sum-exp of the scaled
 * logits. A row with sel_cnt 0 gets out = 0 and lse = -inf. A listed id
 * outside [0, cache count * nS) is skipped on the device: its block is never
 * read and contributes nothing (a row whose ids are all skipped gets out = 0
 * and lse = -inf). sel_cnt is clamped to [0, kmax]. */
lcsa_status lcsa_block_sparse_attn(const lcsa_geom* gq, const void* q_blk,
                                   const lcsa_kv_cache* cache,
                                   const int32_t* sel_idx, const int32_t* sel_cnt,
                                   int32_t kmax, float scale, void* out, float* lse,
                                   void* stream);

/* lcsa_block_sparse_attn ([FN] Key design 2, as above) with q read in token
 * layout [B][T][H][W][NH][D] (geometry gq, the chunk's q as given to
 * lcsa_partition_pool) instead of from q_blk: each query row is D
 * contiguous values there too, and the partition need not write q_blk.
 * Same results, arguments, errors and layouts otherwise. */
lcsa_status lcsa_block_sparse_attn_tok(const lcsa_geom* gq, const void* q,
                                       const lcsa_kv_cache* cache,
                                       const int32_t* sel_idx, const int32_t* sel_cnt,
                                       int32_t kmax, float scale, void* out, float* lse,
                                       void* stream);

/* ---- FlashVSR+ local lists ----------------------------------------------- */

/* [FP] "FlashVSR+" project page (flashvsr.tech), Abstract and Hybrid
 * Attention: most DiT blocks of the hybrid student attend a compact local
 * space-time neighbourhood, and periodic global blocks keep sparse global
 * interaction. A local layer needs no draft: its list is every key block of
 * the allowed set of lcsa_draft_mask (key TB not later than the query's, and
 * inside the params->local_range window under params->border), with the k
 * fields of params ignored; the temporal extent of the neighbourhood is the
 * cache that the caller keeps for that layer. A global layer is
 * lcsa_draft_mask with a window covering the whole grid. */

/* Largest number of allowed key blocks over the query rows of a chunk
 * against the TBs held by `cache`. Host only. */
lcsa_status lcsa_max_candidates(const lcsa_geom* gq, int64_t q_first_abs_tb,
                                const lcsa_kv_cache* cache,
                                const lcsa_select_params* params, int32_t* n_out);

/* sel_idx[i] = every allowed key block of query block i, ascending logical
 * ids, padded with -1 up to kmax; sel_cnt[i] the count. kmax >=
 * lcsa_max_candidates() (LCSA_ERR_CAPACITY otherwise). */
lcsa_status lcsa_local_lists(const lcsa_geom* gq, int64_t q_first_abs_tb,
                             const lcsa_kv_cache* cache, const lcsa_select_params* params,
                             int32_t kmax, int32_t* sel_idx, int32_t* sel_cnt, void* stream);

/* ---- Stage-1 segment-masked attention ---------------------------------- */

/* [FN] Key design 1, Stage 1: images are one-frame videos in the same 3D
 * attention, and a block-diagonal segment mask keeps every token's attention
 * inside its own segment (weights exp(q.k/sqrt(d)) times the same-segment
 * indicator, normalised over the same masked sum; no block sparsity, no
 * causality). frame_seg is a HOST array of gq->frames segment ids, one per
 * latent frame of the chunk; a token's segment is its frame's. These calls
 * take the chunk as a cold start: the cache must hold exactly the chunk's
 * temporal blocks, in order (view position p = temporal block
 * q_first_abs_tb + p), else LCSA_ERR_PARAM. At most 2 * LCSA_MAX_SLOTS
 * frames. */

/* Longest segment list of the chunk: nS times the largest number of the
 * chunk's temporal blocks that share a segment with one temporal block. The
 * smallest kmax lcsa_segment_lists accepts. Host only. */
lcsa_status lcsa_segment_max_list(const lcsa_geom* gq, const int32_t* frame_seg,
                                  int32_t* kmax_out);

/* For each query block i (temporal block a): sel_idx[i] = every key block of
 * every temporal block p of the chunk with a frame in the segment of one of
 * a's frames, ascending logical ids (p * nS + s), padded with -1 up to kmax;
 * sel_cnt[i] the count. kmax >= lcsa_segment_max_list() (LCSA_ERR_CAPACITY
 * otherwise). */
lcsa_status lcsa_segment_lists(const lcsa_geom* gq, int64_t q_first_abs_tb,
                               const lcsa_kv_cache* cache, const int32_t* frame_seg,
                               int32_t kmax, int32_t* sel_idx, int32_t* sel_cnt,
                               void* stream);

/* Attention of lcsa_block_sparse_attn over the listed key blocks, with the
 * token-level segment mask: key token b of a listed block is used by query
 * token a only if frame_seg of their latent frames are equal. Layouts,
 * scale, out and lse as in lcsa_block_sparse_attn; a query token with no
 * usable key gets out = 0 and lse = -inf. */
lcsa_status lcsa_segment_attn(const lcsa_geom* gq, const void* q_blk, int64_t q_first_abs_tb,
                              const lcsa_kv_cache* cache, const int32_t* frame_seg,
                              const int32_t* sel_idx, const int32_t* sel_cnt, int32_t kmax,
                              float scale, void* out, float* lse, void* stream);

/* lcsa_segment_attn with q read in token layout, as lcsa_block_sparse_attn_tok
 * does; everything else as lcsa_segment_attn. */
lcsa_status lcsa_segment_attn_tok(const lcsa_geom* gq, const void* q, int64_t q_first_abs_tb,
                                  const lcsa_kv_cache* cache, const int32_t* frame_seg,
                                  const int32_t* sel_idx, const int32_t* sel_cnt, int32_t kmax,
                                  float scale, void* out, float* lse, void* stream);

/* ---- Backward of the block-sparse attention ------------------------------ */

/* [FN] Key design 1 trains the student on all frames of a clip in parallel
 * under the block-sparse causal mask, and Key design 2 gives the attention
 * on the selected block pairs. The backward takes the training shape: the
 * keys are the chunk's own blocks (logical id = block index in the chunk,
 * (t, by, bx) order), the selection is held fixed, and q, k, v, out (the
 * forward output), dout (dL/dout) and the gradients dq, dk, dv are bf16 in
 * the token layout [B][T][H][W][NH][D]. lse is the forward's natural
 * log-sum-exp ([B][NH][nq][128] float32, from lcsa_block_sparse_attn).
 * sel_idx rows must be ascending (as every list builder here writes them),
 * with ids < nq; larger ids are skipped, as in the forward. scale 0 means
 * 1/sqrt(D). bf16 only (LCSA_ERR_DTYPE otherwise). */

/* Bytes of device workspace lcsa_block_sparse_attn_bwd needs for g: the
 * scaled lse and rowsum(dout * out) of every query (B*NH*nq*256 float32)
 * and the inverse lists (B*NH*nq counts, B*NH*nq*nq int32). Host only. */
lcsa_status lcsa_attn_bwd_workspace_size(const lcsa_geom* g, size_t* bytes_out);

/* dq, dk, dv of the attention over the listed blocks (all three written in
 * full; key blocks no row selects get dk = dv = 0). workspace: a device
 * buffer of at least lcsa_attn_bwd_workspace_size() bytes, 256-byte
 * aligned, owned by the caller and overwritten. Deterministic: no atomics. */
lcsa_status lcsa_block_sparse_attn_bwd(const lcsa_geom* g, const void* q, const void* k,
                                       const void* v, const void* out, const void* dout,
                                       const float* lse, const int32_t* sel_idx,
                                       const int32_t* sel_cnt, int32_t kmax, float scale,
                                       void* dq, void* dk, void* dv, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * lcsa_block_sparse_attn_bwd with its workspace taken from a scratch array
 * the library holds on each GPU for the life of the process
 * (LCSA_NOALLOC_SCRATCH_BYTES per GPU), instead of a caller buffer. Same
 * arguments, layouts, results and errors otherwise; a chunk whose workspace
 * (lcsa_attn_bwd_workspace_size) exceeds the scratch is LCSA_ERR_CAPACITY,
 * before any device work. The call allocates and frees nothing. Every call
 * on one GPU shares that GPU's scratch: calls that overlap on one GPU (on
 * concurrent streams, or from several threads) race and must be serialised
 * by the caller. The scratch keeps the last call's contents; each call
 * writes every byte it reads before reading it. */
#define LCSA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
lcsa_status lcsa_block_sparse_attn_bwd_noalloc(const lcsa_geom* g, const void* q, const void* k,
                                               const void* v, const void* out, const void* dout,
                                               const float* lse, const int32_t* sel_idx,
                                               const int32_t* sel_cnt, int32_t kmax, float scale,
                                               void* dq, void* dk, void* dv, void* stream);

/* Text of the last error on this thread ("" after success). */
const char* lcsa_last_error(void);

/* Interface version of this header: 5. */
int32_t lcsa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LCSA_H */
