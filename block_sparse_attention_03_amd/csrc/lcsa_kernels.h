// Launch interface between the C-ABI entry points (lcsa_api.hip) and the
// gfx950 kernels. Arguments are validated before these are called.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/lcsa.h"

namespace lcsa {

// Order of the held temporal blocks, oldest first, passed by value so a
// step needs no host-to-device copy.
struct RingView {
  int32_t n;                         // TBs in the view
  int32_t slot[LCSA_MAX_SLOTS];      // ring slot of view position p
  int64_t abs_tb[LCSA_MAX_SLOTS];    // absolute TB index of view position p
};

struct PartitionArgs {
  const void* q;
  const void* k;
  const void* v;
  void* q_blk;
  double* q_pool;
  void* k_ring;
  void* v_ring;
  double* kpool_ring;
  int32_t B, NH, D, T, H, W;
  int32_t n_slots, first_slot;
  int32_t dtype;
};

struct DraftArgs {
  const double* q_pool;     // [B][NH][nq][D]
  const double* kpool_ring; // [B][NH][n_slots][D][nS]
  int32_t* sel_idx;         // [B][NH][nq][kmax]
  int32_t* sel_cnt;         // [B][NH][nq]
  double* probs;            // [B][NH][nq][n_keys] or null
  int32_t B, NH, D, ntb_q, nby, nbx, n_slots, kmax;
  int64_t q_first_abs_tb;
  RingView view;
  int32_t local_range, border, topk_fixed, ratio_base;
  int64_t ratio_num, ratio_den;      // reduced fraction incl. resolution scale
  int32_t row_stride;                // LDS scores per row (>= max candidates)
  int32_t gx;                        // query rows (consecutive bx) per workgroup
  float* scores;                     // split dense path: [B][NH][nq][ws_stride] float32, or null
  int32_t ws_stride;                 // scores per workspace row (set by the launcher)
};

struct AttnArgs {
  const void* q_blk;        // [B][NH][nq][128][D], read when q_tok is null
  const void* q_tok;        // q in token layout [B][T][H][W][NH][D], or null
  const void* k_ring;       // [B][NH][n_slots][nS][128][D]
  const void* v_ring;       // [B][NH][n_slots][nS][D][128]
  const int32_t* sel_idx;   // [B][NH][nq][kmax]
  const int32_t* sel_cnt;   // [B][NH][nq]
  void* out;                // [B][T][H][W][NH][D]
  float* lse;               // [B][NH][nq][128] or null
  int32_t B, NH, D, T, H, W;
  int32_t n_slots, kmax;
  RingView view;
  float scale;              // softmax scale on q.k
  // segment-masked kernels only: bit 2*dq + dk of qmask[a][p] is set when
  // frame dq of query TB a and frame dk of key view position p share a segment
  uint8_t qmask[LCSA_MAX_SLOTS][LCSA_MAX_SLOTS];
};

struct SegListArgs {
  int32_t* sel_idx;         // [B][NH][nq][kmax]
  int32_t* sel_cnt;         // [B][NH][nq]
  int32_t rows, nq, nS, kmax;
  int32_t n_tb[LCSA_MAX_SLOTS];                 // key TBs listed for query TB a
  int8_t tb[LCSA_MAX_SLOTS][LCSA_MAX_SLOTS];    // those TBs, ascending
};

struct LocalListArgs {
  int32_t* sel_idx;         // [B][NH][nq][kmax]
  int32_t* sel_cnt;         // [B][NH][nq]
  int32_t rows, nq, nby, nbx, kmax;
  int32_t local_range, border;
  int32_t n_vis[LCSA_MAX_SLOTS];  // view positions visible to query TB a (a prefix)
};

// Backward of the block-sparse attention on the training shape: the keys
// are the chunk's own blocks (logical id = block index in the chunk).
struct BwdArgs {
  const void* q;            // token layout [B][T][H][W][NH][D], bf16
  const void* k;
  const void* v;
  const void* out;          // forward output O
  const void* dout;         // dL/dO
  const float* lse;         // [B][NH][nq][128] natural log-sum-exp of the forward
  const int32_t* sel_idx;   // [B][NH][nq][kmax], ascending ids < nq, -1 padded
  const int32_t* sel_cnt;   // [B][NH][nq]
  void* dq;                 // token layout, bf16
  void* dk;
  void* dv;
  float* ld2;               // workspace [B][NH][nq][256]: lse * log2(e) of the 128 queries,
                            // then rowsum(dO * O) of the same queries
  int32_t* inv_cnt;         // workspace [B][NH][nq]: query blocks selecting key block j
  int32_t* inv_idx;         // workspace [B][NH][nq][nq]: those query blocks, ascending
  int32_t B, NH, D, T, H, W, kmax;
  float scale;
};

hipError_t launch_partition_pool(const PartitionArgs& a, hipStream_t s);
hipError_t launch_draft_mask(const DraftArgs& a, hipStream_t s);
// Workspace bytes lcsa_draft_mask's split dense path needs for a (0 when
// the call takes another path).
size_t draft_workspace_bytes(const DraftArgs& a);
hipError_t launch_block_sparse_attn(const AttnArgs& a, int32_t dtype, bool segment, hipStream_t s);
hipError_t launch_segment_lists(const SegListArgs& a, hipStream_t s);
hipError_t launch_local_lists(const LocalListArgs& a, hipStream_t s);
hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t s);

}  // namespace lcsa
