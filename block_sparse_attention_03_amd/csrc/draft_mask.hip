// Steps 3-4 of LCSA: the masked draft block map, its row softmax and the
// per-row top-k selection.
//
// [HW] "How FlashVSR works" 2.2 step 3: score every (query block, key block)
// pair by the dot product of their mean vectors over sqrt(D), add the local
// mask (-inf outside the local_range x local_range neighbourhood, step 2),
// softmax each row and keep the strongest top-k pairs; k follows the
// topk_ratio rule. [FN] "FlashVSR" note, Key design 1: a latent only sees
// the current and past temporal blocks; Key design 3: two border rules.
//
// No dense mask exists: candidates are enumerated from block coordinates.
// The scoring layouts (kernels below) share the selections of
// draft_select.h:
//  * tile path (up to 768 candidates per row, e.g. the 11x11 window): a
//    workgroup scores a 4x4 tile of query blocks against the union of their
//    windows on the fp64 matrix cores;
//  * row-group path (larger windows, small whole-grid windows, and any call
//    that asks for the probabilities): a workgroup scores `gx` query rows of
//    one block row with the vector ALU, each pooled key fetched once;
//  * dense path (a window covering the grid, 1,024 to 2,304 candidates):
//    16 rows of a temporal block against every visible key on the fp64
//    matrix cores, scores kept in LDS as float32; with a workspace, the split
//    pair instead (64-row scoring workgroups writing float32 scores to device
//    memory, then one wave per row selecting).
// Scores land at each row's candidate index; then one wave per row takes the
// softmax (when asked for) and selects exactly k candidates, ties to the
// lower logical id. The window paths keep float64 scores, so the selection
// is decided on values equal to the exact ones up to summation order; the
// dense paths rank float32 scores and settle a float32 tie at the k-th place
// on recomputed float64 scores. Rows are ranked on the raw dot products:
// dividing by sqrt(D) is monotone and leaves the order as it is, so the
// division is only applied to the softmax written to probs.
#include "draft_select.h"
#include "lcsa_kernels.h"
#include "lcsa_window.h"

namespace lcsa {
namespace {
// NW waves per workgroup: one key of the group's union per thread, so a
// union of up to 64 * NW keys is scored in one round of D loads per thread.
template <int GX, int D, int NW>
__global__ __launch_bounds__(64 * NW) void draft_mask_kernel(DraftArgs a) {
  extern __shared__ double smem[];
  double* qs = smem;                                    // [D][GX]
  double* sc = smem + D * GX;                           // [GX][row_stride]
  uint32_t* hist_all = reinterpret_cast<uint32_t*>(sc + (size_t)GX * a.row_stride);  // [4][256]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nby = a.nby, nbx = a.nbx, nS = nby * nbx;
  const int ngx = (nbx + GX - 1) / GX;
  int task = xcd_task(a.B * a.NH * a.ntb_q * nby * ngx);
  if (task < 0) return;
  const int gxi = task % ngx;
  task /= ngx;
  const int by = task % nby;
  task /= nby;
  const int tq = task % a.ntb_q;
  task /= a.ntb_q;
  const int h = task % a.NH;
  const int b = task / a.NH;
  const int bx0 = gxi * GX;
  const int ng = min(GX, nbx - bx0);
  const int64_t qtb = a.q_first_abs_tb + tq;
  const int nq = a.ntb_q * nS;
  const int64_t n_keys = (int64_t)a.view.n * nS;

  int nvis = 0;
  for (int p = 0; p < a.view.n; ++p)
    if (a.view.abs_tb[p] <= qtb) nvis = p + 1;
  int ylo, yhi, uxlo, uxhi, tmp;
  window_range(by, nby, a.local_range, a.border, &ylo, &yhi);
  window_range(bx0, nbx, a.local_range, a.border, &uxlo, &tmp);
  window_range(bx0 + ng - 1, nbx, a.local_range, a.border, &tmp, &uxhi);
  const int ny = yhi - ylo + 1, nux = uxhi - uxlo + 1;
  const int n_union = nvis * ny * nux;

  int xlo[GX], xhi[GX];
#pragma unroll
  for (int g = 0; g < GX; ++g) {
    window_range(min(bx0 + g, nbx - 1), nbx, a.local_range, a.border, &xlo[g], &xhi[g]);
  }

  const size_t bh = (size_t)b * a.NH + h;
  const int row0 = tq * nS + by * nbx + bx0;
  __shared__ int32_t slot_tab[LCSA_MAX_SLOTS];
  stage_slots(a.view, slot_tab);
  for (int i = tid; i < D * GX; i += 64 * NW) {
    const int d = i / GX, g = i % GX;
    qs[i] = g < ng ? a.q_pool[(bh * nq + row0 + g) * D + d] : 0.0;
  }
  __syncthreads();

  // Phase A: score every key of the group's union window against each row.
  const SmallDiv div_nux(nux), div_ny(ny);
  for (int u = tid; u < n_union; u += 64 * NW) {
    const int r2 = div_nux(u), ux = u - r2 * nux;
    const int p = div_ny(r2), yy = r2 - p * ny;
    const int x = uxlo + ux, y = ylo + yy;
    const double* kp = a.kpool_ring + (bh * a.n_slots + slot_tab[p]) * (size_t)D * nS +
                       (size_t)y * nbx + x;
    double acc[GX];
#pragma unroll
    for (int g = 0; g < GX; ++g) acc[g] = 0.0;
#pragma unroll 16
    for (int d = 0; d < D; ++d) {
      const double kv = kp[(size_t)d * nS];
#pragma unroll
      for (int g = 0; g < GX; ++g) acc[g] = fma(qs[d * GX + g], kv, acc[g]);
    }
#pragma unroll
    for (int g = 0; g < GX; ++g) {
      if (g < ng && x >= xlo[g] && x <= xhi[g]) {
        const int nx = xhi[g] - xlo[g] + 1;
        sc[(size_t)g * a.row_stride + (p * ny + yy) * nx + (x - xlo[g])] = acc[g];
      }
    }
  }
  __syncthreads();

  // Phase B: one wave per row: softmax, exact top-k, sorted index list.
  uint32_t* hist = hist_all + wave * 256;
  for (int g = wave; g < ng; g += NW) {
    int gxlo, gxhi;  // recomputed: a dynamic index into xlo[] would spill
    window_range(bx0 + g, nbx, a.local_range, a.border, &gxlo, &gxhi);
    select_row(a, sc + (size_t)g * a.row_stride, bh * nq + row0 + g, nvis, ylo, ny, gxlo, gxhi,
               n_keys, hist, lane, sqrt((double)D));
  }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Matrix-core path for windows of up to kTileMaxCand candidates per row. A
// workgroup scores a 4 x 4 tile of query blocks (16 rows, one
// v_mfma_f64_16x16x4f64 row tile) against the union of their windows in
// tiles of 16 keys: A = pooled queries (staged d-major in LDS), B = pooled
// keys read straight from the d-major pooled ring (16 consecutive keys per d
// are one 128-byte run). Lane l holds A[l%16][l/16], B[l/16][l%16] and
// outputs D[4j + l/16][l%16], j = 0..3. Each output lands in LDS at its
// row's candidate index; then one wave per row runs select_row(). At most
// 128 registers per lane, so two workgroups share a CU where the LDS allows
// (up to 484 candidates per row): one's selection overlaps the other's
// scoring, and a half tile of key loads in flight per wave suffices.
constexpr int kTileMaxCand = 768;
// Fewer tiles than CUs (1536x2688 step: 189) leave CUs idle, so there each
// tile takes 16 waves, one row per wave in the selection phase (draft
// 39-40 -> 35 us); from one tile per CU on, 8 waves (two rows each) and two
// workgroups per CU.
constexpr long long kTileWideBelow = 256;
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 4) void draft_tile_kernel(DraftArgs a) {
  extern __shared__ double smem[];
  double* sc = smem;                                  // [16][row_stride] scores
  double* sa = sc + 16 * (size_t)a.row_stride;        // [D][16] pooled queries, d-major
  // the selection's histograms reuse the pooled-query region once scoring is done
  uint32_t* hist_all = reinterpret_cast<uint32_t*>(sa);  // [waves][256]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nby = a.nby, nbx = a.nbx, nS = nby * nbx;
  const int nty = (nby + 3) / 4, ntx = (nbx + 3) / 4;
  int task = xcd_task(a.B * a.NH * a.ntb_q * nty * ntx);
  if (task < 0) return;
  const int tx = task % ntx;
  task /= ntx;
  const int ty = task % nty;
  task /= nty;
  const int tq = task % a.ntb_q;
  task /= a.ntb_q;
  const int h = task % a.NH;
  const int b = task / a.NH;
  const int by0 = 4 * ty, bx0 = 4 * tx;
  const int by1 = min(by0 + 3, nby - 1), bx1 = min(bx0 + 3, nbx - 1);
  const int64_t qtb = a.q_first_abs_tb + tq;
  const int nq = a.ntb_q * nS;
  const int64_t n_keys = (int64_t)a.view.n * nS;
  const size_t bh = (size_t)b * a.NH + h;

  int nvis = 0;
  for (int p = 0; p < a.view.n; ++p)
    if (a.view.abs_tb[p] <= qtb) nvis = p + 1;
  int uylo, uyhi, uxlo, uxhi, tmp;
  window_range(by0, nby, a.local_range, a.border, &uylo, &tmp);
  window_range(by1, nby, a.local_range, a.border, &tmp, &uyhi);
  window_range(bx0, nbx, a.local_range, a.border, &uxlo, &tmp);
  window_range(bx1, nbx, a.local_range, a.border, &tmp, &uxhi);
  const int nuy = uyhi - uylo + 1, nux = uxhi - uxlo + 1;
  const int U = nvis * nuy * nux;

  __shared__ int32_t slot_tab[LCSA_MAX_SLOTS];
  stage_slots(a.view, slot_tab);
  // A operand: row rr of the tile is query block (by0 + rr/4, bx0 + rr%4),
  // staged d-major ([D][16]) so that the 16 rows of one k read 128
  // contiguous bytes (conflict-free); padding rows of an edge tile are 0
  for (int e = tid; e < 16 * D; e += 64 * NW) {
    const int rr = e % 16, d = e / 16;
    const int qy = by0 + (rr >> 2), qx = bx0 + (rr & 3);
    sa[e] = (qy < nby && qx < nbx)
                ? a.q_pool[(bh * nq + (size_t)tq * nS + qy * nbx + qx) * D + d]
                : 0.0;
  }
  __syncthreads();
  // lane (r, dq) holds A[r][4 s2 + dq] of k-step s2
  const int r = lane & 15, dq = lane >> 4;
  const double* arow = sa + dq * 16 + r;

  // this lane's four output rows: (qy, qx) = (by0 + j, bx0 + dq), with
  // their windows; an empty y range marks a row outside the grid
  const int oqx = bx0 + dq;
  int oxlo, oxhi;
  window_range(min(oqx, nbx - 1), nbx, a.local_range, a.border, &oxlo, &oxhi);
  const int onx = oxhi - oxlo + 1;
  const bool ocol = oqx < nbx;
  int oylo[4], oyhi[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    window_range(min(by0 + j, nby - 1), nby, a.local_range, a.border, &oylo[j], &oyhi[j]);
    if (by0 + j >= nby) oyhi[j] = oylo[j] - 1;
  }
  const SmallDiv div_nux(nux), div_nuy(nuy);

  // key u of tile t lives at (p, y, x); u >= U pads with key 0 (a valid
  // address) and is zeroed after the load
  auto key_ptr = [&](int u, int& p, int& y, int& x) {
    const int uu = u < U ? u : 0;
    const int r2 = div_nux(uu), ux = uu - r2 * nux;
    p = div_nuy(r2);
    y = uylo + r2 - p * nuy;
    x = uxlo + ux;
    return a.kpool_ring + (bh * a.n_slots + slot_tab[p]) * (size_t)D * nS + (size_t)y * nbx + x;
  };
  // One half tile (16 of the 32 k-steps) of key loads in flight at a time;
  // the other resident workgroup covers their latency.
  constexpr int HS = D / 8;  // k-steps per half tile
  const int ntiles = U > 16 * wave ? (U - 16 * wave + 16 * NW - 1) / (16 * NW) : 0;
  for (int it = 0; it < ntiles; ++it) {
    const int t = wave + it * NW;
    const int u = 16 * t + r;
    int p, y, x;
    const double* kp = key_ptr(u, p, y, x);
    // a padding key (u >= U, loaded from key 0) only feeds output column u,
    // which is never stored
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      double bf[HS];
#pragma unroll
      for (int s2 = 0; s2 < HS; ++s2) bf[s2] = kp[(size_t)(hh * HS * 4 + 4 * s2 + dq) * nS];
#pragma unroll
      for (int s2 = 0; s2 < HS; ++s2)
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(arow[(hh * HS + s2) * 64], bf[s2], acc, 0, 0, 0);
    }
    if (u < U && ocol && x >= oxlo && x <= oxhi) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (y < oylo[j] || y > oyhi[j]) continue;
        const int ny = oyhi[j] - oylo[j] + 1;
        sc[(size_t)(4 * j + dq) * a.row_stride + (p * ny + (y - oylo[j])) * onx + (x - oxlo)] =
            acc[j];
      }
    }
  }
  __syncthreads();  // scores complete; the pooled-query region becomes the histograms

  uint32_t* hist = hist_all + wave * 256;
  for (int ro = wave; ro < 16; ro += NW) {
    const int qy = by0 + (ro >> 2), qx = bx0 + (ro & 3);
    if (qy >= nby || qx >= nbx) continue;  // uniform per wave
    int ylo, yhi, xlo, xhi;
    window_range(qy, nby, a.local_range, a.border, &ylo, &yhi);
    window_range(qx, nbx, a.local_range, a.border, &xlo, &xhi);
    select_row(a, sc + (size_t)ro * a.row_stride, bh * nq + (size_t)tq * nS + qy * nbx + qx, nvis,
               ylo, yhi - ylo + 1, xlo, xhi, n_keys, hist, lane, sqrt((double)D));
  }
}

// ---- whole-grid windows ----------------------------------------------------
// When the window covers the whole grid (FlashVSR+ global layers, small
// grids under an 11x11 window), every query row of a temporal block has the
// same candidates: all key blocks of the visible TBs, in id order. A
// workgroup scores 16 consecutive rows of one TB against all of them on the
// fp64 matrix cores (A = pooled queries held in registers, B = 16 keys of
// the d-major pooled ring per product), so the pooled keys leave L2 once per
// 16 rows. The scores are kept in LDS as float32 (16 rows of up to 2,304
// candidates fit), and the selection stays exact on the float64 scores:
// rounding to float32 is monotone, so a candidate whose float32 score is
// above the k-th one has a larger float64 score as well, and only a tie of
// float32 values at the k-th place can hide an order; the tied candidates'
// float64 scores are then recomputed (one wave-wide dot product each) and
// the same selection runs on them.
constexpr int kDenseWaves = 8;               // 16 rows: two per wave in the selection
constexpr int kDenseMinCand = 1024;          // below this the row-group path is faster

template <int D>
__global__ __launch_bounds__(64 * kDenseWaves, 1) void draft_dense_kernel(DraftArgs a) {
  constexpr int KS = D / 4;  // k-steps of one 16 x 16 x 4 product chain
  extern __shared__ float dsm[];
  const int rs = a.row_stride;  // >= candidates, = 16 (mod 64): conflict-free score writes
  float* sc = dsm;              // [16][rs]
  uint32_t* hist_all = reinterpret_cast<uint32_t*>(dsm + 16 * (size_t)rs);  // [waves][264]

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nS = a.nby * a.nbx;
  const int ngr = (nS + 15) / 16;
  int task = xcd_task(a.B * a.NH * a.ntb_q * ngr);
  if (task < 0) return;
  const int gr = task % ngr;
  task /= ngr;
  const int tq = task % a.ntb_q;
  task /= a.ntb_q;
  const int h = task % a.NH;
  const int b = task / a.NH;
  const size_t bh = (size_t)b * a.NH + h;
  const int64_t qtb = a.q_first_abs_tb + tq;
  int nvis = 0;
  for (int p = 0; p < a.view.n; ++p)
    if (a.view.abs_tb[p] <= qtb) nvis = p + 1;
  const int n = nvis * nS;
  const int64_t n_keys = (int64_t)a.view.n * nS;
  const int nq = a.ntb_q * nS;
  const int s0 = 16 * gr;
  const int nrows = min(16, nS - s0);
  const size_t row0 = bh * nq + (size_t)tq * nS + s0;

  // lane (r, dq) holds A[r][4 s2 + dq] and B[4 s2 + dq][r] of k-step s2 and
  // outputs D[4 j + dq][r]: query row 4 j + dq against key 16 t + r
  const int r = lane & 15, dq = lane >> 4;
  double qa[KS];
#pragma unroll
  for (int s2 = 0; s2 < KS; ++s2)
    qa[s2] = r < nrows ? a.q_pool[(row0 + r) * D + 4 * s2 + dq] : 0.0;

  __shared__ int32_t slot_tab[LCSA_MAX_SLOTS];
  stage_slots(a.view, slot_tab);
  __syncthreads();
  const SmallDiv div_ns(nS);
  const int ntiles = (n + 15) / 16;
  // key u of tile t; u >= n reads key 0 (a valid address) and is never stored
  auto key_col = [&](int t) {
    int u = 16 * t + r;
    u = u < n ? u : 0;
    const int p = div_ns(u), sp = u - p * nS;
    return a.kpool_ring + (bh * a.n_slots + slot_tab[p]) * (size_t)D * nS + sp +
           (size_t)dq * nS;
  };
  // Two register buffers of B in turn: the next tile's keys are in flight
  // while this tile's products run. The loads are unconditional (a tile past
  // the last reads key 0 and is never stored): a load under a branch leaves
  // the compiler's wait counts conservative, and each product would then
  // wait for the next tile's loads issued just before it.
  auto load_tile = [&](int t, double (&b)[KS]) {
    const double* kp = key_col(t);
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) b[s2] = kp[(size_t)4 * s2 * nS];
  };
  auto score_tile = [&](int t, const double (&b)[KS]) {
    f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s2 = 0; s2 < KS; s2 += 2) {
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[s2], b[s2], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[s2 + 1], b[s2 + 1], acc1, 0, 0, 0);
    }
    const int u = 16 * t + r;
    if (t < ntiles && u < n) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[(size_t)(4 * j + dq) * rs + u] = (float)(acc0[j] + acc1[j]);
    }
  };
  double b0[KS], b1[KS];
  if (wave < ntiles) {  // uniform per wave
    load_tile(wave, b0);
    for (int t = wave; t < ntiles; t += 2 * kDenseWaves) {
      load_tile(t + kDenseWaves, b1);
      score_tile(t, b0);
      load_tile(t + 2 * kDenseWaves, b0);
      score_tile(t + kDenseWaves, b1);
    }
  }
  __syncthreads();

  for (int ro = wave; ro < nrows; ro += kDenseWaves) {
    float* srow = sc + (size_t)ro * rs;
    float v[kDenseM];
#pragma unroll
    for (int m = 0; m < kDenseM; ++m) {
      const int c = lane + 64 * m;
      v[m] = srow[c < n ? c : 0];
    }
    select_dense<D>(a, slot_tab, srow, v, n, row0 + ro, bh, nS, n_keys,
                    a.q_pool + (row0 + ro) * D, hist_all + wave * kHistStride, lane);
  }
}

template <int D>
hipError_t launch_dense(DraftArgs a, hipStream_t s) {
  const int nS = a.nby * a.nbx;
  const long long n_max = (long long)a.view.n * nS;
  a.row_stride = (int32_t)((n_max + 63) / 64 * 64 + 16);
  const long long tasks = (long long)a.B * a.NH * a.ntb_q * ((nS + 15) / 16);
  const long long wgs = 8 * ((tasks + 7) / 8);
  const size_t shmem = 16 * (size_t)a.row_stride * sizeof(float) + kDenseWaves * kHistStride * 4;
  if (shmem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)draft_dense_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(draft_dense_kernel<D>, dim3((unsigned)wgs), dim3(64 * kDenseWaves), shmem, s,
                     a);
  return hipGetLastError();
}

// Split form of the dense path, for callers that pass a workspace: the
// scores go to device memory and two kernels replace the fused one.
// Scoring: a workgroup takes 64 rows of one temporal block (16 per wave,
// held in registers as the A operand) against a chunk of 256 candidates;
// each 16-key tile of the pooled ring is loaded once into LDS and read by
// all four waves, so the pooled keys leave L2 once per 64 rows. The
// products run in the fused kernel's order, so the float32 scores are the
// same values. Selection: one wave per row over the whole chip, where the
// fused kernel's one workgroup per CU left part of the chip idle in its
// last round.
constexpr int kScoreTiles = 16;                       // 16-key tiles per scoring workgroup
constexpr int kSelWaves = 4;                          // rows per selection workgroup

// Workspace row stride: whole groups of four scores per lane (64 lanes).
inline int split_row_stride(long long n_max) { return (int)(((n_max + 255) / 256) * 256); }

template <int D>
__global__ __launch_bounds__(256, 2) void draft_score_kernel(DraftArgs a) {
  constexpr int KS = D / 4;      // k-steps of one 16 x 16 x 4 product chain
  constexpr int PER = D / 16;    // doubles one thread stages per tile
  // tile layout for the B fragments: (d, key r) at ((d / 8 * 4 + d % 4) * 16 + r) * 2 + d / 4 % 2,
  // so lane (r, dq) reads k-steps 2 sp and 2 sp + 1 as one 16-byte pair.
  // Before the tiles, the same memory stages the pooled queries: 32 rows at
  // a time, D + 2 doubles per row (the A fragment reads of 16 rows then fall
  // into distinct banks)
  constexpr int QS = D + 2;
  constexpr int LDS_D = 2 * 16 * D > 32 * QS ? 2 * 16 * D : 32 * QS;
  __shared__ __attribute__((aligned(16))) double lds_d[LDS_D];
  __shared__ int32_t slot_tab[LCSA_MAX_SLOTS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nS = a.nby * a.nbx;
  const int ngr = (nS + 63) / 64;
  const int n_max = a.view.n * nS;
  const int nch = (n_max + 16 * kScoreTiles - 1) / (16 * kScoreTiles);
  int task = xcd_task(a.B * a.NH * a.ntb_q * ngr * nch);
  if (task < 0) return;
  const int ch = task % nch;
  task /= nch;
  const int gr = task % ngr;
  task /= ngr;
  const int tq = task % a.ntb_q;
  task /= a.ntb_q;
  const size_t bh = (size_t)task;  // b * NH + h
  const int64_t qtb = a.q_first_abs_tb + tq;
  int nvis = 0;
  for (int p = 0; p < a.view.n; ++p)
    if (a.view.abs_tb[p] <= qtb) nvis = p + 1;
  const int n = nvis * nS;
  const int c0 = ch * 16 * kScoreTiles;
  if (c0 >= n) return;  // uniform: the chunk lies past this TB's candidates
  const int ntl = min(kScoreTiles, (n - c0 + 15) / 16);
  const int nq = a.ntb_q * nS;
  const int s0 = 64 * gr + 16 * wave;
  const int nrows = nS - s0;  // rows of this wave: min(16, nrows), none if <= 0
  const size_t row0 = bh * nq + (size_t)tq * nS + s0;

  stage_slots(a.view, slot_tab);
  const int r = lane & 15, dq = lane >> 4;
  // pooled queries: two passes of 32 rows, each row's D doubles read as
  // consecutive 16-byte pieces (rows past the TB's last block read as 0)
  const int tid2 = 2 * tid;
  const size_t grow0 = bh * nq + (size_t)tq * nS + 64 * gr;  // the workgroup's first row
  constexpr int QL = 32 * D / 512;                           // 16-byte loads per thread per pass
  double2 qx[2][QL];
#pragma unroll
  for (int ps = 0; ps < 2; ++ps)
#pragma unroll
    for (int i = 0; i < QL; ++i) {
      const int f = tid2 + 512 * i, rr = 32 * ps + f / D;
      qx[ps][i] = 64 * gr + rr < nS
                      ? *reinterpret_cast<const double2*>(a.q_pool + (grow0 + rr) * D + f % D)
                      : make_double2(0.0, 0.0);
    }
  double qa[KS];
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
#pragma unroll
    for (int i = 0; i < QL; ++i) {
      const int f = tid2 + 512 * i;
      *reinterpret_cast<double2*>(lds_d + (f / D) * QS + f % D) = qx[ps][i];
    }
    __syncthreads();
    if ((wave >> 1) == ps) {  // uniform per wave
      const double* qr = lds_d + (16 * (wave & 1) + r) * QS + dq;
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) qa[s2] = qr[4 * s2];
    }
    __syncthreads();
  }
  double (*kt)[16 * D] = reinterpret_cast<double (*)[16 * D]>(lds_d);

  // staging: thread (kr, dg) loads key c0 + 16 t + kr at d = dg + 16 e; a
  // key past the candidates reads key 0 (a valid address), never stored
  const int kr = tid & 15, dg = tid >> 4;
  const SmallDiv div_ns(nS);
  double pre[PER];
  auto load_tile = [&](int t) {
    int u = c0 + 16 * t + kr;
    u = u < n ? u : 0;
    const int p = div_ns(u), sp = u - p * nS;
    const double* kp = a.kpool_ring + (bh * a.n_slots + slot_tab[p]) * (size_t)D * nS + sp;
#pragma unroll
    for (int e = 0; e < PER; ++e) pre[e] = kp[(size_t)(dg + 16 * e) * nS];
  };
  auto stage_tile = [&](int buf) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int d = dg + 16 * e;
      kt[buf][(((d >> 3) * 4 + (d & 3)) * 16 + kr) * 2 + ((d >> 2) & 1)] = pre[e];
    }
  };

  float* ws = a.scores;
  const int rs = a.ws_stride;
  load_tile(0);
  stage_tile(0);
  load_tile(1);
  __syncthreads();
  for (int t = 0; t < ntl; ++t) {
    const double* kb = kt[t & 1];
    f64x4 acc0 = {0.0, 0.0, 0.0, 0.0}, acc1 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int sp = 0; sp < KS / 2; ++sp) {
      const double2 bb = *reinterpret_cast<const double2*>(kb + ((sp * 4 + dq) * 16 + r) * 2);
      acc0 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[2 * sp], bb.x, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[2 * sp + 1], bb.y, acc1, 0, 0, 0);
    }
    const int u = c0 + 16 * t + r;
    if (u < n) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (4 * j + dq < nrows) ws[(row0 + 4 * j + dq) * rs + u] = (float)(acc0[j] + acc1[j]);
    }
    if (t + 1 < ntl) {  // uniform
      stage_tile((t + 1) & 1);  // read by every wave in iteration t - 1, before the last barrier
      load_tile(t + 2);
    }
    __syncthreads();
  }
}

// One wave per row: the split selection over its float32 scores in the
// workspace (this wave's LDS row is its scratch).
template <int D>
__global__ __launch_bounds__(64 * kSelWaves) void draft_select_kernel(DraftArgs a) {
  extern __shared__ float xsm[];
  __shared__ int32_t slot_tab[LCSA_MAX_SLOTS];
  stage_slots(a.view, slot_tab);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nS = a.nby * a.nbx;
  const int nq = a.ntb_q * nS;
  const long long rows = (long long)a.B * a.NH * nq;
  const long long row = (long long)blockIdx.x * kSelWaves + wave;
  if (row >= rows) return;
  const size_t bh = (size_t)(row / nq);
  const int tq = (int)(row % nq) / nS;
  const int64_t qtb = a.q_first_abs_tb + tq;
  int nvis = 0;
  for (int p = 0; p < a.view.n; ++p)
    if (a.view.abs_tb[p] <= qtb) nvis = p + 1;
  const int n = nvis * nS;
  const int64_t n_keys = (int64_t)a.view.n * nS;
  const int ls = a.ws_stride + 16;  // LDS row: the candidates and 8 spare entries
  float* s = xsm + (size_t)wave * (ls + kHistStride);
  uint32_t* hist = reinterpret_cast<uint32_t*>(s + ls);
  select_split<D>(a, slot_tab, a.scores + (size_t)row * a.ws_stride, s, n, (size_t)row, bh, nS,
                  n_keys, a.q_pool + (size_t)row * D, hist, lane);
}

template <int D>
hipError_t launch_split(DraftArgs a, hipStream_t s) {
  const int nS = a.nby * a.nbx;
  const long long n_max = (long long)a.view.n * nS;
  a.ws_stride = split_row_stride(n_max);
  const long long ngr = (nS + 63) / 64;
  const long long nch = (n_max + 16 * kScoreTiles - 1) / (16 * kScoreTiles);
  const long long tasks = (long long)a.B * a.NH * a.ntb_q * ngr * nch;
  hipLaunchKernelGGL(draft_score_kernel<D>, dim3((unsigned)(8 * ((tasks + 7) / 8))), dim3(256), 0, s,
                     a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = (long long)a.B * a.NH * a.ntb_q * nS;
  const size_t shmem = (size_t)kSelWaves * (a.ws_stride + 16 + kHistStride) * sizeof(float);
  if (shmem > 64 * 1024) {
    e = hipFuncSetAttribute((const void*)draft_select_kernel<D>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(draft_select_kernel<D>, dim3((unsigned)((rows + kSelWaves - 1) / kSelWaves)),
                     dim3(64 * kSelWaves), shmem, s, a);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_tile_nw(const DraftArgs& a, long long tasks, hipStream_t s) {
  const long long wgs = 8 * ((tasks + 7) / 8);
  constexpr size_t kAux = (size_t)D * 16 * sizeof(double) > NW * 256 * 4
                             ? (size_t)D * 16 * sizeof(double)
                             : NW * 256 * 4;
  const size_t shmem = 16 * (size_t)a.row_stride * sizeof(double) + kAux;
  if (shmem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)draft_tile_kernel<D, NW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((draft_tile_kernel<D, NW>), dim3((unsigned)wgs), dim3(64 * NW), shmem, s, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_tile(const DraftArgs& a, hipStream_t s) {
  const long long tasks = (long long)a.B * a.NH * a.ntb_q * ((a.nby + 3) / 4) * ((a.nbx + 3) / 4);
  return tasks < kTileWideBelow ? launch_tile_nw<D, 16>(a, tasks, s)
                                : launch_tile_nw<D, 8>(a, tasks, s);
}

template <int GX, int D, int NW>
hipError_t launch(const DraftArgs& a, hipStream_t s) {
  const int ngx = (a.nbx + GX - 1) / GX;
  const long long tasks = (long long)a.B * a.NH * a.ntb_q * a.nby * ngx;
  const long long groups = 8 * ((tasks + 7) / 8);
  const size_t shmem =
      (size_t)D * GX * sizeof(double) + (size_t)GX * a.row_stride * sizeof(double) + NW * 256 * 4;
  if (shmem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)draft_mask_kernel<GX, D, NW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((draft_mask_kernel<GX, D, NW>), dim3((unsigned)groups), dim3(64 * NW), shmem, s,
                     a);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_gx(const DraftArgs& a, hipStream_t s) {
  switch (a.gx) {
    case 8: return launch<8, D, NW>(a, s);
    case 4: return launch<4, D, NW>(a, s);
    case 2: return launch<2, D, NW>(a, s);
    default: return launch<1, D, NW>(a, s);
  }
}

// Eight waves where the group's union window has 257..512 keys (one key per
// thread, one round of loads instead of a second round for a few threads);
// four otherwise.
template <int D>
hipError_t launch_d(const DraftArgs& a, hipStream_t s) {
  const long long uy = a.local_range < a.nby ? a.local_range : a.nby;
  const long long ux = a.local_range + a.gx - 1 < a.nbx ? a.local_range + a.gx - 1 : a.nbx;
  const long long union_max = (long long)a.view.n * uy * ux;
  return union_max > 256 && union_max <= 512 ? launch_gx<D, 8>(a, s) : launch_gx<D, 4>(a, s);
}

}  // namespace

// Whether a call takes the dense path: a window covering the whole grid and
// between kDenseMinCand and kDenseMaxCand candidates, without probabilities.
static bool takes_dense(const DraftArgs& a) {
  const bool whole_grid = a.border == 0
                              ? (a.nby <= a.local_range && a.nbx <= a.local_range)
                              : (a.local_range / 2 >= a.nby - 1 && a.local_range / 2 >= a.nbx - 1);
  const long long n_max = (long long)a.view.n * a.nby * a.nbx;
  return !a.probs && whole_grid && n_max >= kDenseMinCand && n_max <= kDenseMaxCand;
}

size_t draft_workspace_bytes(const DraftArgs& a) {
  if (!takes_dense(a)) return 0;
  const long long nS = (long long)a.nby * a.nbx;
  return (size_t)a.B * a.NH * a.ntb_q * nS * split_row_stride(a.view.n * nS) * sizeof(float);
}

hipError_t launch_draft_mask(const DraftArgs& a, hipStream_t s) {
  // The tile path pays where 4 x 4 neighbouring rows share most of a window
  // that is smaller than the grid, or where its tiles alone fill the chip.
  // A window spanning a small grid gives every row of a temporal block the
  // same candidates and few tiles; there the row-group path's many small
  // workgroups fill the chip better (768x1408 step: 24 vs 33 us; a 12-TB
  // chunk of the same grid has 864 tiles and keeps the tile path).
  // A window covering the whole grid gives every row of a temporal block
  // all visible keys: one dense score matrix per TB, scored 16 rows at a
  // time. It pays from about a thousand candidates per row (FlashVSR+ global
  // layer at 4K, 2,040: 434 -> 244 us), where the row groups' re-reads of
  // the pooled keys dominate; below that the row-group path's many small
  // workgroups win (768x1408 step, 264 candidates: 25 vs 44 us). With a
  // workspace the dense path runs as the split pair instead (scores in device
  // memory, one wave per row for the selection: 4K global layer 204-231 ->
  // 134-140 us). The draft's float64 probabilities come from the paths below.
  if (takes_dense(a)) {
    if (a.scores) return a.D == 64 ? launch_split<64>(a, s) : launch_split<128>(a, s);
    return a.D == 64 ? launch_dense<64>(a, s) : launch_dense<128>(a, s);
  }
  const bool window_inside = a.local_range < a.nby || a.local_range < a.nbx;
  const long long tiles =
      (long long)a.B * a.NH * a.ntb_q * ((a.nby + 3) / 4) * ((a.nbx + 3) / 4);
  if (a.row_stride <= kTileMaxCand && (window_inside || tiles >= 512))
    return a.D == 64 ? launch_tile<64>(a, s) : launch_tile<128>(a, s);
  return a.D == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace lcsa
