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
// Two scoring layouts share one selection routine:
//  * tile path (up to 768 candidates per row, e.g. the 11x11 window): a
//    workgroup scores a 4x4 tile of query blocks against the union of their
//    windows on the fp64 matrix cores;
//  * row-group path (larger windows): a workgroup scores `gx` query rows of
//    one block row with the vector ALU, each pooled key fetched once.
// Scores land in LDS at each row's candidate index; then one wave per row
// takes the softmax and selects exactly k candidates (value-range bucket
// select, ties to the lower logical id). Scores are float64 so the
// selection is decided on values equal to the exact ones up to summation
// order. Rows are ranked on the raw dot products: dividing by sqrt(D) is
// monotone and leaves the order as it is, so the division is only applied
// to the softmax written to probs.
#include "lcsa_kernels.h"
#include "lcsa_window.h"

namespace lcsa {
namespace {

// XCD-contiguous task order: workgroups are dealt to the 8 XCDs in turn, so
// XCD x takes tasks [x*per, (x+1)*per) and neighbouring query tiles, whose
// windows share pooled keys, hit the same L2. Launch 8*per workgroups;
// returns -1 for the padding ones.
__device__ inline int xcd_task(int n_tasks) {
  const int per = (n_tasks + 7) / 8;
  const int t = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  return t < n_tasks ? t : -1;
}

// Quotient of a small non-negative int by a divisor d >= 1 through an fp32
// reciprocal, exact for n < 2^22: (n + 0.5) / d lies at least 0.5 / d from
// an integer, and the two correctly rounded fp32 steps (1/d, then the
// product) move it by less than (n + 0.5) * 2^-23 / d < 0.5 / d.
struct SmallDiv {
  float inv;
  __device__ explicit SmallDiv(int d) : inv(1.0f / (float)d) {}
  __device__ int operator()(int n) const { return (int)(((float)n + 0.5f) * inv); }
};

__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ inline int32_t topk_dev(const DraftArgs& a, int64_t n_allowed, int64_t n_keys) {
  if (n_allowed <= 0) return 0;
  if (a.topk_fixed > 0) return (int32_t)(a.topk_fixed < n_allowed ? a.topk_fixed : n_allowed);
  const int64_t base = a.ratio_base == 0 ? n_allowed : n_keys;
  // the host reduced num/den and checked num < 2^32, so base * num < 2^56
  const uint64_t kk = ((uint64_t)base * (uint64_t)a.ratio_num) / (uint64_t)a.ratio_den;
  const int64_t k = kk > (uint64_t)n_allowed ? n_allowed : (int64_t)kk;
  return (int32_t)(k < 1 ? 1 : k);
}

// ---- DPP wave primitives (gfx9 row operations: no LDS round trip) --------
template <int CTRL, int ROWS>
__device__ inline double dpp_keep(double v) {  // lanes outside ROWS keep their value
  const int lo = __double2loint(v), hi = __double2hiint(v);
  return __hiloint2double(__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xF, false),
                          __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xF, false));
}

__device__ inline double lane63_f64(double v) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 63),
                          __builtin_amdgcn_readlane(__double2loint(v), 63));
}

// quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror, row_bcast:15,
// row_bcast:31: the full-wave result ends in lane 63.
__device__ inline double wave_max_dpp(double v) {
  v = fmax(v, dpp_keep<0xB1, 0xF>(v));
  v = fmax(v, dpp_keep<0x4E, 0xF>(v));
  v = fmax(v, dpp_keep<0x141, 0xF>(v));
  v = fmax(v, dpp_keep<0x140, 0xF>(v));
  v = fmax(v, dpp_keep<0x142, 0xA>(v));
  v = fmax(v, dpp_keep<0x143, 0xC>(v));
  return lane63_f64(v);
}

__device__ inline double wave_min_dpp(double v) {
  v = fmin(v, dpp_keep<0xB1, 0xF>(v));
  v = fmin(v, dpp_keep<0x4E, 0xF>(v));
  v = fmin(v, dpp_keep<0x141, 0xF>(v));
  v = fmin(v, dpp_keep<0x140, 0xF>(v));
  v = fmin(v, dpp_keep<0x142, 0xA>(v));
  v = fmin(v, dpp_keep<0x143, 0xC>(v));
  return lane63_f64(v);
}

// Inclusive prefix sum over lanes 0..63 (row_shr 1,2,4,8 with zero fill,
// then row_bcast:15 / :31 to carry across rows).
__device__ inline uint32_t wave_prefix_sum_dpp(uint32_t x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return (uint32_t)v;
}

// One wave: softmax (optional probs), exact top-k and the sorted index list
// of query row `row`, whose candidates are scores s[0 .. n) enumerated as
// c = (p*ny + (y - ylo))*nx + (x - xlo) over visible TBs p < nvis.
//
// Exact top-k by value-range bucketing: the candidates in [lo, hi] are
// binned into 256 equal-width bins (a monotone map of the value, so every
// key in a higher bin is larger than every key in a lower one); the bin
// holding the k-th largest becomes the new [lo, hi] (its own min and max)
// and is refined again, until it is kept whole or holds one value, whose
// copies are then taken lowest index first. Each level removes at least
// one distinct value, so the loop ends; smooth score rows need 1-2 levels.
__device__ void select_row(const DraftArgs& a, const double* s, size_t row, int nvis, int ylo,
                           int ny, int gxlo, int gxhi, int64_t n_keys, uint32_t* hist, int lane,
                           double sqrt_d) {
  const int nby = a.nby, nbx = a.nbx, nS = nby * nbx;
  const int yhi = ylo + ny - 1;
  const int nx = gxhi - gxlo + 1;
  const int n = nvis * ny * nx;
  const int k = topk_dev(a, n, n_keys);
  int32_t* out = a.sel_idx + row * a.kmax;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  double lo = INFINITY, hi = -INFINITY;
  for (int c = lane; c < n; c += 64) {
    lo = fmin(lo, s[c]);
    hi = fmax(hi, s[c]);
  }
  lo = wave_min_dpp(lo);
  hi = wave_max_dpp(hi);

  if (a.probs) {
    double* pr = a.probs + row * n_keys;
    double z = 0.0;
    for (int c = lane; c < n; c += 64) z += exp((s[c] - hi) / sqrt_d);
    z = wave_sum_f64(z);
    for (int64_t j = lane; j < n_keys; j += 64) {
      const int p = (int)(j / nS), rem = (int)(j % nS);
      const int y = rem / nbx, x = rem % nbx;
      double val = 0.0;
      if (p < nvis && y >= ylo && y <= yhi && x >= gxlo && x <= gxhi)
        val = exp((s[(p * ny + (y - ylo)) * nx + (x - gxlo)] - hi) / sqrt_d) / z;
      pr[j] = val;
    }
  }

  int kr = k;
  if (k >= n) {  // every candidate kept: the range already covers them all
    kr = n;
  } else if (k > 0) {
    for (int level = 0; level <= n && lo < hi; ++level) {
      const double scale = 256.0 / (hi - lo);
#pragma unroll
      for (int q = 0; q < 4; ++q) hist[lane * 4 + q] = 0u;
      wave_sync();
      for (int c = lane; c < n; c += 64) {
        const double v = s[c];
        if (v >= lo && v <= hi) {
          int bn = (int)((v - lo) * scale);
          bn = bn < 0 ? 0 : (bn > 255 ? 255 : bn);
          atomicAdd(&hist[255 - bn], 1u);  // reversed: position 0 is the top bin
        }
      }
      wave_sync();
      uint32_t hb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hb[q] = hist[lane * 4 + q];
      const uint32_t tot = hb[0] + hb[1] + hb[2] + hb[3];
      uint32_t ab = wave_prefix_sum_dpp(tot) - tot;  // candidates in higher bins
      int found = -1;
      uint32_t fa = 0, fc = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (found < 0 && ab < (uint32_t)kr && ab + hb[q] >= (uint32_t)kr) {
          found = 255 - (lane * 4 + q);
          fa = ab;
          fc = hb[q];
        }
        ab += hb[q];
      }
      const uint64_t bal = __ballot(found >= 0);
      wave_sync();
      if (bal == 0) break;  // only with NaN scores; the emit below stays in bounds
      const int src = __ffsll((long long)bal) - 1;
      const int bin = __builtin_amdgcn_readlane(found, src);
      const int ca = __builtin_amdgcn_readlane((int)fa, src);
      const int cb = __builtin_amdgcn_readlane((int)fc, src);
      kr -= ca;
      double nlo = INFINITY, nhi = -INFINITY;
      for (int c = lane; c < n; c += 64) {
        const double v = s[c];
        if (v >= lo && v <= hi) {
          int bn = (int)((v - lo) * scale);
          bn = bn < 0 ? 0 : (bn > 255 ? 255 : bn);
          if (bn == bin) {
            nlo = fmin(nlo, v);
            nhi = fmax(nhi, v);
          }
        }
      }
      lo = wave_min_dpp(nlo);
      hi = wave_max_dpp(nhi);
      if (cb == kr) break;  // the whole bin is kept
    }
  }
  // Emit in ascending candidate order (= ascending logical id): values above
  // the final range, then the first kr values inside it.
  int eq_before = 0, sel_before = 0;
  const SmallDiv div_nx(nx), div_ny(ny);
  if (k > 0) {
    for (int base = 0; base < n; base += 64) {
      const int c = base + lane;
      const bool valid = c < n;
      const double v = valid ? s[c] : 0.0;
      const bool gt = valid && v > hi;
      const bool eq = valid && v >= lo && v <= hi;
      const uint64_t beq = __ballot(eq);
      const int r = eq_before + __popcll(beq & lt_mask);
      const bool want = gt || (eq && r < kr);
      const int pos = sel_before + __popcll(__ballot(want) & lt_mask);
      const bool sel = want && pos < k;  // never more than k (only NaN scores could ask)
      const uint64_t bsel = __ballot(sel);
      if (sel) {
        const int r3 = div_nx(c), xx = c - r3 * nx;
        const int p = div_ny(r3), yy = r3 - p * ny;
        out[pos] = p * nS + (ylo + yy) * nbx + gxlo + xx;
      }
      eq_before += __popcll(beq);
      sel_before += __popcll(bsel);
    }
  }
  for (int pos = sel_before + lane; pos < a.kmax; pos += 64) out[pos] = -1;
  if (lane == 0) a.sel_cnt[row] = sel_before;
}

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
    const double* kp = a.kpool_ring + (bh * a.n_slots + a.view.slot[p]) * (size_t)D * nS +
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
constexpr int kTileWaves = 8;  // 16 rows: two per wave in the selection phase

template <int D>
__global__ __launch_bounds__(64 * kTileWaves, 4) void draft_tile_kernel(DraftArgs a) {
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

  // A operand: row rr of the tile is query block (by0 + rr/4, bx0 + rr%4),
  // staged d-major ([D][16]) so that the 16 rows of one k read 128
  // contiguous bytes (conflict-free); padding rows of an edge tile are 0
  for (int e = tid; e < 16 * D; e += 64 * kTileWaves) {
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
    return a.kpool_ring + (bh * a.n_slots + a.view.slot[p]) * (size_t)D * nS + (size_t)y * nbx + x;
  };
  // One half tile (16 of the 32 k-steps) of key loads in flight at a time;
  // the other resident workgroup covers their latency.
  constexpr int HS = D / 8;  // k-steps per half tile
  const int ntiles = U > 16 * wave ? (U - 16 * wave + 16 * kTileWaves - 1) / (16 * kTileWaves) : 0;
  for (int it = 0; it < ntiles; ++it) {
    const int t = wave + it * kTileWaves;
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
  for (int ro = wave; ro < 16; ro += kTileWaves) {
    const int qy = by0 + (ro >> 2), qx = bx0 + (ro & 3);
    if (qy >= nby || qx >= nbx) continue;  // uniform per wave
    int ylo, yhi, xlo, xhi;
    window_range(qy, nby, a.local_range, a.border, &ylo, &yhi);
    window_range(qx, nbx, a.local_range, a.border, &xlo, &xhi);
    select_row(a, sc + (size_t)ro * a.row_stride, bh * nq + (size_t)tq * nS + qy * nbx + qx, nvis,
               ylo, yhi - ylo + 1, xlo, xhi, n_keys, hist, lane, sqrt((double)D));
  }
}

template <int D>
hipError_t launch_tile(const DraftArgs& a, hipStream_t s) {
  const long long tasks = (long long)a.B * a.NH * a.ntb_q * ((a.nby + 3) / 4) * ((a.nbx + 3) / 4);
  const long long wgs = 8 * ((tasks + 7) / 8);
  constexpr size_t kAux = (size_t)D * 16 * sizeof(double) > kTileWaves * 256 * 4
                             ? (size_t)D * 16 * sizeof(double)
                             : kTileWaves * 256 * 4;
  const size_t shmem = 16 * (size_t)a.row_stride * sizeof(double) + kAux;
  if (shmem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)draft_tile_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(draft_tile_kernel<D>, dim3((unsigned)wgs), dim3(64 * kTileWaves), shmem, s, a);
  return hipGetLastError();
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

hipError_t launch_draft_mask(const DraftArgs& a, hipStream_t s) {
  // The tile path pays where 4 x 4 neighbouring rows share most of a window
  // that is smaller than the grid, or where its tiles alone fill the chip.
  // A window spanning a small grid gives every row of a temporal block the
  // same candidates and few tiles; there the row-group path's many small
  // workgroups fill the chip better (768x1408 step: 24 vs 33 us; a 12-TB
  // chunk of the same grid has 864 tiles and keeps the tile path).
  const bool window_inside = a.local_range < a.nby || a.local_range < a.nbx;
  const long long tiles =
      (long long)a.B * a.NH * a.ntb_q * ((a.nby + 3) / 4) * ((a.nbx + 3) / 4);
  if (a.row_stride <= kTileMaxCand && (window_inside || tiles >= 512))
    return a.D == 64 ? launch_tile<64>(a, s) : launch_tile<128>(a, s);
  return a.D == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace lcsa
