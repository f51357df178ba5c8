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

// The view's ring slots, copied to LDS at kernel start. The keys of one
// wave can lie in different temporal blocks, and a per-lane index into the
// kernel-argument array compiles to a vector load from argument memory
// followed by a wait on every outstanding load (which serialised the key
// prefetch); a ds_read of this table costs neither. Needs a barrier before
// the first read.
__device__ inline void stage_slots(const RingView& v, int32_t* tab) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < LCSA_MAX_SLOTS; ++i)
    if (tid == i) tab[i] = v.slot[i];
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

// Register form of select_row, for rows of at most kRegCand candidates when
// no probabilities are asked for. Lane l holds the candidates
// [l M, l M + M) (M = ceil(n / 64)) of the row's float64 scores in
// registers, so each refinement level is one pass over registers rather
// than over LDS, and the kept ids go to their places through prefix sums of
// per-lane counts (candidate order = ascending logical id), with no ballot
// per 64 candidates. Same result as select_row: the k largest scores,
// equal scores taken lowest index first.
constexpr int kRegM = 8;
constexpr int kRegCand = 64 * kRegM;

__device__ void select_row_regs(const DraftArgs& a, const double* s, size_t row, int nvis,
                                int ylo, int ny, int gxlo, int gxhi, int64_t n_keys,
                                uint32_t* hist, int lane) {
  const int nbx = a.nbx, nS = a.nby * nbx;
  const int nx = gxhi - gxlo + 1;
  const int n = nvis * ny * nx;
  const int k = topk_dev(a, n, n_keys);
  int32_t* out = a.sel_idx + row * a.kmax;
  const int M = (n + 63) >> 6;
  const int cbase = lane * M;
  double v[kRegM];
  uint32_t valid = 0;
  double lo = INFINITY, hi = -INFINITY;
#pragma unroll
  for (int m = 0; m < kRegM; ++m) {
    const bool in_row = m < M && cbase + m < n;
    v[m] = s[in_row ? cbase + m : 0];
    if (in_row && v[m] == v[m]) {  // NaN scores are never kept
      valid |= 1u << m;
      lo = fmin(lo, v[m]);
      hi = fmax(hi, v[m]);
    }
  }
  lo = wave_min_dpp(lo);
  hi = wave_max_dpp(hi);
  const int n_valid = __builtin_amdgcn_readlane((int)wave_prefix_sum_dpp(__popc(valid)), 63);
  uint32_t taken = 0, in = 0;  // in: undecided candidates, all in [lo, hi]
  int kr = 0;
  if (k >= n_valid) {
    taken = valid;
  } else if (k > 0) {
    in = valid;
    kr = k;
    for (int level = 0; level <= n && lo < hi; ++level) {
      const double scale = 256.0 / (hi - lo);
      auto bin_of = [&](double x) {
        const int b = (int)((x - lo) * scale);
        return b < 0 ? 0 : (b > 255 ? 255 : b);
      };
#pragma unroll
      for (int q = 0; q < 4; ++q) hist[lane * 4 + q] = 0u;
      wave_sync();
#pragma unroll
      for (int m = 0; m < kRegM; ++m)
        if ((in >> m) & 1u) atomicAdd(&hist[255 - bin_of(v[m])], 1u);  // position 0: top bin
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
      if (bal == 0) break;  // unreachable: 1 <= kr < candidates in range
      const int src = __ffsll((long long)bal) - 1;
      const int bin = __builtin_amdgcn_readlane(found, src);
      kr -= __builtin_amdgcn_readlane((int)fa, src);
      const int cb = __builtin_amdgcn_readlane((int)fc, src);
      // above the bin: kept; below: dropped; in it: the new range
      double nlo = INFINITY, nhi = -INFINITY;
#pragma unroll
      for (int m = 0; m < kRegM; ++m) {
        if ((in >> m) & 1u) {
          const int bn = bin_of(v[m]);
          if (bn > bin) {
            taken |= 1u << m;
            in &= ~(1u << m);
          } else if (bn < bin) {
            in &= ~(1u << m);
          } else {
            nlo = fmin(nlo, v[m]);
            nhi = fmax(nhi, v[m]);
          }
        }
      }
      lo = wave_min_dpp(nlo);
      hi = wave_max_dpp(nhi);
      if (cb == kr) {  // the whole bin is kept
        taken |= in;
        in = 0;
        kr = 0;
        break;
      }
    }
    // the undecided candidates now share one value: the first kr of them
    // in candidate order are kept
    const int pe = __popc(in);
    int e = (int)wave_prefix_sum_dpp((uint32_t)pe) - pe;
    for (uint32_t t = in; t; t &= t - 1, ++e)
      if (e < kr) taken |= t & (~t + 1u);
  }
  // emit in ascending candidate order
  const int pt = __popc(taken);
  const int incl = (int)wave_prefix_sum_dpp((uint32_t)pt);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  int pos = incl - pt;
  const SmallDiv div_nx(nx), div_ny(ny);
  for (uint32_t t = taken; t; t &= t - 1, ++pos) {
    if (pos < k) {
      const int c = cbase + __builtin_ctz(t);
      const int r3 = div_nx(c), xx = c - r3 * nx;
      const int p = div_ny(r3), yy = r3 - p * ny;
      out[pos] = p * nS + (ylo + yy) * nbx + gxlo + xx;
    }
  }
  const int cnt = total < k ? total : k;
  for (int q = cnt + lane; q < a.kmax; q += 64) out[q] = -1;
  if (lane == 0) a.sel_cnt[row] = cnt;
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
  if (!a.probs && n <= kRegCand) {
    select_row_regs(a, s, row, nvis, ylo, ny, gxlo, gxhi, n_keys, hist, lane);
    return;
  }
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

  __shared__ int32_t slot_tab[LCSA_MAX_SLOTS];
  stage_slots(a.view, slot_tab);
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
    return a.kpool_ring + (bh * a.n_slots + slot_tab[p]) * (size_t)D * nS + (size_t)y * nbx + x;
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
constexpr int kDenseMaxCand = 2304;          // candidates per row held in LDS
constexpr int kDenseMinCand = 1024;          // below this the row-group path is faster
constexpr int kHistStride = 264;             // per-wave histogram / list, 8 spare entries

// Order-preserving maps of float32 / float64 to unsigned integers.
__device__ inline uint32_t ordered_key(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline uint64_t ordered_key(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  return (u >> 63) ? ~u : (u | (1ull << 63));
}

template <int CTRL, int ROWS>
__device__ inline uint32_t dpp_keep32(uint32_t v) {  // lanes outside ROWS keep their value
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false);
}

// Full-wave min / max of unsigned keys and floats (the same DPP steps as the
// float64 reductions above; the result is read from lane 63).
__device__ inline uint32_t wave_min_u(uint32_t v) {
  v = min(v, dpp_keep32<0xB1, 0xF>(v));
  v = min(v, dpp_keep32<0x4E, 0xF>(v));
  v = min(v, dpp_keep32<0x141, 0xF>(v));
  v = min(v, dpp_keep32<0x140, 0xF>(v));
  v = min(v, dpp_keep32<0x142, 0xA>(v));
  v = min(v, dpp_keep32<0x143, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ inline uint32_t wave_max_u(uint32_t v) {
  v = max(v, dpp_keep32<0xB1, 0xF>(v));
  v = max(v, dpp_keep32<0x4E, 0xF>(v));
  v = max(v, dpp_keep32<0x141, 0xF>(v));
  v = max(v, dpp_keep32<0x140, 0xF>(v));
  v = max(v, dpp_keep32<0x142, 0xA>(v));
  v = max(v, dpp_keep32<0x143, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ inline int wave_sum_i(int v) {
  return __builtin_amdgcn_readlane((int)wave_prefix_sum_dpp((uint32_t)v), 63);
}

// Exact top-kr over the keys ks[lane + 64 m] (in LDS) of the slots m set in
// `in`, restricted to [klo, khi]. On return the keys above khi are taken,
// and of those in [klo, khi] (n_in of them) the first kr in candidate order;
// either kr == n_in (all taken) or klo == khi (one value). Radix steps of 8
// bits starting below the highest bit where the range's smallest and
// largest keys differ, so the first histogram already spreads over the
// occupied range; every step fixes at least 8 more bits.
__device__ void narrow_range(const uint32_t* ks, int n, uint64_t in, uint32_t& klo, uint32_t& khi,
                             int& kr, int& n_in, uint32_t* hist, int lane) {
  n_in = 0;
  for (int level = 0; level < 6; ++level) {
    uint32_t mn = ~0u, mx = 0u;
    int cnt = 0;
    for (int m = 0; 64 * m < n; ++m) {
      const uint32_t kv = ks[lane + 64 * m];
      if (((in >> m) & 1u) && kv >= klo && kv <= khi) {
        mn = min(mn, kv);
        mx = max(mx, kv);
        ++cnt;
      }
    }
    mn = wave_min_u(mn);
    mx = wave_max_u(mx);
    cnt = wave_sum_i(cnt);
    n_in = cnt;
    if (cnt == 0) return;
    klo = mn;
    khi = mx;
    if (cnt <= kr) {
      kr = cnt;
      return;
    }
    if (mn == mx) return;
    const int top = 32 - __builtin_clz(mn ^ mx);
    const int shift = top > 8 ? top - 8 : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[lane * 4 + q] = 0u;
    wave_sync();
    for (int m = 0; 64 * m < n; ++m) {
      const uint32_t kv = ks[lane + 64 * m];
      if (((in >> m) & 1u) && kv >= klo && kv <= khi)
        atomicAdd(&hist[255 - (int)((kv >> shift) & 255u)], 1u);  // position 0: top digit
    }
    wave_sync();
    uint32_t hb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) hb[q] = hist[lane * 4 + q];
    const uint32_t tot = hb[0] + hb[1] + hb[2] + hb[3];
    uint32_t ab = wave_prefix_sum_dpp(tot) - tot;  // keys in higher digits
    int found = -1;
    uint32_t fa = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (found < 0 && ab < (uint32_t)kr && ab + hb[q] >= (uint32_t)kr) {
        found = 255 - (lane * 4 + q);
        fa = ab;
      }
      ab += hb[q];
    }
    const uint64_t bal = __ballot(found >= 0);
    wave_sync();
    if (bal == 0) return;  // unreachable: 1 <= kr < cnt
    const int src = __ffsll((long long)bal) - 1;
    const uint32_t digit = (uint32_t)__builtin_amdgcn_readlane(found, src);
    kr -= __builtin_amdgcn_readlane((int)fa, src);
    const uint32_t above = shift + 8 >= 32 ? 0u : (~0u << (shift + 8));
    klo = (mn & above) | (digit << shift);
    khi = klo | ((1u << shift) - 1u);
  }
}

// float64 score of candidate c (key id) against the pooled query qrow, in
// one fixed summation order.
template <int D>
__device__ inline double dense_score64(const DraftArgs& a, const int32_t* slot_tab,
                                       const double* qrow, size_t bh, int nS,
                                       const SmallDiv& div_ns, int c) {
  const int p = div_ns(c), sp = c - p * nS;
  const double* kp = a.kpool_ring + (bh * a.n_slots + slot_tab[p]) * (size_t)D * nS + sp;
  double w = 0.0;
#pragma unroll 4
  for (int d = 0; d < D; ++d) w = fma(qrow[d], kp[(size_t)d * nS], w);
  return w;
}

// One wave, general form: top-k and the sorted index list of query row `row`
// from its n float32 scores in LDS (candidate index = key id), which the
// selection overwrites with its 32-bit keys. It runs in stages: the float32 score,
// then, only for candidates tied at the k-th place, the high and the low
// half of the float64 score (recomputed from the pooled query qrow and the
// pooled ring); candidates still tied after that are exact ties and go to
// the lower id.
template <int D>
__device__ void select_dense_staged(const DraftArgs& a, const int32_t* slot_tab, float* s, int n,
                                    size_t row, size_t bh, int nS, int64_t n_keys,
                                    const double* qrow, uint32_t* hist, int lane) {
  const int k = topk_dev(a, n, n_keys);
  int32_t* out = a.sel_idx + row * a.kmax;
  uint32_t* ks = reinterpret_cast<uint32_t*>(s);
  uint64_t live = 0;  // bit m: slot m is still undecided (non-NaN candidate)
  for (int m = 0; 64 * m < n; ++m) {
    const int c = lane + 64 * m;
    if (c < n) {
      const float v = s[c];
      ks[c] = ordered_key(v);
      if (!__builtin_isnan(v)) live |= 1ull << m;
    }
  }
  uint64_t taken = 0;  // bit m: slot m is selected
  int kr = k;
  const SmallDiv div_ns(nS);
  for (int stage = 0; stage < 3 && kr > 0; ++stage) {
    if (stage > 0) {  // the next finer key of the tied candidates
      for (int m = 0; 64 * m < n; ++m) {
        if ((live >> m) & 1u) {
          const int c = lane + 64 * m;
          const double w = dense_score64<D>(a, slot_tab, qrow, bh, nS, div_ns, c);
          const uint64_t k64 = ordered_key(w);
          ks[c] = stage == 1 ? (uint32_t)(k64 >> 32) : (uint32_t)k64;
          if (__builtin_isnan(w)) live &= ~(1ull << m);
        }
      }
    }
    wave_sync();
    uint32_t lo = 0, hi = ~0u;
    int n_in = 0;
    narrow_range(ks, n, live, lo, hi, kr, n_in, hist, lane);
    uint64_t in_range = 0;
    for (int m = 0; 64 * m < n; ++m) {
      if ((live >> m) & 1u) {
        const uint32_t kv = ks[lane + 64 * m];
        if (kv > hi) taken |= 1ull << m;
        else if (kv >= lo) in_range |= 1ull << m;
      }
    }
    live = in_range;
    if (n_in <= kr) {  // the whole range is kept
      taken |= live;
      live = 0;
      kr = 0;
    }
  }
  // Emit in ascending candidate order: the taken ones, then the first kr of
  // the exact ties left in `live`.
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int eq_before = 0, sel_before = 0;
  if (k > 0) {
    for (int m = 0; 64 * m < n; ++m) {
      const bool gt = (taken >> m) & 1u;
      const bool eq = (live >> m) & 1u;
      const uint64_t beq = __ballot(eq);
      const int r = eq_before + __popcll(beq & lt_mask);
      const bool want = gt || (eq && r < kr);
      const int pos = sel_before + __popcll(__ballot(want) & lt_mask);
      const bool sel = want && pos < k;  // never more than k
      const uint64_t bsel = __ballot(sel);
      if (sel) out[pos] = lane + 64 * m;
      eq_before += __popcll(beq);
      sel_before += __popcll(bsel);
    }
  }
  for (int pos = sel_before + lane; pos < a.kmax; pos += 64) out[pos] = -1;
  if (lane == 0) a.sel_cnt[row] = sel_before;
}

__device__ inline float wave_min_f32(float v) {
  v = fminf(v, __uint_as_float(dpp_keep32<0xB1, 0xF>(__float_as_uint(v))));
  v = fminf(v, __uint_as_float(dpp_keep32<0x4E, 0xF>(__float_as_uint(v))));
  v = fminf(v, __uint_as_float(dpp_keep32<0x141, 0xF>(__float_as_uint(v))));
  v = fminf(v, __uint_as_float(dpp_keep32<0x140, 0xF>(__float_as_uint(v))));
  v = fminf(v, __uint_as_float(dpp_keep32<0x142, 0xA>(__float_as_uint(v))));
  v = fminf(v, __uint_as_float(dpp_keep32<0x143, 0xC>(__float_as_uint(v))));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}
__device__ inline float wave_max_f32(float v) {
  v = fmaxf(v, __uint_as_float(dpp_keep32<0xB1, 0xF>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_keep32<0x4E, 0xF>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_keep32<0x141, 0xF>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_keep32<0x140, 0xF>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_keep32<0x142, 0xA>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_keep32<0x143, 0xC>(__float_as_uint(v))));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}

constexpr int kDenseM = (kDenseMaxCand + 63) / 64;  // scores per lane in registers
constexpr int kBoundaryMax = 256;                   // boundary-bin members ranked pairwise

// Bin of x among 256 equal bins over [mn, mn + 256 / scale]: a monotone map
// of the value, so every score in a higher bin is larger.
__device__ __forceinline__ int bin256(float x, float mn, float scale) {
  const int b = (int)((x - mn) * scale);
  return b < 0 ? 0 : (b > 255 ? 255 : b);
}

// One wave: the 256-bin histogram of the scores v[m] of the slots set in
// `valid` (position 0 is the top bin; slots without a candidate count into
// spare entries past the histogram, so there is no branch per slot), and
// the bin holding the k-th largest score: bstar, the candidates still to
// take inside it (kr) and its size (cb). False when no bin holds it (only
// with NaN scores). The histogram's memory is free again on return.
template <int M>
__device__ __forceinline__ bool boundary_bin(const float (&v)[M], uint64_t valid, float mn,
                                             float scale, int k, uint32_t* hist, int lane,
                                             int& bstar, int& kr, int& cb) {
#pragma unroll
  for (int q = 0; q < 4; ++q) hist[lane * 4 + q] = 0u;
  wave_sync();
#pragma unroll
  for (int m = 0; m < M; ++m)
    atomicAdd(&hist[((valid >> m) & 1u) ? 255 - bin256(v[m], mn, scale) : 256 + (lane & 7)], 1u);
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
    if (found < 0 && ab < (uint32_t)k && ab + hb[q] >= (uint32_t)k) {
      found = 255 - (lane * 4 + q);
      fa = ab;
      fc = hb[q];
    }
    ab += hb[q];
  }
  const uint64_t bal = __ballot(found >= 0);
  wave_sync();  // every lane has read the histogram
  const int src = bal ? __ffsll((long long)bal) - 1 : 0;
  bstar = __builtin_amdgcn_readlane(found, src);
  kr = k - __builtin_amdgcn_readlane((int)fa, src);
  cb = __builtin_amdgcn_readlane((int)fc, src);
  return bal != 0;
}

// One wave: the cb boundary-bin members, scores s[i] and candidate ids
// ids[i] (ascending), ranked by larger score, then equal score of lower id;
// the members ranked below kr get the taken flag (top bit of ids[i]). True
// when a float32 tie group straddles the kr-th place (then the float64
// scores must decide).
__device__ __forceinline__ bool rank_members(const float* s, uint32_t* ids, int cb, int kr,
                                             int lane) {
  bool straddle = false;
  for (int i = lane; i < cb; i += 64) {
    const float vi = s[i];
    const uint32_t ci = ids[i] & 0x7fffffffu;
    int gt = 0, eq_lo = 0, eq = 0;
    for (int j = 0; j < cb; ++j) {  // ids of earlier rounds may carry the taken flag
      const float vj = s[j];
      gt += vj > vi;
      eq += vj == vi;
      eq_lo += (vj == vi) & ((ids[j] & 0x7fffffffu) < ci);
    }
    // a float32 tie group [gt, gt + eq) cut by the k-th place
    straddle |= gt < kr && gt + eq > kr;
    if (gt + eq_lo < kr) ids[i] = ci | 0x80000000u;  // taken
  }
  return __ballot(straddle) != 0;
}

// One wave, usual case: the row's float32 scores in registers, one 256-bin
// histogram over [min, max] (bins are a monotone function of the value),
// every candidate in a bin above the k-th one's bin taken, and the members
// of that boundary bin ranked pairwise (score descending, id ascending).
// Falls back to select_dense_staged when the boundary bin is large or a
// float32 tie straddles the k-th place (then the float64 scores decide).
// v[m]: the score of candidate lane + 64 m (any value past n); s: this
// wave's LDS row of at least n + 8 floats, scratch for the boundary list and
// the staged selection.
template <int D>
__device__ void select_dense(const DraftArgs& a, const int32_t* slot_tab, float* s,
                             const float (&v)[kDenseM], int n, size_t row, size_t bh, int nS,
                             int64_t n_keys, const double* qrow, uint32_t* hist, int lane) {
  constexpr int M = kDenseM;
  const int k = topk_dev(a, n, n_keys);
  int32_t* out = a.sel_idx + row * a.kmax;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t valid = 0;
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int c = lane + 64 * m;
    if (c < n && !__builtin_isnan(v[m])) {
      valid |= 1ull << m;
      mn = fminf(mn, v[m]);
      mx = fmaxf(mx, v[m]);
    }
  }
  mn = wave_min_f32(mn);
  mx = wave_max_f32(mx);
  const int n_valid = wave_sum_i(__popcll(valid));
  bool general = false;
  uint64_t taken = 0;
  if (k > 0 && k < n_valid) {
    const float scale = 256.f / (mx - mn);
    general = !(mx > mn) || !(scale < INFINITY);  // one value, or a range beyond float32
    int bstar = 0, kr = 0, cb = 0;
    if (!general) {
      auto bin_of = [&](float x) { return bin256(x, mn, scale); };
      general = !boundary_bin<M>(v, valid, mn, scale, k, hist, lane, bstar, kr, cb) ||
                cb > kBoundaryMax;
      if (!general) {
        // the boundary bin's members, in candidate order: scores over the
        // row's LDS scores (held in registers now), ids over the histogram
        uint32_t* ids = hist;
        int base = 0;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const bool onv = (valid >> m) & 1u;
          const int bn = bin_of(v[m]);
          if (onv && bn > bstar) taken |= 1ull << m;
          const bool inb = onv && bn == bstar;
          const uint64_t bb = __ballot(inb);
          // members go to their list position, the others to spare entries
          // (past the row's candidates, past the list)
          const int idx = base + __popcll(bb & lt_mask);
          s[inb ? idx : n + (lane & 7)] = v[m];
          ids[inb ? idx : 256 + (lane & 7)] = (uint32_t)(lane + 64 * m);
          base += __popcll(bb);
        }
        wave_sync();
        general = rank_members(s, ids, cb, kr, lane);
        wave_sync();
        if (!general) {
          base = 0;
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const bool inb = ((valid >> m) & 1u) && bin_of(v[m]) == bstar;
            const uint64_t bb = __ballot(inb);
            if (inb && (ids[base + __popcll(bb & lt_mask)] & 0x80000000u)) taken |= 1ull << m;
            base += __popcll(bb);
          }
        }
        wave_sync();
      }
    }
    if (general) {
      // restore the row's scores and settle it in stages
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int c = lane + 64 * m;
        if (c < n) s[c] = v[m];
      }
      wave_sync();
      select_dense_staged<D>(a, slot_tab, s, n, row, bh, nS, n_keys, qrow, hist, lane);
      return;
    }
  } else if (k > 0) {
    taken = valid;  // every candidate kept
  }
  // emit in ascending candidate order
  int sel_before = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const bool want = (taken >> m) & 1u;
    const uint64_t bw = __ballot(want);
    const int pos = sel_before + __popcll(bw & lt_mask);
    if (want && pos < k) out[pos] = lane + 64 * m;
    sel_before += __popcll(bw);
  }
  sel_before = sel_before < k ? sel_before : k;
  for (int pos = sel_before + lane; pos < a.kmax; pos += 64) out[pos] = -1;
  if (lane == 0) a.sel_cnt[row] = sel_before;
}

// One wave, split path: the same selection as select_dense, over the row's
// float32 scores in the workspace (src, ws_stride floats). Lane l holds the
// candidates [l M, l M + M) (M = ws_stride / 64: a multiple of four, at
// most kDenseM), so a per-lane count and one prefix sum over the lanes give
// every list position in candidate order: the boundary bin's members and
// the emitted ids go straight to their places, with no pass of ballots over
// the slots.
template <int D>
__device__ void select_split(const DraftArgs& a, const int32_t* slot_tab, const float* src,
                             float* s, int n, size_t row, size_t bh, int nS, int64_t n_keys,
                             const double* qrow, uint32_t* hist, int lane) {
  constexpr int MX = kDenseM;
  const int M = a.ws_stride >> 6;
  const int cbase = lane * M;
  const int k = topk_dev(a, n, n_keys);
  int32_t* out = a.sel_idx + row * a.kmax;
  // every load issued before the first wait; a slot past this lane's M
  // reads the row's first four scores and is never used
  float v[MX];
#pragma unroll
  for (int i = 0; i < MX / 4; ++i) {
    const float4 x = *reinterpret_cast<const float4*>(src + (4 * i < M ? cbase + 4 * i : 0));
    v[4 * i] = x.x;
    v[4 * i + 1] = x.y;
    v[4 * i + 2] = x.z;
    v[4 * i + 3] = x.w;
  }
  uint64_t valid = 0;
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int m = 0; m < MX; ++m) {
    if (m < M && cbase + m < n && !__builtin_isnan(v[m])) {
      valid |= 1ull << m;
      mn = fminf(mn, v[m]);
      mx = fmaxf(mx, v[m]);
    }
  }
  mn = wave_min_f32(mn);
  mx = wave_max_f32(mx);
  const int n_valid = wave_sum_i(__popcll(valid));
  uint64_t taken = 0;
  if (k > 0 && k < n_valid) {
    const float scale = 256.f / (mx - mn);
    bool general = !(mx > mn) || !(scale < INFINITY);  // one value, or a range beyond float32
    if (!general) {
      auto bin_of = [&](float x) { return bin256(x, mn, scale); };
      int bstar = 0, kr = 0, cb = 0;
      general = !boundary_bin<MX>(v, valid, mn, scale, k, hist, lane, bstar, kr, cb) ||
                cb > kBoundaryMax;
      if (!general) {
        uint64_t member = 0;
#pragma unroll
        for (int m = 0; m < MX; ++m) {
          if ((valid >> m) & 1u) {
            const int bn = bin_of(v[m]);
            if (bn > bstar) taken |= 1ull << m;
            else if (bn == bstar) member |= 1ull << m;
          }
        }
        if (cb == kr) {  // the whole boundary bin is kept
          taken |= member;
        } else {
          // the members, in candidate order: scores over this wave's LDS
          // row, ids over the histogram; each lane's run starts at its
          // exclusive prefix of the member counts
          uint32_t* ids = hist;
          const int pm = __popcll(member);
          const int mbase = (int)wave_prefix_sum_dpp((uint32_t)pm) - pm;
          int pos = mbase;
#pragma unroll
          for (int m = 0; m < MX; ++m) {
            if ((member >> m) & 1u) {
              s[pos] = v[m];
              ids[pos] = (uint32_t)(cbase + m);
              ++pos;
            }
          }
          wave_sync();
          general = rank_members(s, ids, cb, kr, lane);
          wave_sync();
          if (!general) {
            pos = mbase;
#pragma unroll
            for (int m = 0; m < MX; ++m) {
              if ((member >> m) & 1u) {
                if (ids[pos] & 0x80000000u) taken |= 1ull << m;
                ++pos;
              }
            }
          }
          wave_sync();
        }
      }
    }
    if (general) {
      // the row's scores into this wave's LDS row, settled in stages
#pragma unroll
      for (int m = 0; m < MX; ++m)
        if (m < M && cbase + m < n) s[cbase + m] = v[m];
      wave_sync();
      select_dense_staged<D>(a, slot_tab, s, n, row, bh, nS, n_keys, qrow, hist, lane);
      return;
    }
  } else if (k > 0) {
    taken = valid;  // every candidate kept
  }
  // emit in ascending candidate order: this lane's run starts at its
  // exclusive prefix of the taken counts
  const int pt = __popcll(taken);
  const int incl = (int)wave_prefix_sum_dpp((uint32_t)pt);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  int pos = incl - pt;
  for (uint64_t t = taken; t; t &= t - 1, ++pos)
    if (pos < k) out[pos] = cbase + __builtin_ctzll(t);
  const int cnt = total < k ? total : k;
  for (int p = cnt + lane; p < a.kmax; p += 64) out[p] = -1;
  if (lane == 0) a.sel_cnt[row] = cnt;
}

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
