// Backward of the block-sparse attention: dQ, dK, dV over the same lists.
//
// [FN] "FlashVSR" note, Key design 2 computes full 128 x 128 attention on
// the selected block pairs only; Key design 1 trains the student on all
// frames of a clip in parallel under the block-sparse causal mask. The
// selection is a discrete choice and is held fixed: the gradient is that of
// softmax attention over the listed blocks. Per query block i with listed
// keys (rows of their blocks):
//   P = exp(scale Q K^T - lse)       (the forward's log-sum-exp)
//   dV += P^T dO     dP = dO V^T     dS = P * (dP - delta),  delta = rowsum(dO * O)
//   dQ = scale dS K  dK += scale dS^T Q
// This is the training-shape backward: keys are the chunk's own blocks, and
// q, k, v, O, dO and the gradients are in the token layout.
//
// Four kernels, all bf16 on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16,
// float32 accumulation):
//  * prep:  per (block, head) lse * log2(e) and delta, into the workspace;
//  * inverse lists: for each key block, the query blocks whose list holds
//           it, ascending (binary search in the sorted lists, wave ballot),
//           so dK / dV need no atomics and are deterministic;
//  * dQ:    one workgroup per query block, walking its list;
//           S^T = K Q^T and dP^T = V dO^T (A = K, V rows from LDS, B = Q, dO
//           rows in registers), then dQ^T += K^T dS^T (A = K^T fragments by
//           transposing LDS reads of the same K rows, B = dS^T straight from
//           the accumulators);
//  * dK/dV: one workgroup per key block, walking its inverse list;
//           S = Q K^T and dP = dO V^T (A = Q, dO rows from LDS, B = K, V rows
//           in registers), then dV^T += dO^T P and dK^T += Q^T dS (A = dO^T,
//           Q^T fragments by transposing reads of the same row tiles, B = P,
//           dS from the accumulators).
// Only row tiles travel from memory: the transposed operands come from
// gfx950's ds_read_b64_tr_b16, so no transposed copy of q, k or dO exists.
// As in the forward, the rows of the first products' A operands are read in
// a permuted order so that each lane's accumulator values form the 8
// contiguous k-elements of the next product's B fragment. Tiles are staged
// in 32-row quarters, double-buffered in LDS with direct global->LDS loads,
// and rows are XOR-swizzled in 16-byte chunks (conflict-free fragment and
// transposing reads).
#include "lcsa_kernels.h"
#include "lds_transpose.h"
#include "mfma_tiles.h"

namespace lcsa {
namespace {

template <int D>
struct Q4 {                                   // one 32-row quarter of a block
  static constexpr int ROWB = 32 * D * 2;     // [32][D] row tile bytes
  static constexpr int KCH = D / 8;           // 16-byte chunks per row
  static constexpr int NS = D / 16;           // k-steps over D
  static constexpr int NO = D / 32;           // 32-row tiles over D
  static constexpr int RLD = ROWB / 4096;     // 1 KB loads per wave for a row tile
};

// Geometry of a chunk-relative block n and its token tau in the token layout.
struct Tok {
  int T, H, W, NH, D, nbx, nS;
  uint32_t qspan;  // bytes from a quarter's first token past its last unit
  // bytes from a block's first token to the first token of its quarter qq
  // (rows 32qq .. 32qq + 31: frame qq / 2, token rows 4 (qq % 2) ..)
  __device__ size_t quarter_bytes(int qq) const {
    return ((size_t)(qq >> 1) * H * W + (size_t)(qq & 1) * 4 * W) * NH * D * 2;
  }
  __device__ size_t off(int b, int h, int n, int tau) const {
    const int bt = n / nS, s = n - bt * nS, by = s / nbx, bx = s - by * nbx;
    const int t = 2 * bt + (tau >> 6), y = 8 * by + ((tau >> 3) & 7), x = 8 * bx + (tau & 7);
    return ((((size_t)b * T + t) * H + y) * W + x) * NH * D + (size_t)h * D;
  }
};

__device__ inline Tok make_tok(const BwdArgs& a) {
  Tok t;
  t.T = a.T;
  t.H = a.H;
  t.W = a.W;
  t.NH = a.NH;
  t.D = a.D;
  t.nbx = a.W / 8;
  t.nS = (a.H / 8) * t.nbx;
  // a quarter's rows lie in 4 token rows of one frame: its last 16-byte unit
  // ends before token 3W + 8 (offsets checked against 32 bits on the host)
  t.qspan = (uint32_t)((size_t)(3 * a.W + 8) * a.NH * a.D * 2);
  return t;
}

// Offsets, in bytes from its block's first token, of this lane's 16-byte
// units of quarter 0 of a [32][D] row tile (token layout source, swizzled
// LDS destination: unit u of wave instruction it lands at +16 u). Quarter qq
// adds (qq / 2) frames and 4 (qq % 2) token rows: Tok::quarter_bytes.
template <int D>
__device__ inline void row_unit_offsets(const Tok& tk, int w, int lane,
                                        uint32_t (&off)[Q4<D>::RLD]) {
  using G = Q4<D>;
#pragma unroll
  for (int it = 0; it < G::RLD; ++it) {
    const int u = (it * 4 + w) * 64 + lane;
    const int row = u / G::KCH, c = swz_t<D>(row, u % G::KCH);
    const size_t tok = ((size_t)((row >> 3) & 7) * tk.W + (row & 7)) * tk.NH * tk.D;
    off[it] = (uint32_t)((tok + c * 8) * 2);
  }
}

// A fragments of the transposed products (dV^T += dO^T P, dK^T += Q^T dS,
// dQ^T += K^T dS^T) come straight from the row tiles in LDS by transposing
// reads (lds_transpose.h); the row tiles use its swizzle swz_t.

// Issue the direct loads of one quarter's row tile (block base + per-lane
// offsets). Buffer loads: the scalar resource holds the tile's base and
// extent, the lane offset is the vector offset, so the loads need no vector
// address arithmetic.
template <int D>
__device__ __forceinline__ void load_rows(const char* qblk, uint32_t span, const uint32_t* off,
                                          char* dst, int w) {  // qblk: the quarter's first token
  const __amdgpu_buffer_rsrc_t r = raw_rsrc(qblk, span);
#pragma unroll
  for (int it = 0; it < Q4<D>::RLD; ++it)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(dst + (it * 4 + w) * 1024), 16, off[it], 0,
                                             0, 0);
}

// Issue the loads of quarter qq of one key block for the dQ kernel: K rows
// and V rows.
template <int D>
__device__ __forceinline__ void issue_dq(const Tok& tk, const char* kb, const char* vb,
                                         const uint32_t* roff, int qq, char* buf, int w) {
  using G = Q4<D>;
  const size_t qo = tk.quarter_bytes(qq);
  load_rows<D>(kb + qo, tk.qspan, roff, buf, w);
  load_rows<D>(vb + qo, tk.qspan, roff, buf + G::ROWB, w);
}

// Issue the loads of quarter qq of one query block for the dK/dV kernel: Q
// rows, dO rows, and (wave 0) the quarter's lse2 and
// delta values: lanes 0-7 fetch 32 lse2 values, lanes 8-15 the 32 delta
// values, the other lanes repeat them into the rest of a 1 KB region.
template <int D>
__device__ __forceinline__ void issue_dkdv(const Tok& tk, const char* qb, const char* ob,
                                           const char* lb, const uint32_t* roff, uint32_t loff,
                                           int qq, char* buf, int w) {
  using G = Q4<D>;
  const size_t qo = tk.quarter_bytes(qq);
  load_rows<D>(qb + qo, tk.qspan, roff, buf, w);
  load_rows<D>(ob + qo, tk.qspan, roff, buf + G::ROWB, w);
  if (w == 0)  // lb: the block's 256 floats (1 KB) of lse2 then delta
    __builtin_amdgcn_raw_ptr_buffer_load_lds(raw_rsrc(lb, 1024), LDS_PTR(buf + 2 * G::ROWB), 16,
                                             loff, 128 * qq, 0, 0);
}

// B fragments of 32 rows (this wave's rows 32w + l32) of block n: D values
// per row, 8 per k-step, straight into registers.
template <int D>
__device__ __forceinline__ void row_frags(const Tok& tk, const void* src, int b, int h, int n,
                                          int row, int g, bf16x8 (&f)[Q4<D>::NS]) {
  const __bf16* p = (const __bf16*)src + tk.off(b, h, n, row);
#pragma unroll
  for (int s = 0; s < Q4<D>::NS; ++s) f[s] = *reinterpret_cast<const bf16x8*>(p + 16 * s + 8 * g);
}

// Write a D x 32 accumulator (rows d, column = this lane's row 32w + l32)
// times `mul` to rows of block n in the token layout, through an LDS stage
// of [128][D] bf16 so the stores are whole 16-byte chunks of a row.
template <int D>
__device__ __forceinline__ void store_rows(const Tok& tk, void* dst, int b, int h, int n,
                                           const f32x16 (&acc)[Q4<D>::NO], float mul, char* st,
                                           int w, int l32, int g, int tid) {
  constexpr int NO = Q4<D>::NO, CH = D / 8;
  const int tau = 32 * w + l32;
#pragma unroll
  for (int dt = 0; dt < NO; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      __bf16 v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] = (__bf16)(acc[dt][4 * ii + j] * mul);
      const int c = 4 * dt + ii;  // chunk of d = 32dt + 8ii .. +8; this lane's half at +8g
      *reinterpret_cast<uint2*>(st + tau * (D * 2) + swz_row<D>(tau, c) * 16 + 8 * g) =
          *reinterpret_cast<const uint2*>(v4);
    }
  __syncthreads();
  uint16_t* o = (uint16_t*)dst;
#pragma unroll
  for (int e0 = 0; e0 < 128 * CH; e0 += 256) {
    const int e = e0 + tid, row = e / CH, c = e % CH;
    *reinterpret_cast<uint4*>(o + tk.off(b, h, n, row) + c * 8) =
        *reinterpret_cast<const uint4*>(st + row * (D * 2) + swz_row<D>(row, c) * 16);
  }
}

// ---------------------------------------------------------------- prep ----
// One workgroup per (block, head), heads fastest: lse * log2(e) and
// delta = rowsum(dO * O) of the block's 128 queries, into the workspace.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  constexpr int CPT = D / 8, ITERS = 128 * CPT / 256, TPI = 256 / CPT;
  const Tok tk = make_tok(a);
  const int nq = (a.T / 2) * tk.nS;
  const int h = blockIdx.x % a.NH, n = (blockIdx.x / a.NH) % nq, b = blockIdx.x / (a.NH * nq);
  const size_t blk = ((size_t)b * a.NH + h) * nq + n;
  const int tid = threadIdx.x, c = tid % CPT, tsub = tid / CPT;

  // each token's CPT chunks sit on CPT consecutive lanes
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const int tau = it * TPI + tsub;
    const size_t o = tk.off(b, h, n, tau) + c * 8;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>((const __bf16*)a.dout + o);
    const bf16x8 y = *reinterpret_cast<const bf16x8*>((const __bf16*)a.out + o);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf((float)x[e], (float)y[e], s);
#pragma unroll
    for (int m = 1; m < CPT; m <<= 1) s += __shfl_xor(s, m, 64);
    if (c == 0) {
      a.ld2[blk * 256 + tau] = a.lse[blk * 128 + tau] * kLog2e;
      a.ld2[blk * 256 + 128 + tau] = s;
    }
  }
}

// ------------------------------------------------------- inverse lists ----
// One wave per (b, h, key block j): scan the query rows in order, binary
// search j in each row's ascending list, compact the hits with a ballot.
__global__ __launch_bounds__(64) void inverse_lists_kernel(BwdArgs a) {
  const int nq = (a.T / 2) * (a.H / 8) * (a.W / 8);
  const int j = blockIdx.x % nq, bh = blockIdx.x / nq;
  const int lane = threadIdx.x;
  int base = 0;
  int32_t* dst = a.inv_idx + ((size_t)bh * nq + j) * nq;
  for (int i0 = 0; i0 < nq; i0 += 64) {
    const int i = i0 + lane;
    bool hit = false;
    if (i < nq) {
      const size_t row = (size_t)bh * nq + i;
      const int32_t* list = a.sel_idx + row * a.kmax;
      int lo = 0, hi = min(a.sel_cnt[row], a.kmax) - 1;
      while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const int v = list[mid];
        if (v == j) {
          hit = true;
          break;
        }
        if ((unsigned)v < (unsigned)j) lo = mid + 1;  // -1 never sits before a valid id
        else hi = mid - 1;
      }
    }
    const uint64_t m = __ballot(hit);
    if (hit) dst[base + __popcll(m & ((1ull << lane) - 1))] = i;
    base += __popcll(m);
  }
  if (lane == 0) a.inv_cnt[(size_t)bh * nq + j] = base;
}

// ------------------------------------------------------------------ dQ ----
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a) {
  using G = Q4<D>;
  constexpr int NS = G::NS, NO = G::NO;
  constexpr int BUF = 2 * G::ROWB;  // K rows, V rows
  __shared__ __attribute__((aligned(16))) char lds[2 * BUF > 128 * D * 2 ? 2 * BUF : 128 * D * 2];

  const Tok tk = make_tok(a);
  const int nS = tk.nS, nq = (a.T / 2) * nS, n_tasks = a.B * a.NH * nq;
  const int per = (n_tasks + 7) / 8;
  const int task = (blockIdx.x & 7) * per + (blockIdx.x >> 3);  // XCD-contiguous
  if (task >= n_tasks) return;
  const int r = task % nq, n_tb = a.T / 2;
  const int i = (n_tb - 1 - r / nS) * nS + r % nS;  // longest lists (latest TBs) first
  const int bh = task / nq, h = bh % a.NH, b = bh / a.NH;
  const size_t row = (size_t)bh * nq + i;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cnt = min(a.sel_cnt[row], a.kmax);
  const int32_t* list = a.sel_idx + row * a.kmax;

  f32x16 acc[NO];
#pragma unroll
  for (int t = 0; t < NO; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;

  if (cnt > 0) {
    bf16x8 qf[NS], of[NS];
    row_frags<D>(tk, a.q, b, h, i, 32 * w + l32, g, qf);
    row_frags<D>(tk, a.dout, b, h, i, 32 * w + l32, g, of);
    const float sl2 = a.scale * kLog2e;
    const float lse2 = a.ld2[row * 256 + 32 * w + l32];
    const float dlt = a.ld2[row * 256 + 128 + 32 * w + l32];
    const int prow = perm32(l32);
    uint32_t roff[G::RLD];
    row_unit_offsets<D>(tk, w, lane, roff);
    const TrOff<D> tro(lane);
    const char *kb = nullptr, *vb = nullptr;
    auto block = [&](int j) {  // an invalid id loads block 0 and is skipped
      j = (unsigned)j < (unsigned)nq ? j : 0;
      const size_t base = tk.off(b, h, j, 0) * 2;
      kb = (const char*)a.k + base;
      vb = (const char*)a.v + base;
    };
    auto issue = [&](int qq, char* buf) { issue_dq<D>(tk, kb, vb, roff, qq, buf, w); };
    auto compute = [&](const char* cur) {
      const char* kr = cur;
      const char* vr = cur + G::ROWB;
      // every product's A fragments are read from LDS right before it; the
      // co-resident workgroup covers that latency
      f32x16 st, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) st[e] = dp[e] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int off = prow * (D * 2) + swz_t<D>(prow, 2 * s + g) * 16;
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kr + off),
                                                     qf[s], st, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(vr + off),
                                                     of[s], dp, 0, 0, 0);
      }
      bf16x8 ds[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[e], sl2, -lse2));
        ds[e >> 3][e & 7] = (__bf16)(p * (dp[e] - dlt));
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int dt = 0; dt < NO; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(kr, tro, ks, dt), ds[ks],
                                                            acc[dt], 0, 0, 0);
    };
    char* buf0 = lds;
    char* buf1 = lds + BUF;
    block(list[0]);
    issue(0, buf0);
    for (int n = 0; n < cnt; ++n) {
      const bool ok = (unsigned)list[n] < (unsigned)nq;  // uniform: skipped id
      // quarter qq of block n sits in buffer qq & 1; the next quarter is in flight
      wait_vm_all();
      __syncthreads();
      issue(1, buf1);
      if (ok) compute(buf0);
      wait_vm_all();
      __syncthreads();
      issue(2, buf0);
      if (ok) compute(buf1);
      wait_vm_all();
      __syncthreads();
      issue(3, buf1);
      if (ok) compute(buf0);
      wait_vm_all();
      __syncthreads();
      if (n + 1 < cnt) {
        block(list[n + 1]);
        issue(0, buf0);
      }
      if (ok) compute(buf1);
    }
  }
  __syncthreads();
  store_rows<D>(tk, a.dq, b, h, i, acc, a.scale, lds, w, l32, g, tid);
}

// --------------------------------------------------------------- dK / dV ----
// Two workgroups per CU (256 registers per lane, 34 KB of LDS each): the
// fragments of every product are read from LDS right before it, and the
// co-resident workgroup covers that latency. Quarter buffers are
// double-buffered in LDS (a deeper prefetch measured no faster).
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a) {
  using G = Q4<D>;
  constexpr int NS = G::NS, NO = G::NO;
  // Q rows, dO rows, then 1 KB for lse2 / delta
  constexpr int BUF = 2 * G::ROWB + 1024;
  __shared__ __attribute__((aligned(16))) char lds[2 * BUF > 128 * D * 2 ? 2 * BUF : 128 * D * 2];

  const Tok tk = make_tok(a);
  const int nS = tk.nS, nq = (a.T / 2) * nS, n_tasks = a.B * a.NH * nq;
  const int per = (n_tasks + 7) / 8;
  const int task = (blockIdx.x & 7) * per + (blockIdx.x >> 3);  // XCD-contiguous
  if (task >= n_tasks) return;
  const int j = task % nq;  // key TBs ascending: the earliest keys have the longest lists
  const int bh = task / nq, h = bh % a.NH, b = bh / a.NH;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const size_t kj = (size_t)bh * nq + j;
  const int cnt = min(a.inv_cnt[kj], nq);
  // read through the constant address space: scalar loads, counted by
  // lgkmcnt, so fetching the next entry never waits for the tile prefetches
  const __attribute__((address_space(4))) int32_t* inv =
      (const __attribute__((address_space(4))) int32_t*)(a.inv_idx + kj * nq);

  f32x16 dk[NO], dv[NO];
#pragma unroll
  for (int t = 0; t < NO; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[t][e] = dv[t][e] = 0.f;

  if (cnt > 0) {
    bf16x8 kf[NS], vf[NS];
    row_frags<D>(tk, a.k, b, h, j, 32 * w + l32, g, kf);
    row_frags<D>(tk, a.v, b, h, j, 32 * w + l32, g, vf);
    const float sl2 = a.scale * kLog2e;
    const int prow = perm32(l32);
    uint32_t roff[G::RLD];
    row_unit_offsets<D>(tk, w, lane, roff);
    const TrOff<D> tro(lane);
    const uint32_t loff = 16 * (lane & 7) + ((lane & 8) ? 512 : 0);
    struct Src {
      const char *q, *o, *l;
    };
    auto source = [&](int i) {
      const size_t base = tk.off(b, h, i, 0) * 2;
      const size_t qrow = (size_t)bh * nq + i;
      return Src{(const char*)a.q + base, (const char*)a.dout + base,
                 (const char*)(a.ld2 + qrow * 256)};
    };
    auto issue = [&](const Src& p, int qq, char* buf) {
      issue_dkdv<D>(tk, p.q, p.o, p.l, roff, loff, qq, buf, w);
    };
    auto compute = [&](const char* cur) {
      const char* qr = cur;
      const char* orr = cur + G::ROWB;
      const float* ld = (const float*)(cur + 2 * G::ROWB);  // [0, 32) lse2, [32, 64) delta
      // every product's A fragments are read from LDS right before it
      f32x16 st, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) st[e] = dp[e] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int off = prow * (D * 2) + swz_t<D>(prow, 2 * s + g) * 16;
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(qr + off),
                                                     kf[s], st, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(orr + off),
                                                     vf[s], dp, 0, 0, 0);
      }
      // element 8ks + e of the accumulators is query 16ks + 8g + e of the quarter
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int q = 16 * ks + 8 * g;
        bf16x8 pb, dsb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(st[8 * ks + e], sl2, -ld[q + e]));
          pb[e] = (__bf16)p;
          dsb[e] = (__bf16)(p * (dp[8 * ks + e] - ld[32 + q + e]));
        }
#pragma unroll
        for (int dt = 0; dt < NO; ++dt) {
          dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(orr, tro, ks, dt), pb,
                                                           dv[dt], 0, 0, 0);
          dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(qr, tro, ks, dt), dsb,
                                                           dk[dt], 0, 0, 0);
        }
      }
    };
    // quarter qq of query block n sits in buffer qq & 1; the next is in flight
    char* buf0 = lds;
    char* buf1 = lds + BUF;
    Src cur = source(inv[0]);
    issue(cur, 0, buf0);
    for (int n = 0; n < cnt; ++n) {
      wait_vm_all();
      __syncthreads();
      issue(cur, 1, buf1);
      compute(buf0);
      wait_vm_all();
      __syncthreads();
      issue(cur, 2, buf0);
      compute(buf1);
      wait_vm_all();
      __syncthreads();
      issue(cur, 3, buf1);
      compute(buf0);
      wait_vm_all();
      __syncthreads();
      if (n + 1 < cnt) {
        cur = source(inv[n + 1]);
        issue(cur, 0, buf0);
      }
      compute(buf1);
    }
  }
  __syncthreads();
  store_rows<D>(tk, a.dk, b, h, j, dk, a.scale, lds, w, l32, g, tid);
  __syncthreads();
  store_rows<D>(tk, a.dv, b, h, j, dv, 1.f, lds, w, l32, g, tid);
}

template <int D>
hipError_t launch(const BwdArgs& a, hipStream_t s) {
  const long long nq = (long long)(a.T / 2) * (a.H / 8) * (a.W / 8);
  const long long tasks = (long long)a.B * a.NH * nq;
  const long long grid = 8 * ((tasks + 7) / 8);
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)tasks), dim3(256), 0, s, a);
  hipLaunchKernelGGL(inverse_lists_kernel, dim3((unsigned)tasks), dim3(64), 0, s, a);
  hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)grid), dim3(256), 0, s, a);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(const BwdArgs& a, hipStream_t s) {
  return a.D == 64 ? launch<64>(a, s) : launch<128>(a, s);
}

}  // namespace lcsa
