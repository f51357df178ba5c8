// Step 5 of LCSA: exact attention over the selected block pairs.
//
// [FN] "FlashVSR" note, Key design 2: only the top-k block pairs of the
// coarse map get full 128 x 128 attention, computed with the original Q, K
// and V. [HW] "How FlashVSR works" 2.2: the operator skips unselected blocks
// outright rather than computing them and multiplying by zero.
//
// One workgroup owns one query block (128 tokens) of one (batch, head) and
// walks its index list; unlisted key blocks are never loaded. bf16 path:
// four waves, each owning 32 query rows, on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, float32 accumulation):
//   S^T = K Q^T     A = K rows from LDS, B = Q held in registers
//   O^T += V^T P^T  A = V^T from LDS,    B = P straight from the S^T
//                   accumulators (each lane owns one query column, so the
//                   row softmax needs one cross-lane exchange per block)
// with an online softmax in base 2 (exp2 of a log2e-prescaled logit).
// A key block is consumed in two 64-key halves. Each half (K [64][D] plus
// V^T [D][64], 32 KB at D = 128) goes straight from global memory into one
// of two LDS buffers (buffer loads into LDS, no register staging): while one
// half is computed the next one is in flight, so 64 KB of LDS per
// workgroup and two workgroups per CU. LDS rows are XOR-swizzled in
// 16-byte chunks so the fragment reads are bank-conflict free, and K rows
// are permuted inside each 32-key tile so the S^T accumulator rows come out
// in the key order of V^T's A fragments. The row max is a max3 tree plus
// one cross-half exchange (v_permlane32_swap); O is rescaled only when the
// running max grows by more than 2^8, and row sums use v_dot2 on the bf16
// probabilities actually multiplied into V.
// fp32 path (small validation workloads): one thread per query row on the
// vector ALU.
#include <type_traits>

#include "lcsa_kernels.h"
#include "mfma_tiles.h"

namespace lcsa {
namespace {

__device__ inline size_t out_offset(const AttnArgs& a, int b, int h, int i, int tau, int d) {
  const int nbx = a.W / 8, nS = (a.H / 8) * nbx;
  const int bt = i / nS, s = i % nS, by = s / nbx, bx = s % nbx;
  const int t = 2 * bt + (tau >> 6);
  const int y = 8 * by + ((tau >> 3) & 7);
  const int x = 8 * bx + (tau & 7);
  return ((((size_t)b * a.T + t) * a.H + y) * a.W + x) * a.NH * a.D + (size_t)h * a.D + d;
}

template <int D>
struct Tile {
  static constexpr int KEYS = 64;                  // keys per sub-tile
  static constexpr int KBYTES = KEYS * D * 2;      // K sub-tile  [64][D]
  static constexpr int VBYTES = D * KEYS * 2;      // V^T sub-tile [D][64]
  static constexpr int BUF = KBYTES + VBYTES;
  static constexpr int KCH = D / 8;                // 16-byte chunks per K row
  static constexpr int KLD = KBYTES / 1024 / 4;    // direct 1 KB loads per wave (K)
  static constexpr int VLD = VBYTES / 1024 / 4;    // direct 1 KB loads per wave (V^T)
  static constexpr int NS = D / 16;                // k-steps of S^T
  static constexpr int NO = D / 32;                // O^T tiles
};

// Direct global -> LDS loads of one 64-key half of a key block. Each wave
// instruction fills 1 KB of LDS, lane l landing at +16l; the lane fetches
// whichever global chunk belongs there under the swizzle. The per-lane byte
// offset (relative to the half's first K row, resp. first V^T column) does
// not depend on the block, so it is computed once, and the per-block part of
// each address is scalar. Instruction it covers K rows 16 it (at D = 128;
// 32 it at D = 64) and V^T rows 32 it on from what instruction 0 covers:
// 4 KB, resp. 8 KB, further, under the same swizzle (the swizzles depend on
// the row modulo 16), so one lane offset per tile serves every instruction.
template <int D>
__device__ __forceinline__ void subtile_offsets(int w, int lane, uint32_t& koff, uint32_t& voff) {
  using T = Tile<D>;
  const int ku = w * 64 + lane;  // unit of instruction 0
  const int row = ku / T::KCH;
  koff = (uint32_t)((row * D + swz_row<D>(row, ku % T::KCH) * 8) * 2);
  const int d = ku >> 3;
  voff = (uint32_t)((d * 128 + swz8(d, ku & 7) * 8) * 2);
}

// Issue the loads of half hf (keys 64hf..64hf+63) into one LDS buffer; w is
// the (uniform) wave index. Buffer loads: the resource holds the block base
// and its size, the half and instruction offsets are the scalar offset
// (with the lane offset they stay inside the block), so a load needs no
// vector address arithmetic at all.
template <int D>
__device__ __forceinline__ void load_subtile(const char* kblk, const char* vblk, int hf, char* buf,
                                             int w, uint32_t koff, uint32_t voff) {
  using T = Tile<D>;
  static_assert(T::KBYTES / T::KLD == 4096 && T::VBYTES / T::VLD == 4096,
                "four waves fill 4 KB of LDS per instruction");
  constexpr int kBlockBytes = 128 * D * 2;
  const __amdgpu_buffer_rsrc_t kr = raw_rsrc(kblk, kBlockBytes);
  const __amdgpu_buffer_rsrc_t vr = raw_rsrc(vblk, kBlockBytes);
#pragma unroll
  for (int it = 0; it < T::KLD; ++it)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, LDS_PTR(buf + (it * 4 + w) * 1024), 16, koff,
                                             64 * hf * D * 2 + 4096 * it, 0, 0);
  char* vb = buf + T::KBYTES;
#pragma unroll
  for (int it = 0; it < T::VLD; ++it)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, LDS_PTR(vb + (it * 4 + w) * 1024), 16, voff,
                                             64 * hf * 2 + 8192 * it, 0, 0);
}

__device__ inline float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Value held by lane l ^ 32 (the other half of this query's keys), through
// v_permlane32_swap: a VALU lane exchange, no LDS round trip.
__device__ inline float partner32(float x, int g) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(g ? r[0] : r[1]);
}

__device__ inline bf16x2 ones2() { return bf16x2{(__bf16)1.f, (__bf16)1.f}; }

// SEG: Stage-1 segment mask. Waves 0-1 hold the block's first latent frame
// (rows 0-63), waves 2-3 the second; key half hf of a block is its frame hf.
// A wave skips a key half whose frame is in another segment than its own.
template <int D, bool SEG>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
  using T = Tile<D>;
  constexpr int NS = T::NS, NO = T::NO;
  constexpr float kLazy = 8.f;  // rescale O only when the row max grows by > 2^8
  __shared__ __attribute__((aligned(16))) char lds[2 * T::BUF];

  const int nS = (a.H / 8) * (a.W / 8);
  const int nq = (a.T / 2) * nS;
  const int n_tasks = a.B * a.NH * nq;
  // XCD-aware order: consecutive workgroups go to the 8 XCDs in turn, so XCD
  // x gets the contiguous task range [x*per, (x+1)*per): neighbouring query
  // blocks of one head (which select overlapping keys) share an L2.
  const int per = (n_tasks + 7) / 8;
  const int task = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (task >= n_tasks) return;
  // longest lists first: query TBs in descending order (a later TB sees more
  // key blocks), so the short lists of the first TBs fill the tail
  // Inside a TB the blocks go column by column: the workgroups an XCD holds
  // at once then cover a few whole columns, so a block's left, right, upper
  // and lower neighbours (whose lists share about half their keys) run
  // together, where a row-major order kept only two or three rows in flight.
  const int r = task % nq, n_tb = a.T / 2;
  const int nby = a.H / 8, rs = r % nS;
  const int i = (n_tb - 1 - r / nS) * nS + (rs % nby) * (a.W / 8) + rs / nby;
  const int bh = task / nq;
  const int h = bh % a.NH, b = bh / a.NH;
  const size_t row = (size_t)bh * nq + i;  // flat query-block row of the lists and q_blk
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int cnt = min(a.sel_cnt[row], a.kmax);
  const int32_t* list = a.sel_idx + row * a.kmax;
  const int tau = 32 * w + l32;          // this lane's query row in the block
  const int n_keys = a.view.n * nS;      // ids outside [0, n_keys) are skipped, never loaded
  uint16_t* out = (uint16_t*)a.out;

  if (cnt <= 0) {
    for (int e = tid; e < 128 * D / 8; e += 256) {
      const int trow = e / (D / 8), c = e % (D / 8);
      *reinterpret_cast<uint4*>(out + out_offset(a, b, h, i, trow, c * 8)) = make_uint4(0, 0, 0, 0);
    }
    if (a.lse && tid < 128) a.lse[row * 128 + tid] = -INFINITY;
    return;
  }

  // this lane's query row: D contiguous values in either layout
  const uint16_t* qb = a.q_tok ? (const uint16_t*)a.q_tok + out_offset(a, b, h, i, tau, 0)
                               : (const uint16_t*)a.q_blk + (row * 128 + tau) * D;
  bf16x8 qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s)
    qf[s] = *reinterpret_cast<const bf16x8*>(qb + 16 * s + 8 * g);

  const size_t bh_slots = (size_t)bh * a.n_slots;
  // View position of a uniform key block id j in [0, n_keys): j / nS by a
  // binary search on the scalar unit (positions are below LCSA_MAX_SLOTS)
  auto view_pos = [&](int j) {
    int p = 0;
#pragma unroll
    for (int step = LCSA_MAX_SLOTS / 2; step > 0; step >>= 1)
      if (j >= (p + step) * nS) p += step;
    return p;
  };
  const int qtb = i / nS;  // query TB (segment mask)
  auto block_base = [&](int j, const char*& kp, const char*& vp) {
    j = (unsigned)j < (unsigned)n_keys ? j : 0;
    const int p = view_pos(j);
    const int s = j - p * nS;
    const size_t blk = (bh_slots + a.view.slot[p]) * nS + s;
    kp = (const char*)a.k_ring + blk * (128 * D * 2);
    vp = (const char*)a.v_ring + blk * (D * 128 * 2);
  };

  f32x16 o[NO];
#pragma unroll
  for (int t = 0; t < NO; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[t][r] = 0.f;
  const float sl2 = a.scale * kLog2e;
  float m = -INFINITY;
  // row sums in four independent v_dot2 chains (one chain of sixteen waits
  // on the instruction's accumulate latency at every step)
  float ls[4] = {0.f, 0.f, 0.f, 0.f};

  // Lane-invariant LDS fragment offsets. K rows prow and prow + 32 share
  // the swizzle (it depends on row & 15), V^T rows 32dt + l32 share it for
  // every dt, so tile and buffer selection are immediate offsets.
  // K rows are read in perm32 order, so S^T's accumulators are P's B
  // fragments in V^T's natural key order
  const int prow = perm32(l32);
  int koff[NS], voff[4];
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) koff[s2] = prow * (D * 2) + swz_row<D>(prow, 2 * s2 + g) * 16;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) voff[ks] = l32 * 128 + swz8(l32, 2 * ks + g) * 16;

  // one 64-key half of a key block held in LDS buffer HB
  auto compute_half = [&](auto hb_tag) {
    constexpr int HB = decltype(hb_tag)::value;
    const char* kb = lds + HB * T::BUF;
    const char* vb = kb + T::KBYTES;
    bf16x8 kf[2][NS];
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      kf[0][s2] = *reinterpret_cast<const bf16x8*>(kb + koff[s2]);
      kf[1][s2] = *reinterpret_cast<const bf16x8*>(kb + koff[s2] + 32 * D * 2);
    }
    __builtin_amdgcn_sched_barrier(0);  // all K fragment reads issue before the first MFMA
    f32x16 sacc[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[0][r] = sacc[1][r] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0][s2], qf[s2], sacc[0], 0, 0, 0);
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[1][s2], qf[s2], sacc[1], 0, 0, 0);
    }
    bf16x8 vf[NO][4];
#pragma unroll
    for (int dt = 0; dt < NO; ++dt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        vf[dt][ks] = *reinterpret_cast<const bf16x8*>(vb + voff[ks] + dt * 32 * 128);

    // row max of the 64 logits (two lanes hold one query's halves)
    float t3[11];
#pragma unroll
    for (int q3 = 0; q3 < 5; ++q3) {
      t3[q3] = max3(sacc[0][3 * q3], sacc[0][3 * q3 + 1], sacc[0][3 * q3 + 2]);
      t3[5 + q3] = max3(sacc[1][3 * q3], sacc[1][3 * q3 + 1], sacc[1][3 * q3 + 2]);
    }
    t3[10] = fmaxf(sacc[0][15], sacc[1][15]);
    float mx = max3(max3(max3(t3[0], t3[1], t3[2]), max3(t3[3], t3[4], t3[5]),
                         max3(t3[6], t3[7], t3[8])), t3[9], t3[10]);
    mx = fmaxf(mx, partner32(mx, g)) * sl2;
    if (__ballot(mx > m + kLazy)) {  // lazy rescale: only when the max grows by > 2^8
      const float mnew = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
#pragma unroll
      for (int e = 0; e < 4; ++e) ls[e] *= alpha;
#pragma unroll
      for (int dt = 0; dt < NO; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      m = mnew;
    }
    bf16x8 pf[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf[kt][hh][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kt][8 * hh + e], sl2, -m));
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pf[kt][hh][e], pf[kt][hh][e + 1]};
          ls[e >> 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2(), ls[e >> 1], false);
        }
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int dt = 0; dt < NO; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt][ks], pf[ks >> 1][ks & 1], o[dt], 0, 0, 0);
  };

  const int dq = __builtin_amdgcn_readfirstlane(w) >> 1;   // this wave's query frame
  const char *kp, *vp;
  uint32_t gkoff, gvoff;
  subtile_offsets<D>(w, lane, gkoff, gvoff);
  // Which halves of key block j this wave computes: none for a skipped id;
  // under the segment mask, the halves whose frame shares this wave's segment
  auto block_flags = [&](int j, bool& ok0, bool& ok1) {
    const bool ok = (unsigned)j < (unsigned)n_keys;  // uniform: skipped id
    ok0 = ok1 = ok;
    if constexpr (SEG) {
      const int p = ok ? view_pos(j) : 0;
      // the dword of qmask[qtb] holding byte p, as a scalar load
      const uint32_t m = ((const uint32_t*)a.qmask[qtb])[p >> 2] >> (8 * (p & 3) + 2 * dq);
      ok0 = ok && (m & 1u);
      ok1 = ok && (m & 2u);
    }
  };
  // List entries are read with scalar loads one block iteration before they
  // are needed (entry it + 2 at the end of iteration it, consumed after the
  // next iteration's first barrier), so no wave waits on a list load.
  const __attribute__((address_space(4))) int32_t* slist =
      (const __attribute__((address_space(4))) int32_t*)list;
  int j_nxt = slist[min(1, cnt - 1)];
  bool ok0, ok1;
  {
    const int j0 = slist[0];
    block_flags(j0, ok0, ok1);
    block_base(j0, kp, vp);
  }
  load_subtile<D>(kp, vp, 0, lds, w, gkoff, gvoff);
  for (int it = 0; it < cnt; ++it) {
    // half 0 of block it is in buffer 0; fetch half 1 into buffer 1
    wait_vm_all();
    __syncthreads();
    load_subtile<D>(kp, vp, 1, lds + T::BUF, w, gkoff, gvoff);
    if (ok0) compute_half(std::integral_constant<int, 0>{});
    // half 1 is in buffer 1; fetch half 0 of the next block into buffer 0
    wait_vm_all();
    __syncthreads();
    bool nok0 = false, nok1 = false;
    if (it + 1 < cnt) {
      block_flags(j_nxt, nok0, nok1);
      block_base(j_nxt, kp, vp);
      load_subtile<D>(kp, vp, 0, lds, w, gkoff, gvoff);
    }
    if (ok1) compute_half(std::integral_constant<int, 1>{});
    ok0 = nok0;
    ok1 = nok1;
    j_nxt = slist[min(it + 2, cnt - 1)];
  }

  // epilogue: normalise, stage the 128 x D tile in LDS, write whole rows
  const float lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
  const float lt = lsum + partner32(lsum, g);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;  // 0 only if every listed id was skipped
  __syncthreads();
  char* st = lds;
#pragma unroll
  for (int dt = 0; dt < NO; ++dt)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      __bf16 v4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v4[j] = (__bf16)(o[dt][4 * ii + j] * inv);
      const int c = 4 * dt + ii;  // 16-byte chunk of d = 32dt + 8ii .. +8
      *reinterpret_cast<uint2*>(st + tau * (D * 2) + swz_row<D>(tau, c) * 16 + 8 * g) =
          *reinterpret_cast<const uint2*>(v4);
    }
  __syncthreads();
  constexpr int CH = D / 8;
#pragma unroll
  for (int e0 = 0; e0 < 128 * CH; e0 += 256) {
    const int e = e0 + tid, trow = e / CH, c = e % CH;
    // O is written once and not read back here: non-temporal, so it does not
    // evict the K / V tiles other query blocks still reuse from L2
    __builtin_nontemporal_store(
        *reinterpret_cast<const u32x4*>(st + trow * (D * 2) + swz_row<D>(trow, c) * 16),
        reinterpret_cast<u32x4*>(out + out_offset(a, b, h, i, trow, c * 8)));
  }
  if (a.lse && g == 0)
    a.lse[row * 128 + tau] = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
}

// fp32 path: one thread per query row, scalar online softmax in chunks of 32
// keys. Meant for small validation workloads, not for throughput.
template <int D, bool SEG>
__global__ __launch_bounds__(128) void attn_f32_kernel(AttnArgs a) {
  __shared__ float ks[128 * D];   // K tile [128][D]
  __shared__ float vts[D * 128];  // V^T tile [D][128]
  const int nS = (a.H / 8) * (a.W / 8);
  const int nq = (a.T / 2) * nS;
  const int task = blockIdx.x;
  const int i = task % nq, bh = task / nq, h = bh % a.NH, b = bh / a.NH;
  const int tau = threadIdx.x;
  const int cnt = min(a.sel_cnt[task], a.kmax);
  const int n_keys = a.view.n * nS;
  const int32_t* list = a.sel_idx + (size_t)task * a.kmax;
  float* out = (float*)a.out;
  if (cnt <= 0) {
    for (int d = 0; d < D; ++d) out[out_offset(a, b, h, i, tau, d)] = 0.f;
    if (a.lse) a.lse[(size_t)task * 128 + tau] = -INFINITY;
    return;
  }
  float q[D], o[D];
  const float* qb = a.q_tok ? (const float*)a.q_tok + out_offset(a, b, h, i, tau, 0)
                            : (const float*)a.q_blk + ((size_t)task * 128 + tau) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qb[d];
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int it = 0; it < cnt; ++it) {
    const int j = list[it];
    if ((unsigned)j >= (unsigned)n_keys) continue;  // uniform across the block
    const int p = j / nS, s = j - p * nS;
    const size_t blk = ((size_t)bh * a.n_slots + a.view.slot[p]) * nS + s;
    const float* kp = (const float*)a.k_ring + blk * 128 * D;
    const float* vp = (const float*)a.v_ring + blk * 128 * D;
    __syncthreads();
    for (int e = tau; e < 128 * D; e += 128) {
      ks[e] = kp[e];
      vts[e] = vp[e];
    }
    __syncthreads();
    for (int c0 = 0; c0 < 128; c0 += 32) {
      if constexpr (SEG) {  // key frame c0 / 64 against this row's frame tau / 64
        if (!((a.qmask[i / nS][p] >> (2 * (tau >> 6) + (c0 >> 6))) & 1u)) continue;
      }
      float sv[32];
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) {
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc = fmaf(q[d], ks[(c0 + kk) * D + d], acc);
        sv[kk] = acc * a.scale;
        mx = fmaxf(mx, sv[kk]);
      }
      const float mnew = fmaxf(m, mx);
      const float alpha = expf(m - mnew);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) {
        const float pv = expf(sv[kk] - mnew);
        l += pv;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(pv, vts[d * 128 + c0 + kk], o[d]);
      }
      m = mnew;
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int d = 0; d < D; ++d) out[out_offset(a, b, h, i, tau, d)] = o[d] * inv;
  if (a.lse) a.lse[(size_t)task * 128 + tau] = l > 0.f ? m + logf(l) : -INFINITY;
}

template <int D, bool SEG>
hipError_t launch_bf16(const AttnArgs& a, hipStream_t s) {
  const long long tasks = (long long)a.B * a.NH * (a.T / 2) * (a.H / 8) * (a.W / 8);
  const long long per = (tasks + 7) / 8;
  hipLaunchKernelGGL((attn_bf16_kernel<D, SEG>), dim3((unsigned)(8 * per)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, bool SEG>
hipError_t launch_f32(const AttnArgs& a, hipStream_t s) {
  const long long tasks = (long long)a.B * a.NH * (a.T / 2) * (a.H / 8) * (a.W / 8);
  hipLaunchKernelGGL((attn_f32_kernel<D, SEG>), dim3((unsigned)tasks), dim3(128), 0, s, a);
  return hipGetLastError();
}

template <bool SEG>
hipError_t launch(const AttnArgs& a, int32_t dtype, hipStream_t s) {
  if (dtype == LCSA_BF16)
    return a.D == 64 ? launch_bf16<64, SEG>(a, s) : launch_bf16<128, SEG>(a, s);
  return a.D == 64 ? launch_f32<64, SEG>(a, s) : launch_f32<128, SEG>(a, s);
}

}  // namespace

hipError_t launch_block_sparse_attn(const AttnArgs& a, int32_t dtype, bool segment,
                                    hipStream_t s) {
  return segment ? launch<true>(a, dtype, s) : launch<false>(a, dtype, s);
}

}  // namespace lcsa
