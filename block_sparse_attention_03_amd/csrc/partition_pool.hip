// Steps 1-2 of LCSA: 3D window partition and block-mean pooling, fused.
//
// [HW] "How FlashVSR works" 2.2 step 1: q, k, v are cut into non-overlapping
// windows of 2 latent frames x 8 x 8 tokens (128 tokens per block). Step 3
// of the same section compresses each block of q and k into one vector by
// its mean ([FN] "FlashVSR" note, Key design 2: block-mean pooling before
// the coarse block map).
//
// One workgroup moves one tile: one of q, k or v for one (batch, head,
// block), so reads and writes of different workgroups overlap and a small
// grid still spreads over the chip. The token layout keeps a token's D
// channels contiguous (D*esize = 128..512 bytes), so every read is a run of
// whole 16-byte chunks; every write is a fully contiguous 128 x D tile. V is
// written transposed ([D][128]) because the attention kernel feeds V^T to
// the matrix cores as the A operand; bf16 V is transposed in LDS by
// gfx950's transposing read. Block means of q and k are accumulated
// in float64 (exact for bf16 inputs of moderate range) and written as
// float64, so the draft selection downstream takes its decision on exact
// pooled values. HBM-bound: the algorithmic traffic of one (block, head) is
// 3 tiles read + 3 tiles written + 2 pooled rows.
#include "lcsa_kernels.h"
#include "lds_transpose.h"

namespace lcsa {
namespace {

constexpr int kThreads = 256;

template <int ESZ>
__device__ inline void widen_chunk(const u32x4& v, double* out);

template <>
__device__ inline void widen_chunk<2>(const u32x4& v, double* out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = (double)__uint_as_float(w[i] << 16);
    out[2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ inline void widen_chunk<4>(const u32x4& v, double* out) {
  out[0] = (double)__uint_as_float(v.x);
  out[1] = (double)__uint_as_float(v.y);
  out[2] = (double)__uint_as_float(v.z);
  out[3] = (double)__uint_as_float(v.w);
}

template <int ESZ, int D>
struct Geo {
  static constexpr int EPC = 16 / ESZ;        // elements per 16-byte chunk
  static constexpr int CPT = D / EPC;         // chunks per token row
  static constexpr int ITERS = 128 * CPT / kThreads;
  static constexpr int TPI = kThreads / CPT;  // tokens covered per iteration
  static constexpr int PITCH = D * ESZ + 16;  // LDS row pitch of the V stage
};

// Token-layout element offset of in-block token tau of block (bt, by, bx).
__device__ inline size_t token_offset(const PartitionArgs& a, int b, int h, int bt, int by, int bx,
                                      int tau) {
  const int t = 2 * bt + (tau >> 6);
  const int y = 8 * by + ((tau >> 3) & 7);
  const int x = 8 * bx + (tau & 7);
  return ((((size_t)b * a.T + t) * a.H + y) * a.W + x) * a.NH * a.D + (size_t)h * a.D;
}

// Load this thread's chunks of one 128 x D block (token layout source). The
// token-layout inputs are read exactly once, so the loads are non-temporal
// (4K step: 234 -> 212 us). The outputs are stored normally: the attention
// kernel reads them next, and non-temporal stores measured slower.
template <int ESZ, int D>
__device__ inline void load_block(const PartitionArgs& a, const char* src, int b, int h, int bt,
                                  int by, int bx, u32x4 (&v)[Geo<ESZ, D>::ITERS]) {
  using G = Geo<ESZ, D>;
  const int c = threadIdx.x % G::CPT, tsub = threadIdx.x / G::CPT;
#pragma unroll
  for (int it = 0; it < G::ITERS; ++it) {
    const int tau = it * G::TPI + tsub;
    v[it] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
        src + (token_offset(a, b, h, bt, by, bx, tau) + c * G::EPC) * ESZ));
  }
}

// Store the chunks as a contiguous [128][D] tile (no store when dst is
// null: uniform per workgroup); acc gets the thread's float64 column sums
// of its EPC channels over its ITERS tokens.
template <int ESZ, int D>
__device__ inline void store_tile_sum(char* dst, const u32x4 (&v)[Geo<ESZ, D>::ITERS],
                                      double (&acc)[Geo<ESZ, D>::EPC]) {
  using G = Geo<ESZ, D>;
  const int c = threadIdx.x % G::CPT, tsub = threadIdx.x / G::CPT;
#pragma unroll
  for (int e = 0; e < G::EPC; ++e) acc[e] = 0.0;
#pragma unroll
  for (int it = 0; it < G::ITERS; ++it) {
    const int tau = it * G::TPI + tsub;
    if (dst) *reinterpret_cast<u32x4*>(dst + ((size_t)tau * D + c * G::EPC) * ESZ) = v[it];
    double w[G::EPC];
    widen_chunk<ESZ>(v[it], w);
#pragma unroll
    for (int e = 0; e < G::EPC; ++e) acc[e] += w[e];
  }
}

template <int ESZ, int D>
__global__ __launch_bounds__(kThreads) void partition_pool_kernel(PartitionArgs a) {
  using G = Geo<ESZ, D>;
  static_assert(64 % G::CPT == 0, "a wave holds whole groups of column chunks");
  constexpr int kWaves = kThreads / 64;
  // one LDS buffer for either role: the V stage, or the per-wave column sums
  __shared__ __attribute__((aligned(16))) char smem[128 * G::PITCH];
  static_assert(kWaves * D * sizeof(double) <= sizeof(smem), "column sums fit the stage");

  // heads vary fastest across workgroups: the heads of one block read the
  // same 128 token rows ([NH][D] contiguous per token) at about the same
  // time; then the tensor (k, v, q), then the block
  const int nby = a.H / 8, nbx = a.W / 8, nS = nby * nbx;
  const int nblk = (a.T / 2) * nS;
  const bool has_q = a.q != nullptr;
  const int roles = has_q ? 3 : 2;
  int idx = blockIdx.x;
  const int h = idx % a.NH;
  idx /= a.NH;
  const int role = idx % roles;  // 0: k, 1: v, 2: q (uniform per workgroup)
  idx /= roles;
  const int n = idx % nblk;
  const int b = idx / nblk;
  const int bt = n / nS, s = n % nS, by = s / nbx, bx = s % nbx;
  const size_t tile = (size_t)128 * D;
  const int slot = (a.first_slot + bt) % a.n_slots;
  const size_t ring_blk = (((size_t)b * a.NH + h) * a.n_slots + slot) * nS + s;
  const int tid = threadIdx.x;

  u32x4 v[G::ITERS];
  const void* src = role == 0 ? a.k : role == 1 ? a.v : a.q;
  load_block<ESZ, D>(a, (const char*)src, b, h, bt, by, bx, v);

  if (role == 1) {
    char* vdst = (char*)a.v_ring + ring_blk * tile * ESZ;
    if constexpr (ESZ == 2) {
      // v (bf16): stage the block row-major under the transposing-read
      // swizzle, then every 16-byte chunk of the [D][128] tile (8 tokens of
      // one channel d) comes from two transposing reads. Wave w takes the
      // pairs (column group dt, 16-token step ks) w, w + 4, ...
      const int c = tid % G::CPT, tsub = tid / G::CPT;
#pragma unroll
      for (int it = 0; it < G::ITERS; ++it) {
        const int tau = it * G::TPI + tsub;
        *reinterpret_cast<u32x4*>(smem + tau * (D * 2) + swz_t<D>(tau, c) * 16) = v[it];
      }
      __syncthreads();
      const int lane = tid & 63, w = tid >> 6;
      const TrOff<D> tro(lane);
#pragma unroll
      for (int pi = w; pi < (D / 32) * 8; pi += kThreads / 64) {
        const int dt = pi % (D / 32), ks = pi / (D / 32);
        const int d = 32 * dt + (lane & 31), kc = 2 * ks + (lane >> 5);
        const bf16x8 x = tr_frag<D>(smem, tro, ks, dt);
        *reinterpret_cast<u32x4*>(vdst + ((size_t)d * 128 + kc * 8) * 2) =
            __builtin_bit_cast(u32x4, x);
      }
      return;
    }
    // v (float32): stage the block, then write it transposed ([D][128])
    const int c = tid % G::CPT, tsub = tid / G::CPT;
#pragma unroll
    for (int it = 0; it < G::ITERS; ++it) {
      const int tau = it * G::TPI + tsub;
      *reinterpret_cast<u32x4*>(smem + tau * G::PITCH + c * 16) = v[it];
    }
    __syncthreads();
    constexpr int KC = 128 / G::EPC;  // 16-byte chunks per transposed row
#pragma unroll
    for (int it = 0; it < G::ITERS; ++it) {
      const int e = it * kThreads + tid;
      const int d = e / KC, kc = e % KC;
      uint32_t w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        w[u] = *reinterpret_cast<const uint32_t*>(smem + (kc * 4 + u) * G::PITCH + d * 4);
      *reinterpret_cast<u32x4*>(vdst + ((size_t)d * 128 + kc * G::EPC) * ESZ) =
          u32x4{w[0], w[1], w[2], w[3]};
    }
    return;
  }

  // q or k: the row-major tile (none for q without q_blk), then the block
  // mean of each channel
  const size_t qb = ((size_t)b * a.NH + h) * nblk + n;
  char* dst = role == 0 ? (char*)a.k_ring + ring_blk * tile * ESZ
            : a.q_blk   ? (char*)a.q_blk + qb * tile * ESZ
                        : nullptr;
  double acc[G::EPC];
  store_tile_sum<ESZ, D>(dst, v, acc);
  // the lanes of a wave holding the same column chunk (lane % CPT) add up,
  // in a fixed xor order; then the waves' sums in order
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int m = G::CPT; m < 64; m <<= 1)
#pragma unroll
    for (int e = 0; e < G::EPC; ++e) acc[e] += __shfl_xor(acc[e], m);
  double* red = reinterpret_cast<double*>(smem);  // [kWaves][D]
  if (lane < G::CPT)
#pragma unroll
    for (int e = 0; e < G::EPC; ++e) red[w * D + lane * G::EPC + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    double sum = 0.0;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) sum += red[ww * D + tid];
    const double mean = sum / 128.0;
    if (role == 2)
      a.q_pool[qb * D + tid] = mean;
    else  // k means go d-major into the pooled ring
      a.kpool_ring[((((size_t)b * a.NH + h) * a.n_slots + slot) * D + tid) * nS + s] = mean;
  }
}

template <int ESZ, int D>
hipError_t launch(const PartitionArgs& a, hipStream_t s) {
  const long long nblk = (long long)(a.T / 2) * (a.H / 8) * (a.W / 8);
  const long long roles = a.q ? 3 : 2;
  const long long wgs = nblk * a.NH * a.B * roles;
  hipLaunchKernelGGL((partition_pool_kernel<ESZ, D>), dim3((unsigned)wgs), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partition_pool(const PartitionArgs& a, hipStream_t s) {
  if (a.dtype == LCSA_BF16) return a.D == 64 ? launch<2, 64>(a, s) : launch<2, 128>(a, s);
  return a.D == 64 ? launch<4, 64>(a, s) : launch<4, 128>(a, s);
}

}  // namespace lcsa
