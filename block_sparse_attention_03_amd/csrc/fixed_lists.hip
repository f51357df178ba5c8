// Index lists that need no draft selection, in the format the attention
// kernel reads (ascending logical key ids, -1 padding, a count per row).
//
// Local lists. [FP] "FlashVSR+" project page, Hybrid Attention: the local
// layers of the hybrid student attend every key block of a compact space-time
// neighbourhood. The list of a query block is its whole allowed set: every
// visible key TB (not later than its own) times the spatial window of the
// border rule ([FN] Key design 3), enumerated in (TB, by, bx) order, which is
// ascending id order.
//
// Segment lists: the key blocks each query block attends under the Stage-1
// block-diagonal segment mask.
//
// [FN] "FlashVSR" note, Key design 1, Stage 1: every token attends all
// tokens of its own segment (a video clip, or an image as a one-frame
// segment), with no block sparsity and no causality. At block granularity a
// query block of temporal block a needs every key block of every temporal
// block p that holds a frame of one of a's segments; the token-level mask
// inside such a pair is applied by the attention kernel. The host derives
// the listed temporal blocks per query TB from the per-frame segment ids;
// this kernel expands them into per-row id lists (all spatial blocks of the
// listed TBs, ascending), so the attention kernel reads the same list format
// as after the draft selection.
#include "lcsa_kernels.h"
#include "lcsa_window.h"

namespace lcsa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void segment_lists_kernel(SegListArgs a) {
  const int row = blockIdx.x;  // flat (b, h, i)
  if (row >= a.rows) return;
  const int i = row % a.nq;
  const int qtb = i / a.nS;
  const int cnt = a.n_tb[qtb] * a.nS;
  int32_t* dst = a.sel_idx + (size_t)row * a.kmax;
  for (int e = threadIdx.x; e < a.kmax; e += kThreads) {
    int32_t id = -1;
    if (e < cnt) id = (int32_t)a.tb[qtb][e / a.nS] * a.nS + e % a.nS;
    dst[e] = id;
  }
  if (threadIdx.x == 0) a.sel_cnt[row] = cnt;
}

__global__ __launch_bounds__(kThreads) void local_lists_kernel(LocalListArgs a) {
  const int row = blockIdx.x;  // flat (b, h, i)
  if (row >= a.rows) return;
  const int i = row % a.nq, nS = a.nby * a.nbx;
  const int qtb = i / nS, s = i % nS, by = s / a.nbx, bx = s % a.nbx;
  int32_t ylo, yhi, xlo, xhi;
  window_range(by, a.nby, a.local_range, a.border, &ylo, &yhi);
  window_range(bx, a.nbx, a.local_range, a.border, &xlo, &xhi);
  const int wy = yhi - ylo + 1, wx = xhi - xlo + 1, per_tb = wy * wx;
  const int cnt = a.n_vis[qtb] * per_tb;
  int32_t* dst = a.sel_idx + (size_t)row * a.kmax;
  for (int e = threadIdx.x; e < a.kmax; e += kThreads) {
    int32_t id = -1;
    if (e < cnt) {
      const int p = e / per_tb, r = e % per_tb;
      id = p * nS + (ylo + r / wx) * a.nbx + xlo + r % wx;
    }
    dst[e] = id;
  }
  if (threadIdx.x == 0) a.sel_cnt[row] = cnt;
}

}  // namespace

hipError_t launch_local_lists(const LocalListArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(local_lists_kernel, dim3((unsigned)a.rows), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_segment_lists(const SegListArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(segment_lists_kernel, dim3((unsigned)a.rows), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace lcsa
