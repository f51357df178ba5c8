// Local spatial window of the block mask ([FN] "FlashVSR" note, Key design
// 3: Boundary-Preserved and Boundary-Truncated rules; [HW] "How FlashVSR
// works" 2.2 step 2: a local_range x local_range block neighbourhood).
// Shared by the host validation code and the draft kernel.
#pragma once

#include <cstdint>

#if defined(__HIPCC__)
#define LCSA_HD __host__ __device__
#else
#define LCSA_HD
#endif

namespace lcsa {

// Inclusive range [lo, hi] of blocks along an axis of n blocks that block i
// may see. border 0 (preserved): a window of r blocks shifted to stay inside
// the grid (the whole axis when n <= r). border 1 (truncated): the centred
// window of r blocks clipped at the edges.
LCSA_HD inline void window_range(int32_t i, int32_t n, int32_t r, int32_t border, int32_t* lo,
                                 int32_t* hi) {
  const int32_t h = r / 2;
  if (border == 0) {
    if (n <= r) {
      *lo = 0;
      *hi = n - 1;
      return;
    }
    int32_t s = i - h;
    s = s < 0 ? 0 : s;
    s = s > n - r ? n - r : s;
    *lo = s;
    *hi = s + r - 1;
  } else {
    *lo = i - h < 0 ? 0 : i - h;
    *hi = i + h > n - 1 ? n - 1 : i + h;
  }
}

}  // namespace lcsa
