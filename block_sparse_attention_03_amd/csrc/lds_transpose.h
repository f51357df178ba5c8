// Transposed 16-bit tiles from LDS with gfx950's transposing read
// (ds_read_b64_tr_b16), for tiles staged row-major: [rows][D] bf16 with
// 16-byte chunks XOR-swizzled per row.
//
// Within each group of 16 lanes the instruction gives lane j, as element t,
// element j % 4 of the 8 bytes read by lane 4 t + j / 4 of the group. So the
// 8 values of column d = 32 dt + (L % 32) at rows 16 ks + 8 (L / 32) + 0..7
// (one MFMA A fragment of the transposed tile, or one 16-byte chunk of a
// transposed row) come from two reads: for half h of those rows lane L reads
// row 16 ks + 8 (L / 32) + 4 h + (L % 16) / 4 at column
// 32 dt + 16 ((L / 16) % 2) + 4 (L % 4). That lane layout was checked on the
// device before these helpers were written.
#pragma once

#include <stdint.h>

#include "mfma_tiles.h"

namespace lcsa {

// Swizzle of such a tile: chunk c of row r sits at c ^ g(r). g is a bijection
// of the row's low four bits, so sixteen rows read at one chunk (128-bit
// fragment reads) hit sixteen bank groups, and it sends the four aligned rows
// one transposing read covers (at four aligned chunks) to four different
// 64-byte bank groups, which c ^ (r % 16) would not. An involution.
template <int D>
__device__ inline int swz_t(int row, int c) {
  if constexpr (D == 128) return c ^ (((row & 3) << 2) | ((row >> 2) & 3));
  else return c ^ ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));  // rows of 128 bytes
}

typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));

// Per-lane byte offsets of the two reads of every 32-column group dt, for
// ks = 0; the swizzle reads rows modulo 16, so k-step ks adds 16 rows.
template <int D>
struct TrOff {
  uint32_t off[2][D / 32];
  __device__ explicit TrOff(int lane) {
    const int grp = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int row = 8 * (grp >> 1) + 4 * h + (sl >> 2);
        const int col = 32 * dt + 16 * (grp & 1) + 4 * (sl & 3);
        off[h][dt] = (uint32_t)(row * (D * 2) + swz_t<D>(row, col >> 3) * 16 + (col & 7) * 2);
      }
  }
};

template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, const TrOff<D>& t, int ks, int dt) {
  typedef __attribute__((address_space(3))) short4v* lp;
  const char* base = tile + ks * 16 * (D * 2);
  const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(base + t.off[0][dt]));
  const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lp)(base + t.off[1][dt]));
  const short8v v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace lcsa
