// Shared pieces of the bf16 matrix-core kernels (the block-sparse attention
// and its backward): vector types, LDS addressing, the swizzles and the row
// order that chains one v_mfma_f32_32x32x16_bf16 into the next.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace lcsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // native vector: stays in VGPRs

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// XOR swizzles of 16-byte chunk c in LDS rows of 256 and 128 bytes: sixteen
// consecutive rows read at one logical chunk hit sixteen different bank
// groups. Involutions: the same map goes logical -> physical and back.
__device__ inline int swz16(int row, int c) { return c ^ (row & 15); }
__device__ inline int swz8(int row, int c) { return c ^ ((row >> 1) & 7); }

// Swizzle of a row of D bf16 values (256 bytes at D = 128, 128 at D = 64).
template <int D>
__device__ inline int swz_row(int row, int c) {
  if constexpr (D == 128) return swz16(row, c);
  else return swz8(row, c);
}

// Row order of a 32-row A operand whose product feeds the next MFMA as its
// B operand. Lane (l, g) of a 32x32 accumulator holds rows 8i + 4g + j
// (i, j = 0..3); reading source row perm32(r) into A row r makes them the
// source rows 16*(i/2) + 8g + 4*(i%2) + j, so accumulator elements 8ks ..
// 8ks + 7 are the source rows 16ks + 8g .. 16ks + 8g + 7: exactly the eight
// contiguous k-elements of the next product's B fragment for k-step ks.
__device__ inline int perm32(int r) {
  const int i = r >> 3, gg = (r >> 2) & 1, j = r & 3;
  return 16 * (i >> 1) + 8 * gg + 4 * (i & 1) + j;
}

// Raw buffer resource over [base, base + bytes) for untyped dword loads
// (word 3: 32-bit data format). A buffer load's address is this base plus a
// 32-bit lane offset plus a scalar offset; the lane offset is range-checked
// against `bytes` (one at or past it reads zeros), the scalar offset is not,
// so callers keep scalar offset + lane offset inside the range themselves.
__device__ inline __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Wait for all of this wave's outstanding vector memory operations
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left at their no-wait maxima).
__device__ inline void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace lcsa
