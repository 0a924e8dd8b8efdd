// Device helpers shared by the decode kernels (gemv.hip, gemv_lut.hip, gemv_bin.hip).
#pragma once
#include "bl_internal.h"

namespace bl {

// Word i (0..3) of a 16-byte lane slot.
__device__ __forceinline__ uint32_t word_of(const uint4& w, int i) {
  return i == 0 ? w.x : (i == 1 ? w.y : (i == 2 ? w.z : w.w));
}

// Non-temporal 16-byte load: packed weights are read once per launch.
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p)));
}

// Lane l of each 16-lane row takes lane l + s of the same row (DPP row_shl).
template <int s>
__device__ __forceinline__ int row_shl(int v) {
  if constexpr (s == 0) return v;
  else return __builtin_amdgcn_mov_dpp(v, 0x100 + s, 0xF, 0xF, true);
}

// One token: the A operand of step (u, i) only needs piece 4 u + i in lane 0 of each row,
// and a 64-bit DPP row_newbcast copies that lane to the whole row in two moves.
template <int n>
__device__ __forceinline__ uint64_t row_bcast64(uint64_t v) {
  return (uint64_t)__builtin_amdgcn_update_dpp((long)0, (long)v, 0x150 + n, 0xF, 0xF, false);
}

}  // namespace bl
