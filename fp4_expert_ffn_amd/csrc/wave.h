// Wave64 cross-lane primitives for gfx950 without LDS round trips:
// DPP row permutations inside each 16-lane row, then v_permlane16_swap /
// v_permlane32_swap across rows.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Every control used here (quad permutations, row mirrors) gives each lane a
// source lane, so no lane reads out of bounds: with old = 0 and bound_ctrl
// set the compiler fuses the move into the consuming instruction
// (v_max_u32_dpp, v_add_f32_dpp), with the same result.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// v_permlane16_swap on (v, v) returns one copy holding rows {0,0,2,2} and one
// holding rows {1,1,3,3} of v; v_permlane32_swap likewise returns the lower and
// the upper half of v, each duplicated.  Combining the two copies reduces over
// row pairs (lanes l, l^16) or halves (lanes l, l^32) whichever copy is which.
__device__ __forceinline__ float sum_rowpair(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float sum_halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the four lanes l, l^16, l^32, l^48 (every lane receives the sum).
__device__ __forceinline__ float sum_rows4(float v) { return sum_halves(sum_rowpair(v)); }

// Max over the four lanes l, l^16, l^32, l^48 (every lane receives it).
__device__ __forceinline__ float max_rows4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Full-wave sum, result in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowHalfMirror>(v);
  v += dpp_f32<kDppRowMirror>(v);
  return sum_rows4(v);
}

// Full-wave unsigned 32-bit max, result in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppQuadXor1>(v));
  v = max(v, dpp_u32<kDppQuadXor2>(v));
  v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  v = max(v, dpp_u32<kDppRowMirror>(v));
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max(a[0], a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max(b[0], b[1]);
}

}  // namespace moe
