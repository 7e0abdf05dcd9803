// Cross-lane reductions of one 64-lane wave on CDNA4 (gfx950), shared by the
// streaming, merge and draft-part kernels.
//
// They move data only through the lane crossbars that need no LDS: DPP quad
// permutations and row mirrors within each 16-lane row, and the permlane16/32
// swaps across rows. A DPP move or a permlane swap is an ordinary VALU
// instruction, so a reduction costs a handful of dependent VALU cycles instead
// of an LDS round trip per step (ds_bpermute / ds_swizzle).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace da {

// permlane16/32 swaps return the pair {x[l], x[l^16]} (resp. l^32) in the two halves.
__device__ __forceinline__ float pair_max16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_add16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_add32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// All-lane reductions: the quad permutations and row mirrors reduce each
// 16-lane row, the permlane swaps combine the rows. Every step combines a lane
// with a partner that holds the mirror-image operand pair, so by commutativity
// every lane ends with the same bits (rotations would leave the lanes of a row
// with sums associated differently).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2, 3, 0, 1]
constexpr int kDppMirror = 0x140;      // row_mirror: lane i <-> 15 - i of its row
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i <-> 7 - i of its half row
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppMirror>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  return pair_max32(pair_max16(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppMirror>(x);
  x += dpp_f<kDppHalfMirror>(x);
  return pair_add32(pair_add16(x));
}

}  // namespace da
