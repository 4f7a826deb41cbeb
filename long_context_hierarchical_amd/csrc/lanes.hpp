// Wave64 lane helpers shared by the attention kernels: bf16 packing and DPP reductions.
#pragma once

#include <hip/hip_runtime.h>

namespace recsa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Round two floats to bf16 (nearest, ties to even) and pack them.
__device__ __forceinline__ bf16x2_t pack_bf16_rne(float lo, float hi) {
  return __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sum over each group of N (4, 8 or 16) consecutive lanes, left in every lane of the group, with
// DPP lane moves (no LDS round trip): pairs of lanes, pairs of pairs, then (N = 8) the two
// quads of the half-row, mirrored, then (N = 16) the two halves of the row, mirrored.
// Every control used here moves lanes within one 16-lane row, so no source lane is out of
// bounds: bound_ctrl (an out-of-bounds source reads 0) changes no result, and it lets the
// compiler drop the move's zero-initialised destination.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16, "groups of 4, 8 or 16 lanes");
  x = x + dpp_move<0xB1>(x);                          // quad_perm [1, 0, 3, 2]
  x = x + dpp_move<0x4E>(x);                          // quad_perm [2, 3, 0, 1]
  if constexpr (N >= 8) x = x + dpp_move<0x141>(x);   // row_half_mirror
  if constexpr (N == 16) x = x + dpp_move<0x140>(x);  // row_mirror
  return x;
}

// Wave-wide sum / max with DPP inside each 16-lane row (pairs, quads, half-rows, rows), then
// the four row results combined in a fixed order from lanes 0, 16, 32 and 48; every lane
// gets the same value.
__device__ __forceinline__ float lane_read(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x = x + dpp_move<0xB1>(x);
  x = x + dpp_move<0x4E>(x);
  x = x + dpp_move<0x141>(x);   // row_half_mirror
  x = x + dpp_move<0x140>(x);   // row_mirror
  return (lane_read(x, 0) + lane_read(x, 16)) + (lane_read(x, 32) + lane_read(x, 48));
}
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_move<0xB1>(x));
  x = fmaxf(x, dpp_move<0x4E>(x));
  x = fmaxf(x, dpp_move<0x141>(x));
  x = fmaxf(x, dpp_move<0x140>(x));
  return fmaxf(fmaxf(lane_read(x, 0), lane_read(x, 16)), fmaxf(lane_read(x, 32), lane_read(x, 48)));
}

}  // namespace recsa
