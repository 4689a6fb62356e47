// Cross-lane reductions of a 64-lane wave on DPP (gfx950), shared by the
// kernels of the library.
#pragma once
#include <hip/hip_runtime.h>

namespace moe {

// Cross-lane butterflies on DPP (no LDS round trip).  Partner lanes: quad_perm
// [1,0,3,2] -> lane ^ 1, [2,3,0,1] -> lane ^ 2, row_half_mirror -> 7 - i
// inside each group of 8, row_mirror -> 15 - i inside each row of 16.  After
// the steps for a group of N lanes every lane of the group holds the same
// value: + and max are commutative, so both partners of a step compute the
// identical result.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int N>   // N in {2, 4, 8, 16}: groups of N consecutive lanes
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<DPP_XOR1>(v);
  if (N >= 4) v += dpp<DPP_XOR2>(v);
  if (N >= 8) v += dpp<DPP_HALF_MIRROR>(v);
  if (N >= 16) v += dpp<DPP_MIRROR>(v);
  return v;
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp<DPP_XOR1>(v));
  if (N >= 4) v = fmaxf(v, dpp<DPP_XOR2>(v));
  if (N >= 8) v = fmaxf(v, dpp<DPP_HALF_MIRROR>(v));
  if (N >= 16) v = fmaxf(v, dpp<DPP_MIRROR>(v));
  return v;
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
// Whole-wave reductions (all 64 lanes active): rows of 16, then the four row
// results in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = group_max<16>(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

}  // namespace moe
