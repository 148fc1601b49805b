// Cross-lane moves used by the weight-streaming kernels.
#pragma once
#include "device_common.hpp"

namespace moe {

// Each lane's value from the lane D places higher in its row of 16 lanes
// (DPP row rotation; a rotation right by n moves lane i's value to lane i + n).
template <int D>
__device__ __forceinline__ uint4 from_lane_above(uint4 v) {
  constexpr int ctrl = 0x120 + ((16 - D) & 15);   // row_ror:(16 - D)
  return make_uint4((uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, ctrl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, ctrl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.z, ctrl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_mov_dpp((int)v.w, ctrl, 0xF, 0xF, false));
}

// from_lane_above<d>(v) for d = 0, 2, 4, ..., 14, known once loops are unrolled.
__device__ __forceinline__ uint4 from_lane_above_even(uint4 v, int d) {
  switch (d) {
    case 0: return v;
    case 2: return from_lane_above<2>(v);
    case 4: return from_lane_above<4>(v);
    case 6: return from_lane_above<6>(v);
    case 8: return from_lane_above<8>(v);
    case 10: return from_lane_above<10>(v);
    case 12: return from_lane_above<12>(v);
    default: return from_lane_above<14>(v);
  }
}

template <int V> struct IntC { static constexpr int value = V; };

}  // namespace moe
