// Wave-wide (64-lane) integer scans and reductions on DPP moves (gfx9 family, gfx950).
//
// An inclusive scan inside each 16-lane row takes row_shr:1, 2, 4, 8 (a lane whose source falls
// outside its row adds 0); row_bcast:15 then adds the last lane of rows 0 and 2 into rows 1 and
// 3, and row_bcast:31 adds lane 31 into rows 2 and 3.  A reduction is the scan's lane 63, read
// into a scalar register.  Every step is a VALU instruction with a DPP source, so a 64-lane scan
// costs six dependent ALU operations rather than six LDS-crossbar permutes.
#pragma once

#include <hip/hip_runtime.h>

#include <limits.h>

namespace pkv {
namespace {

// x of the lane CTRL selects, or `fill` where that lane is outside the row or its row is masked
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_or(int x, int fill) {
  return __builtin_amdgcn_update_dpp(fill, x, CTRL, ROW_MASK, 0xf, false);
}

__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_or<0x111>(x, 0);       // row_shr:1
  x += dpp_or<0x112>(x, 0);       // row_shr:2
  x += dpp_or<0x114>(x, 0);       // row_shr:4
  x += dpp_or<0x118>(x, 0);       // row_shr:8
  x += dpp_or<0x142, 0xa>(x, 0);  // row_bcast:15 into rows 1 and 3
  x += dpp_or<0x143, 0xc>(x, 0);  // row_bcast:31 into rows 2 and 3
  return x;
}

__device__ __forceinline__ int wave_incl_max(int x) {
  x = max(x, dpp_or<0x111>(x, INT_MIN));
  x = max(x, dpp_or<0x112>(x, INT_MIN));
  x = max(x, dpp_or<0x114>(x, INT_MIN));
  x = max(x, dpp_or<0x118>(x, INT_MIN));
  x = max(x, dpp_or<0x142, 0xa>(x, INT_MIN));
  x = max(x, dpp_or<0x143, 0xc>(x, INT_MIN));
  return x;
}

// value of lane `src` (a wave-uniform index), in a scalar register
__device__ __forceinline__ int lane_value(int x, int src) { return __builtin_amdgcn_readlane(x, src); }

// sum and maximum over the 64 lanes, the same in every lane
__device__ __forceinline__ int wave_sum(int x) { return lane_value(wave_incl_scan(x), 63); }
__device__ __forceinline__ int wave_max(int x) { return lane_value(wave_incl_max(x), 63); }

}  // namespace
}  // namespace pkv
