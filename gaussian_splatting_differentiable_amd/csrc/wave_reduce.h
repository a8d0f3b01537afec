// Wave64 reduce-scatter of the 9 per-lane gradient values of one splat.
//
// "What the 3DGS Literature Left on the Table", Step 2 (Figure 6): instead of 9
// full butterflies, halve the set of live components at each exchange so that
// the sums end on distinct lanes and one atomic instruction with 9 active lanes
// writes them all. On gfx950 the first two exchanges are the lane-half swaps
// v_permlane32_swap (lanes 0-31 <-> 32-63) and v_permlane16_swap (rows 0,2 <->
// rows 1,3); each swap moves one component pair across, so one add per pair
// sums it. The last 16 lanes of each row are summed with four DPP row
// rotations (ror 8, 4, 2, 1), which fold into v_add_f32_dpp.
//
//   after swap32 : lanes 0-31 hold components 0-4, lanes 32-63 hold 5-9 (9 = 0)
//   after swap16 : row 0 {0,1,2}, row 1 {3,4,-}, row 2 {5,6,7}, row 3 {8,-,-}
//   row sums     : every lane of a row holds its row's (up to) three sums
// Lane 16 r + s (s < 3) then owns component comp_of(r, s).
#pragma once
#include "gs_common.h"

__device__ __forceinline__ float swap_sum32(float x, float y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float swap_sum16(float x, float y) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int m = __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false);
  return v + __int_as_float(m);
}

// sum over the 16 lanes of each row; every lane ends with its row's sum
__device__ __forceinline__ float row_sum16(float v) {
  v = dpp_add<0x128>(v);  // row_ror:8
  v = dpp_add<0x124>(v);  // row_ror:4
  v = dpp_add<0x122>(v);  // row_ror:2
  v = dpp_add<0x121>(v);  // row_ror:1
  return v;
}

// Component owned by lane (row r, slot s), or -1.
__device__ __forceinline__ int comp_of_lane(int lane) {
  const int r = lane >> 4, s = lane & 15;
  if (s >= 3) return -1;
  // row 0: 0 1 2 | row 1: 3 4 - | row 2: 5 6 7 | row 3: 8 - -
  const int base = (r == 0) ? 0 : (r == 1) ? 3 : (r == 2) ? 5 : 8;
  const int cnt = (r == 0 || r == 2) ? 3 : (r == 1) ? 2 : 1;
  return s < cnt ? base + s : -1;
}

// Reduce g[0..8] over the wave; returns the sum of component comp_of_lane(lane)
// on the lanes that own one (garbage elsewhere).
__device__ __forceinline__ float reduce_scatter9(const float g[9]) {
  // lanes 0-31 keep components j, lanes 32-63 keep j+5
  const float t0 = swap_sum32(g[0], g[5]);
  const float t1 = swap_sum32(g[1], g[6]);
  const float t2 = swap_sum32(g[2], g[7]);
  const float t3 = swap_sum32(g[3], g[8]);
  const float t4 = swap_sum32(g[4], 0.0f);
  // even rows keep t0..t2, odd rows keep t3, t4, 0
  const float u0 = row_sum16(swap_sum16(t0, t3));
  const float u1 = row_sum16(swap_sum16(t1, t4));
  const float u2 = row_sum16(swap_sum16(t2, 0.0f));
  const int s = __lane_id() & 15;
  return s == 0 ? u0 : (s == 1 ? u1 : u2);
}
