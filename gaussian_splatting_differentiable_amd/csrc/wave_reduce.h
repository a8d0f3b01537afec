// Wave64 reduce-scatter of the 9 per-lane gradient values of one splat.
//
// "What the 3DGS Literature Left on the Table", Step 2 (Figure 6): instead of 9
// full butterflies, halve the set of live values at each exchange so that the
// sums end on distinct lanes and one atomic instruction with 9 active lanes
// writes them all. On gfx950:
//
//   swap32 (v_permlane32_swap, lanes 0-31 <-> 32-63), pairs (0,5) (1,6) (2,7)
//          (3,8) (4,-): lanes 0-31 keep components 0-4, lanes 32-63 keep 5-8;
//   swap16 (v_permlane16_swap, rows 0,2 <-> rows 1,3), pairs (t0,t1) (t2,t3)
//          (t4,-): row 0 keeps {0,2,4}, row 1 {1,3,-}, row 2 {5,7,-}, row 3
//          {6,8,-}; every lane now holds three partial sums of 4 lanes each;
//   ror8   (DPP row_ror:8, lane s <-> s^8) on the pair (u0,u1): lanes 0-7 keep
//          u0, lanes 8-15 keep u1; u2 is summed on all 16 lanes;
//   mirror (DPP row_half_mirror, lane s <-> 7-s within each 8) on (v,u2):
//          lanes 0-3 and 8-11 keep v, lanes 4-7 and 12-15 keep u2;
//   two quad_perm adds finish each group of 4 lanes.
//
// Lane 16 r + s then owns: s = 0 -> {0,1,5,6}[r], s = 8 -> {2,3,7,8}[r],
// s = 4 and r = 0 -> 4. 27 instructions for the 9 sums.
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

// a + (b as seen through the DPP control CTRL)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float a, float b) {
  const int m = __builtin_amdgcn_update_dpp(0, __float_as_int(b), CTRL, 0xF, 0xF, false);
  return a + __int_as_float(m);
}

constexpr int DPP_ROW_ROR8 = 0x128;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_QUAD_2301 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_QUAD_1032 = 0xB1;  // quad_perm [1,0,3,2]

// Component owned by lane (row r, slot s), or -1.
__device__ __forceinline__ int comp_of_lane(int lane) {
  const int r = lane >> 4, s = lane & 15;
  if (s == 0) return r < 2 ? r : r + 3;      // 0 1 5 6
  if (s == 8) return r < 2 ? r + 2 : r + 5;  // 2 3 7 8
  if (s == 4 && r == 0) return 4;
  return -1;
}

// Reduce g[0..8] over the wave; returns the sum of component comp_of_lane(lane)
// on the lanes that own one (partial sums elsewhere).
__device__ __forceinline__ float reduce_scatter9(const float g[9]) {
  const float t0 = swap_sum32(g[0], g[5]);
  const float t1 = swap_sum32(g[1], g[6]);
  const float t2 = swap_sum32(g[2], g[7]);
  const float t3 = swap_sum32(g[3], g[8]);
  const float t4 = swap_sum32(g[4], 0.0f);
  const float u0 = swap_sum16(t0, t1);
  const float u1 = swap_sum16(t2, t3);
  const float u2 = swap_sum16(t4, 0.0f);
  const int s = __lane_id() & 15;
  const bool lo8 = s < 8, lo4 = (s & 4) == 0;
  const float v = dpp_add<DPP_ROW_ROR8>(lo8 ? u0 : u1, lo8 ? u1 : u0);
  const float w = dpp_add<DPP_ROW_ROR8>(u2, u2);
  float x = dpp_add<DPP_ROW_HALF_MIRROR>(lo4 ? v : w, lo4 ? w : v);
  x = dpp_add<DPP_QUAD_2301>(x, x);
  x = dpp_add<DPP_QUAD_1032>(x, x);
  return x;
}
