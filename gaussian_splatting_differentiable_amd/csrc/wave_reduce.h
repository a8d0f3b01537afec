// Reduce-scatter of the 9 per-lane gradient values of one splat over each
// 16-lane row of a wave (the four rows reduce four different splats at once).
//
// "What the 3DGS Literature Left on the Table", Step 2 (Figure 6): instead of 9
// full butterflies, halve the set of live values at each exchange so that the
// sums end on distinct lanes and one atomic instruction writes them all. On
// gfx950 a row of 16 lanes is exactly the reach of the DPP row operations, so
// every exchange stays inside the row (lane s of the row):
//
//   ror8   (row_ror:8, s <-> s^8) on the pairs (g0,g1) (g2,g3) (g4,g5) (g6,g7):
//          lanes s < 8 keep the first of each pair, s >= 8 the second; g8 is
//          summed on every lane;
//   mirror (row_half_mirror, s <-> s^7 within each 8) on the two pairs left:
//          s mod 8 < 4 keeps the first, the others the second; g8 again;
//   quad   (quad_perm [2,3,0,1], s <-> s^2) on the pair left and g8, then
//          (quad_perm [1,0,3,2], s <-> s^1) on (that, g8).
//
// The sums end on lanes s = 0, 8, 4, 12, 2, 10, 6, 14 (components 0-7) and
// every odd lane (component 8). 21 VALU instructions for four splats' 9 sums:
// the two bank-aligned levels exchange with complementary bank masks and need
// no selects; the two quad levels take one select pair each.
#pragma once
#include "gs_common.h"

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

// Component whose row sum lane s (0-15) of its row owns after
// reduce_scatter9_row, or -1.
__host__ __device__ __forceinline__ int comp_of_row_lane(int s) {
  switch (s & 15) {
    case 0: return 0;
    case 8: return 1;
    case 4: return 2;
    case 12: return 3;
    case 2: return 4;
    case 10: return 5;
    case 6: return 6;
    case 14: return 7;
    case 1: return 8;
    default: return -1;
  }
}

// The pair exchanges of the two bank-aligned levels: lanes of the DPP banks in
// the first mask keep x summed with its partner, the others y. Two DPP adds
// with complementary bank masks write every lane, so no select is needed. The
// s_nop gives the two wait states a DPP read of a VGPR needs after the VALU
// instruction that wrote it.
__device__ __forceinline__ float pair_ror8(float x, float y) {
  float r;
  __asm__("s_nop 1\n\t"
          "v_add_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0x3 bound_ctrl:1\n\t"
          "v_add_f32_dpp %0, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xc bound_ctrl:1"
          : "=&v"(r)
          : "v"(x), "v"(y));
  return r;
}
__device__ __forceinline__ float pair_mirror(float x, float y) {
  float r;
  __asm__("s_nop 1\n\t"
          "v_add_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0x5 bound_ctrl:1\n\t"
          "v_add_f32_dpp %0, %2, %2 row_half_mirror row_mask:0xf bank_mask:0xa bound_ctrl:1"
          : "=&v"(r)
          : "v"(x), "v"(y));
  return r;
}

// Reduce g[0..8] over each 16-lane row; returns the row's sum of component
// comp_of_row_lane(lane) on the lanes that own one (partial sums elsewhere).
// lo2 / lo1: bit 1 / bit 0 of the lane index is clear.
__device__ __forceinline__ float reduce_scatter9_row(const float g[9], bool lo2, bool lo1) {
  const float t0 = pair_ror8(g[0], g[1]);
  const float t1 = pair_ror8(g[2], g[3]);
  const float t2 = pair_ror8(g[4], g[5]);
  const float t3 = pair_ror8(g[6], g[7]);
  const float t4 = dpp_add<DPP_ROW_ROR8>(g[8], g[8]);
  const float u0 = pair_mirror(t0, t1);
  const float u1 = pair_mirror(t2, t3);
  const float u2 = dpp_add<DPP_ROW_HALF_MIRROR>(t4, t4);
  const float v = dpp_add<DPP_QUAD_2301>(lo2 ? u0 : u1, lo2 ? u1 : u0);
  const float w = dpp_add<DPP_QUAD_2301>(u2, u2);
  return dpp_add<DPP_QUAD_1032>(lo1 ? v : w, lo1 ? w : v);
}
