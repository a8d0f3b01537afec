// Reduce-scatter of the 9 per-lane gradient values of one splat over each
// 32-lane half of a wave (the two halves reduce different splats at once).
//
// "What the 3DGS Literature Left on the Table", Step 2 (Figure 6): instead of 9
// full butterflies, halve the set of live values at each exchange so that the
// sums end on distinct lanes and one atomic instruction writes them all. On
// gfx950, within each half (lane L = 16 r + s, r the row of 16):
//
//   swap16 (v_permlane16_swap, rows 0 <-> 1 of the half), pairs (0,5) (1,6)
//          (2,7) (3,8) (4,-): row 0 keeps components 0-4, row 1 keeps 5-8;
//   ror8   (DPP row_ror:8, lane s <-> s^8) on the pairs (t0,t1) (t2,t3):
//          lanes s < 8 keep t0, t2 and s >= 8 keep t1, t3; t4 is summed on all;
//   mirror (DPP row_half_mirror, lane s <-> s^7 within each 8) on (u0,u1):
//          s mod 8 < 4 keeps u0, else u1; u2 is summed on all;
//   two quad_perm adds (s <-> s^2 on the pair (v, u2), then s <-> s^1).
//
// Lane (r, s) then owns: s = 0 -> {0,5}[r], s = 8 -> {1,6}[r], s = 4 ->
// {2,7}[r], s = 12 -> {3,8}[r], s = 2 and r = 0 -> 4. 22 VALU instructions for
// two splats' 9 sums (the zero operand of the unpaired swap stays in a
// register; the bank-aligned exchanges need no selects).
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

// Component owned by lane (row r, slot s) of its half, or -1.
__device__ __forceinline__ int comp_of_half_lane(int lane) {
  const int r = (lane >> 4) & 1, s = lane & 15;
  if (s == 0) return r ? 5 : 0;
  if (s == 8) return r ? 6 : 1;
  if (s == 4) return r ? 7 : 2;
  if (s == 12) return r ? 8 : 3;
  if (s == 2 && r == 0) return 4;
  return -1;
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

// Reduce g[0..8] over each 32-lane half; returns the half's sum of component
// comp_of_half_lane(lane) on the lanes that own one (partial sums elsewhere).
// zero: a register holding 0.0f (the partner of the unpaired component).
__device__ __forceinline__ float reduce_scatter9_half(const float g[9], float zero) {
  const float t0 = swap_sum16(g[0], g[5]);
  const float t1 = swap_sum16(g[1], g[6]);
  const float t2 = swap_sum16(g[2], g[7]);
  const float t3 = swap_sum16(g[3], g[8]);
  const float t4 = swap_sum16(g[4], zero);
  const bool lo2 = (__lane_id() & 2) == 0;
  // lanes s < 8 of each row (banks 0, 1) keep t0 / t2, lanes s >= 8 t1 / t3
  const float u0 = pair_ror8(t0, t1);
  const float u1 = pair_ror8(t2, t3);
  const float u2 = dpp_add<DPP_ROW_ROR8>(t4, t4);
  // lanes s mod 8 < 4 (banks 0, 2) keep u0, the others u1
  const float v = pair_mirror(u0, u1);
  const float w = dpp_add<DPP_ROW_HALF_MIRROR>(u2, u2);
  float x = dpp_add<DPP_QUAD_2301>(lo2 ? v : w, lo2 ? w : v);
  x = dpp_add<DPP_QUAD_1032>(x, x);
  return x;
}
