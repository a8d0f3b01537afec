// Internal device helpers shared by the HIP kernels of the rasterizer.
// gfx950 only: wave64, 16x16 tiles, 8x8 sub-tiles per wavefront.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gs.h"
#include "cull.h"

#define GS_WAVE 64
#define GS_TILE_PX 256
#define GS_MAX_TILES 65535

// Splat record as three 16-byte vectors: (mx,my,a,b) (c,o,r,g) (b,tau,depth,pad).
struct __align__(16) Splat {
  float4 p0, p1, p2;
};

// Camera constants prepared on the host for the kernels.
struct CamK {
  int width, height, tiles_x, tiles_y;
  float fx, fy, cx, cy;
  float R[9];
  float t[3];
  float centre[3];  // camera centre in world coordinates, -R^T t
  float znear, lowpass;
  float bg[3];      // background colour seen through the final transmittance
  int bg_on;        // bg is not black (or the backward has a dL/dT_final)
  // A batch of `views` cameras of one size is one image of views x vty tile
  // rows: view v owns tile rows [v vty, (v + 1) vty) and pixel rows
  // [v height, (v + 1) height) of the outputs; tiles_y = views x vty. A splat
  // record carries its view in its pad word (int bits; 0 for a single view).
  int views, vty;
  int view;         // the projection's camera index within its batch
};

// The tile schedule a sort may build beside its last tile pass
// (gs_sort_keys_plan): where, with which knobs and worker count.
struct SortPlan {
  void *fwd_state;
  int mode, force_k, force_h, nblocks;
  double lambda_, beta, eps;
  int64_t cap;  // the pairs the forward state holds
};

// View index stored in a splat record's pad word.
__device__ __forceinline__ int record_view(const Splat &s) { return __float_as_int(s.p2.w); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Lanes of the wave where p holds, as a scalar mask (the bool goes straight to
// the ballot, with no round trip through a 0/1 vector register).
__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Orders this wave's LDS stores before its later LDS loads (and the reverse),
// for LDS that only this wave uses: no workgroup barrier is needed.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// First error of a frame wins: the status word keeps the first non-OK code.
__device__ __forceinline__ void report_status(int32_t *status, int32_t code) {
  atomicCAS(status, (int32_t)GS_OK, code);
}

// Value of v in the first active lane, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_first(int v) { return __builtin_amdgcn_readfirstlane(v); }

static inline int gs_div_up(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
