// Internal device helpers shared by the HIP kernels of the rasterizer.
// gfx950 only: wave64, 16x16 tiles, 8x8 sub-tiles per wavefront.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gs.h"

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

// Value of v in the first active lane, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_first(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Canonical fp32 quadratic form of the conic at offset (dx, dy). Forward,
// backward and the sub-tile cull must all take the hit decision from exactly
// this expression (Step 5 of the literature page: fwd and bwd agree bit-for-bit).
__device__ __forceinline__ float canon_q(float a, float b2, float c, float dx, float dy) {
  return __builtin_fmaf(c * dy, dy, __builtin_fmaf(b2 * dx, dy, (a * dx) * dx));
}

// Conservative test: can the ellipse q <= tau touch any sample point of the
// rectangle [x0,x1] x [y0,y1] (pixel-centre coordinates)? Computes the minimum
// of q over the rectangle widened by 1/64 px, compared with tau * (1 + 2^-7).
// Never rejects a rectangle that holds a hit pixel; may accept a few extra.
__device__ __forceinline__ bool rect_may_hit(float mx, float my, float a, float b, float c,
                                             float tau, float x0, float x1, float y0, float y1) {
  if (!(tau > 0.0f)) return false;
  const float g = 0.015625f;
  x0 -= g; x1 += g; y0 -= g; y1 += g;
  const float cxp = fminf(fmaxf(mx, x0), x1);
  const float cyp = fminf(fmaxf(my, y0), y1);
  if (cxp == mx && cyp == my) return true;
  float qmin = 3.0e38f;
  // a horizontal edge faces the centre when the centre lies above/below the box
  if (cyp != my) {
    const float dy = cyp - my;
    const float dx = fminf(fmaxf(-b * dy / a, x0 - mx), x1 - mx);
    qmin = fminf(qmin, a * dx * dx + 2.0f * b * dx * dy + c * dy * dy);
  }
  if (cxp != mx) {
    const float dx = cxp - mx;
    const float dy = fminf(fmaxf(-b * dx / c, y0 - my), y1 - my);
    qmin = fminf(qmin, a * dx * dx + 2.0f * b * dx * dy + c * dy * dy);
  }
  return qmin <= tau * 1.0078125f;
}

static inline int gs_div_up(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }
