// The canonical hit test and the conservative sub-tile cull of the raster
// kernels. Host and device compile the same code (the tests run the cull on the
// CPU over every sub-tile of random, needle-thin and screen-sized splats).
//
// "What the 3DGS Literature Left on the Table", Step 5: the forward and the
// backward pass must take the same hit decision from one canonical fp32 form of
// q; Step 1 (c): a batch of staged splats is culled against each wavefront's
// part of the tile before any pixel evaluates it.
#pragma once
#include <hip/hip_runtime.h>

// Canonical fp32 quadratic form of the conic at offset (dx, dy), with b2 = 2b.
// Forward, backward and the sub-tile cull take the hit decision from exactly
// this expression: q <= tau.
__host__ __device__ __forceinline__ float canon_q(float a, float b2, float c, float dx, float dy) {
  return __builtin_fmaf(c * dy, dy, __builtin_fmaf(b2 * dx, dy, (a * dx) * dx));
}

// Conservative test: can the ellipse q <= tau touch any sample point of the
// rectangle [x0,x1] x [y0,y1] (pixel-centre coordinates)? Computes the minimum
// of q over the rectangle widened by 1/64 px (a convex quadratic whose centre
// lies outside takes its minimum on an edge that faces the centre, at the 1D
// minimum clamped to the edge) and compares it with
//   tau (1 + 2^-7) + 2^-17 S,   S = a DX^2 + 2 |b| DX DY + c DY^2,
// DX, DY the largest offsets from the centre over the rectangle. S bounds the
// magnitude of the terms of q anywhere in the rectangle, so 2^-17 S exceeds the
// rounding error of the canonical q at any pixel plus that of the minimum here
// (each below 2^-21 S: a handful of roundings of terms no larger than S) even
// where the terms cancel, as they do along a long, thin, tilted splat. Never
// rejects a rectangle that holds a hit pixel; may accept a few extra.
__host__ __device__ __forceinline__ bool rect_may_hit(float mx, float my, float a, float b,
                                                      float c, float tau, float x0, float x1,
                                                      float y0, float y1) {
#pragma clang fp contract(off)
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
  const float DX = fmaxf(fabsf(x0 - mx), fabsf(x1 - mx));
  const float DY = fmaxf(fabsf(y0 - my), fabsf(y1 - my));
  const float S = a * DX * DX + 2.0f * fabsf(b) * DX * DY + c * DY * DY;
  return qmin <= tau * 1.0078125f + S * 0x1p-17f;
}
