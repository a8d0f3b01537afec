// Canonical fp32 row spans of the opacity-aware exact conic-tile binning.
//
// "What the 3DGS Literature Left on the Table", Step 1 (b), Figure 3 (right):
// for every tile row the ellipse q(d) <= tau covers, the row's horizontal tile
// span is solved in closed form from the quadratic boundary dx(dy).
// Reading: tile (tx, ty) is emitted when the ellipse q <= tau (1 + 2^-10) meets
// the tile's pixel-sample hull widened by 2^-8 px.
//
// Every translation unit that includes this header must be compiled with
// -ffp-contract=off: each operation rounds on its own and fmaf appears only
// where written, so the emitted tiles are reproducible bit for bit.
#pragma once
#include "gs_common.h"

#define GUARD_TAU 1.0009765625f  // 1 + 2^-10
#define LO_EDGE 15.50390625f     // 15.5 + 2^-8
#define HI_EDGE 0.49609375f      // 0.5 - 2^-8
#define GUARD_PX 0.00390625f     // 2^-8

struct RowSpans {
  float mx, my, a, b, c, det, at, rx, ry, dys;
  int ty_a, ty_b;  // tile rows of the record's own view, [0, vty)
  int row0;        // the view's first tile row in the batch image
  bool ok;
};

__device__ __forceinline__ float clampf(float v, float lo, float hi) { return fminf(fmaxf(v, lo), hi); }

// vty: tile rows per view; views: views in the batch. Spans are solved in the
// record's own view (its coordinates); a tile row ty of that view is row
// row0 + ty of the batch image. A record naming no view of the batch has none.
__device__ __forceinline__ RowSpans spans_setup(const Splat &s, int vty, int views) {
  RowSpans r;
  r.mx = s.p0.x; r.my = s.p0.y; r.a = s.p0.z; r.b = s.p0.w; r.c = s.p1.x;
  const float tau = s.p2.y;
  const int view = record_view(s);
  r.ok = false;
  r.ty_a = r.ty_b = 0;
  r.row0 = view * vty;
  const int tiles_y = vty;
  if (!(tau > 0.0f) || view < 0 || view >= views) return r;
  const float tb = tau * GUARD_TAU;
  r.det = __builtin_fmaf(r.a, r.c, -(r.b * r.b));
  if (!(r.det > 0.0f) || !(r.a > 0.0f) || !(r.c > 0.0f)) return r;
  r.at = r.a * tb;
  r.ry = sqrtf(r.at / r.det);
  r.rx = sqrtf((r.c * tb) / r.det);
  const float sx = sqrtf(tb / (r.c * r.det));
  r.dys = -(r.b * sx);
  const float ytop = r.my - r.ry, ybot = r.my + r.ry;
  r.ty_a = (int)clampf(ceilf((ytop - LO_EDGE) * 0.0625f), 0.0f, (float)tiles_y);
  r.ty_b = (int)clampf(floorf((ybot - HI_EDGE) * 0.0625f) + 1.0f, 0.0f, (float)tiles_y);
  r.ok = true;
  return r;
}

// Column span [tx0, tx1) of tile row ty; empty when tx1 <= tx0.
__device__ __forceinline__ void row_span(const RowSpans &r, int ty, int W, int H, int tiles_x,
                                         int &tx0, int &tx1) {
  tx0 = tx1 = 0;
  const float y0 = (float)(16 * ty) + HI_EDGE;
  const float y1 = fminf((float)(16 * ty) + 15.5f, (float)H - 0.5f) + GUARD_PX;
  const float d0 = y0 - r.my, d1 = y1 - r.my;
  if (d0 > r.ry || d1 < -r.ry) return;
  const float e0 = fmaxf(d0, -r.ry), e1 = fminf(d1, r.ry);
  float xr, xl;
  if (e0 <= r.dys && r.dys <= e1) {
    xr = r.mx + r.rx;
  } else {
    const float dy = fminf(fmaxf(r.dys, e0), e1);
    const float D = fmaxf(r.at - (r.det * dy) * dy, 0.0f);
    xr = r.mx + (sqrtf(D) - r.b * dy) / r.a;
  }
  const float ndys = -r.dys;
  if (e0 <= ndys && ndys <= e1) {
    xl = r.mx - r.rx;
  } else {
    const float dy = fminf(fmaxf(ndys, e0), e1);
    const float D = fmaxf(r.at - (r.det * dy) * dy, 0.0f);
    xl = r.mx + (-(r.b * dy) - sqrtf(D)) / r.a;
  }
  if (xl > (float)W - HI_EDGE) return;
  tx0 = (int)clampf(ceilf((xl - LO_EDGE) * 0.0625f), 0.0f, (float)tiles_x);
  tx1 = (int)clampf(floorf((xr - HI_EDGE) * 0.0625f) + 1.0f, 0.0f, (float)tiles_x);
}
