/* Oracle: opacity-aware exact conic-tile binning, fp32 mirror mode.
 * TEST INFRASTRUCTURE ONLY.
 *
 * [3DGS-CUDA] Step 1 (b) and Figure 3 (right): a splat's alpha can exceed the
 * 1/255 cutoff only inside the ellipse q(d) <= 2 ln(255 o) = tau; for each tile
 * row that the ellipse covers, the quadratic boundary dx(dy) is solved in closed
 * form to get the row's exact horizontal tile span [tx0, tx1).
 *
 * Reading (the pages leave the rectangle and the rounding open): tile (tx, ty)
 * is emitted when the ellipse q <= tau*(1 + 2^-10) meets the tile's pixel-sample
 * hull [16tx+0.5, min(16tx+15.5, W-0.5)] x [16ty+0.5, min(16ty+15.5, H-0.5)]
 * widened by 2^-8 px on every side. The guard makes every pixel whose
 * canonical q <= tau fall in an emitted tile.
 *
 * The operation sequence below is the canonical one: plain fp32 operations,
 * round-to-nearest, correctly rounded sqrt and division, fmaf only where
 * written, no transcendental (tau comes from the record).
 */
#include <math.h>
#include "oracle.h"

#define GUARD_TAU 1.0009765625f      /* 1 + 2^-10 */
#define LO_EDGE 15.50390625f         /* 15.5 + 2^-8 */
#define HI_EDGE 0.49609375f          /* 0.5 - 2^-8 */
#define GUARD_PX 0.00390625f         /* 2^-8 */

static float clampf(float v, float lo, float hi) { return fminf(fmaxf(v, lo), hi); }

/* Calls emit(tile) for every emitted tile in (ty, tx) ascending order; returns
   the number of emitted tiles. */
typedef void (*emit_fn)(void *ctx, int tile);

static int bin_splat(const float *s, int W, int H, emit_fn emit, void *ctx) {
  const int tiles_x = (W + 15) / 16, tiles_y = (H + 15) / 16;
  const float mx = s[0], my = s[1], a = s[2], b = s[3], c = s[4], tau = s[9];
  if (!(tau > 0.0f)) return 0;
  const float tb = tau * GUARD_TAU;
  const float det = fmaf(a, c, -(b * b));
  if (!(det > 0.0f) || !(a > 0.0f) || !(c > 0.0f)) return 0;
  const float at = a * tb;
  const float ry = sqrtf(at / det);
  const float rx = sqrtf((c * tb) / det);
  const float sx = sqrtf(tb / (c * det));
  const float dys = -(b * sx); /* dy of the rightmost point; the leftmost is at -dys */
  const float Wf = (float)W, Hf = (float)H;

  const float ytop = my - ry, ybot = my + ry;
  const int ty_a = (int)clampf(ceilf((ytop - LO_EDGE) * 0.0625f), 0.0f, (float)tiles_y);
  const int ty_b = (int)clampf(floorf((ybot - HI_EDGE) * 0.0625f) + 1.0f, 0.0f, (float)tiles_y);
  int count = 0;
  for (int ty = ty_a; ty < ty_b; ty++) {
    const float y0 = (float)(16 * ty) + HI_EDGE;
    const float y1 = fminf((float)(16 * ty) + 15.5f, Hf - 0.5f) + GUARD_PX;
    const float d0 = y0 - my, d1 = y1 - my;
    if (d0 > ry || d1 < -ry) continue;
    const float e0 = fmaxf(d0, -ry), e1 = fminf(d1, ry);
    float xr, xl;
    if (e0 <= dys && dys <= e1) {
      xr = mx + rx;
    } else {
      const float dy = fminf(fmaxf(dys, e0), e1);
      const float D = fmaxf(at - (det * dy) * dy, 0.0f);
      xr = mx + (sqrtf(D) - b * dy) / a;
    }
    const float ndys = -dys;
    if (e0 <= ndys && ndys <= e1) {
      xl = mx - rx;
    } else {
      const float dy = fminf(fmaxf(ndys, e0), e1);
      const float D = fmaxf(at - (det * dy) * dy, 0.0f);
      xl = mx + (-(b * dy) - sqrtf(D)) / a;
    }
    if (xl > Wf - HI_EDGE) continue; /* right of the last sample column */
    const int tx0 = (int)clampf(ceilf((xl - LO_EDGE) * 0.0625f), 0.0f, (float)tiles_x);
    const int tx1 = (int)clampf(floorf((xr - HI_EDGE) * 0.0625f) + 1.0f, 0.0f, (float)tiles_x);
    for (int tx = tx0; tx < tx1; tx++) {
      if (emit) emit(ctx, ty * tiles_x + tx);
      count++;
    }
  }
  return count;
}

void or_bin_count(int n, const float *splats, int width, int height, int32_t *counts) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; i++) counts[i] = bin_splat(splats + 12 * (int64_t)i, width, height, 0, 0);
}

typedef struct {
  uint64_t *keys;
  int32_t *ids;
  int64_t pos;
  uint32_t depth_bits;
  int32_t id;
} emit_ctx;

static void emit_pair(void *vctx, int tile) {
  emit_ctx *e = (emit_ctx *)vctx;
  e->keys[e->pos] = ((uint64_t)(uint32_t)tile << 32) | e->depth_bits;
  e->ids[e->pos] = e->id;
  e->pos++;
}

void or_bin_emit(int n, const float *splats, int width, int height, const int64_t *offsets,
                 uint64_t *keys, int32_t *ids) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < n; i++) {
    const float *s = splats + 12 * (int64_t)i;
    union { float f; uint32_t u; } db;
    db.f = s[10];
    emit_ctx e = {keys, ids, offsets[i], db.u, i};
    bin_splat(s, width, height, emit_pair, &e);
  }
}
