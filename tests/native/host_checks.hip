// Host-side checks of code the raster kernels share with the host: the sub-tile
// cull (cull.h) and the forward state's layout (render_common.h). Built for the
// host only by the CPU tests; it calls the same inline functions the kernels do.
#include <stdint.h>
#include <math.h>

#include "cull.h"
#include "render_common.h"

// Bytes of the forward state for T tiles and a pair capacity, and the pair
// capacity a state of `bytes` bytes serves (what the forward checks a frame
// against).
extern "C" int64_t state_bytes(int T, int64_t cap) { return (int64_t)fwd_layout(T, cap).total; }
extern "C" int64_t state_capacity(int T, int64_t bytes) {
  return fwd_state_capacity(T, (size_t)bytes);
}

// For every sub-tile that a splat record could touch, whether some pixel of it
// passes the canonical hit test, and whether the cull keeps it.
// records [n][12] (mx, my, a, b, c, o, r, g, b, tau, depth, view).
// out[0] += sub-tiles holding a hit that the cull rejects (must stay 0)
// out[1] += sub-tiles holding a hit; out[2] += sub-tiles kept without a hit.
extern "C" void cull_check(int n, const float *rec, int width, int height, int64_t *out) {
  for (int i = 0; i < n; i++) {
    const float *s = rec + 12 * (int64_t)i;
    const float mx = s[0], my = s[1], a = s[2], b = s[3], c = s[4], tau = s[9];
    if (!(tau > 0.0f)) continue;
    // the ellipse's bounding box in pixels (fp64, generous), clipped to the image
    const double det = (double)a * c - (double)b * b;
    if (!(det > 0.0)) continue;
    const double rx = sqrt((double)c * tau / det) + 2.0, ry = sqrt((double)a * tau / det) + 2.0;
    const int sx0 = (int)fmax(0.0, floor((mx - rx) / 8.0)), sx1 = (int)fmin((width - 1) / 8, floor((mx + rx) / 8.0));
    const int sy0 = (int)fmax(0.0, floor((my - ry) / 8.0)), sy1 = (int)fmin((height - 1) / 8, floor((my + ry) / 8.0));
    for (int sy = sy0; sy <= sy1; sy++) {
      for (int sx = sx0; sx <= sx1; sx++) {
        const int x0 = 8 * sx, y0 = 8 * sy;
        const int x1 = x0 + 7 < width - 1 ? x0 + 7 : width - 1;
        const int y1 = y0 + 7 < height - 1 ? y0 + 7 : height - 1;
        bool hit = false;
        for (int py = y0; py <= y1 && !hit; py++)
          for (int px = x0; px <= x1 && !hit; px++) {
            const float dx = ((float)px + 0.5f) - mx, dy = ((float)py + 0.5f) - my;
            hit = canon_q(a, 2.0f * b, c, dx, dy) <= tau;
          }
        const bool kept = rect_may_hit(mx, my, a, b, c, tau, (float)x0 + 0.5f, (float)x1 + 0.5f,
                                       (float)y0 + 0.5f, (float)y1 + 0.5f);
        if (hit) out[1]++;
        if (hit && !kept) out[0]++;
        if (!hit && kept) out[2]++;
      }
    }
  }
}
