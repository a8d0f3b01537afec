// gs_bin_tiles: exact opacity-aware conic-tile binning.
//
// "What the 3DGS Literature Left on the Table", Step 1 (b), Figure 3 (right):
// alpha can reach the 1/255 cutoff only inside the ellipse q(d) <= 2 ln(255 o);
// for every tile row the ellipse covers, the row's horizontal tile span is
// solved in closed form from the quadratic boundary dx(dy), so no rejected
// tile is ever evaluated.
//
// Emission rule (a reading; the page leaves the rectangle and the rounding
// open): tile (tx, ty) is emitted when the ellipse q <= tau (1 + 2^-10) meets
// the tile's pixel-sample hull, widened by 2^-8 px. This TU is compiled with
// -ffp-contract=off: every operation below rounds on its own and fmaf appears
// only where written, so the emitted pairs are reproducible bit for bit.
//
// Kernels: k_bin_count (per-splat pair count into offsets[]), a device-wide
// exclusive scan (scan.hip), then k_bin_emit (keys/ids at the offsets).
#include "gs_common.h"

namespace {

#define GUARD_TAU 1.0009765625f  // 1 + 2^-10
#define LO_EDGE 15.50390625f     // 15.5 + 2^-8
#define HI_EDGE 0.49609375f      // 0.5 - 2^-8
#define GUARD_PX 0.00390625f     // 2^-8

struct RowSpans {
  float mx, my, a, b, c, det, at, rx, ry, dys;
  int ty_a, ty_b;
  bool ok;
};

__device__ __forceinline__ float clampf(float v, float lo, float hi) { return fminf(fmaxf(v, lo), hi); }

__device__ __forceinline__ RowSpans spans_setup(const Splat &s, int tiles_y) {
  RowSpans r;
  r.mx = s.p0.x; r.my = s.p0.y; r.a = s.p0.z; r.b = s.p0.w; r.c = s.p1.x;
  const float tau = s.p2.y;
  r.ok = false;
  r.ty_a = r.ty_b = 0;
  if (!(tau > 0.0f)) return r;
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

__global__ void __launch_bounds__(256) k_bin_count(int n, const Splat *__restrict__ splats, int W,
                                                   int H, int tiles_x, int tiles_y,
                                                   int32_t *__restrict__ counts) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const RowSpans r = spans_setup(splats[i], tiles_y);
  int cnt = 0;
  if (r.ok) {
    for (int ty = r.ty_a; ty < r.ty_b; ty++) {
      int a, b;
      row_span(r, ty, W, H, tiles_x, a, b);
      cnt += b > a ? b - a : 0;
    }
  }
  counts[i] = cnt;
}

__global__ void __launch_bounds__(256) k_bin_emit(int n, const Splat *__restrict__ splats, int W,
                                                  int H, int tiles_x, int tiles_y,
                                                  const int32_t *__restrict__ offsets,
                                                  int64_t capacity, uint64_t *__restrict__ keys,
                                                  int32_t *__restrict__ ids,
                                                  int32_t *__restrict__ status) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = offsets[n];
  if (total > capacity) {
    if (i == 0) *status = GS_ERR_CAPACITY;
    return;
  }
  if (i == 0) *status = GS_OK;
  if (i >= n) return;
  const Splat s = splats[i];
  const RowSpans r = spans_setup(s, tiles_y);
  if (!r.ok) return;
  const uint64_t depth_bits = (uint64_t)__float_as_uint(s.p2.z);
  int64_t pos = offsets[i];
  for (int ty = r.ty_a; ty < r.ty_b; ty++) {
    int a, b;
    row_span(r, ty, W, H, tiles_x, a, b);
    for (int tx = a; tx < b; tx++) {
      keys[pos] = ((uint64_t)(uint32_t)(ty * tiles_x + tx) << 32) | depth_bits;
      ids[pos] = i;
      pos++;
    }
  }
}

}  // namespace

hipError_t gs_launch_scan_i32(const int32_t *in, int32_t *out, int n, int32_t *block_buf,
                              hipStream_t st);

hipError_t gs_launch_bin(int n, const float *splats, const CamK &cam, int64_t capacity,
                         int32_t *offsets, uint64_t *keys, int32_t *ids, int32_t *status,
                         int32_t *scan_buf, hipStream_t st) {
  const Splat *sp = reinterpret_cast<const Splat *>(splats);
  dim3 block(256), grid(gs_div_up(n > 0 ? n : 1, 256));
  if (n > 0)
    hipLaunchKernelGGL(k_bin_count, grid, block, 0, st, n, sp, cam.width, cam.height, cam.tiles_x,
                       cam.tiles_y, offsets);
  // exclusive scan of the n counts, total in offsets[n]
  hipError_t e = gs_launch_scan_i32(offsets, offsets, n, scan_buf, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bin_emit, grid, block, 0, st, n, sp, cam.width, cam.height, cam.tiles_x,
                     cam.tiles_y, offsets, capacity, keys, ids, status);
  return hipGetLastError();
}
