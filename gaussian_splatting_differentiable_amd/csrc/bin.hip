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
// Kernels: the counting pass and the prefix sum of the counts (sort.hip: the
// offsets and the status, plus what the sort needs from the same pass over the
// records), then, only when the caller asks for them, k_bin_emit (keys/ids at
// the offsets in splat-id order). The sort stage re-emits the pairs directly
// in depth order, so the frame does not need the id-order list.
#include "bin_spans.h"

namespace {

__global__ void __launch_bounds__(256) k_bin_emit(int n, const Splat *__restrict__ splats, int W,
                                                  int H, int tiles_x, int vty, int views,
                                                  const int32_t *__restrict__ offsets,
                                                  int64_t capacity, uint64_t *__restrict__ keys,
                                                  int32_t *__restrict__ ids) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = offsets[n];
  if (total > capacity || i >= n) return;
  const Splat s = splats[i];
  const RowSpans r = spans_setup(s, vty, views);
  if (!r.ok) return;
  const uint64_t depth_bits = (uint64_t)__float_as_uint(s.p2.z);
  int64_t pos = offsets[i];
  for (int ty = r.ty_a; ty < r.ty_b; ty++) {
    int a, b;
    row_span(r, ty, W, H, tiles_x, a, b);
    for (int tx = a; tx < b; tx++) {
      keys[pos] = ((uint64_t)(uint32_t)((r.row0 + ty) * tiles_x + tx) << 32) | depth_bits;
      ids[pos] = i;
      pos++;
    }
  }
}

}  // namespace

hipError_t gs_launch_bin_count(int n, const float *splats, const CamK &cam, int64_t cap,
                               int32_t *offsets, int32_t *tile_counts, int32_t *status, void *ws,
                               hipStream_t st);

hipError_t gs_launch_bin(int n, const float *splats, const CamK &cam, int64_t capacity,
                         int32_t *offsets, int32_t *tile_counts, uint64_t *keys, int32_t *ids,
                         int32_t *status, void *ws, hipStream_t st) {
  const Splat *sp = reinterpret_cast<const Splat *>(splats);
  dim3 block(256), grid(gs_div_up(n > 0 ? n : 1, 256));
  hipError_t e = gs_launch_bin_count(n, splats, cam, capacity, offsets, tile_counts, status, ws, st);
  if (e != hipSuccess || !keys) return e;
  hipLaunchKernelGGL(k_bin_emit, grid, block, 0, st, n, sp, cam.width, cam.height, cam.tiles_x,
                     cam.vty, cam.views, offsets, capacity, keys, ids);
  return hipGetLastError();
}
