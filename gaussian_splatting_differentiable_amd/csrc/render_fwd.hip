// gs_render_fwd: front-to-back alpha blending of 16x16 tiles.
//
// "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on GPUs",
// section 2.1, Eq. 2-3: alpha = o exp(-q/2); C = sum c alpha T; a pixel stops
// blending once T falls below 1e-4.
// "What the 3DGS Literature Left on the Table": Step 1 (b) the alpha >= 1/255
// cutoff as q <= tau; Step 1 (c) sub-tile culling of staged splat batches with a
// vote (ballot) and a find-first-set worklist; Step 1 (e) base-2 exponential;
// Step 5 branch-light blending with one canonical q for forward and backward;
// Step 6.3 log2(o) folded into the exponent.
//
// gfx950 mapping: one wavefront owns one 8x8 sub-tile (64 lanes = 64 pixels) and
// walks its tile's list in batches of 64 splats that the lanes stage into LDS
// (one record per lane, three 16-byte loads). Each lane tests its staged splat
// against the sub-tile's sample rectangle; the ballot of those tests is the
// worklist, walked on the scalar unit. No barrier is needed: each wave is a
// workgroup.
#include "gs_common.h"

namespace {

constexpr float NEG_HALF_LOG2E = -0.72134752044448170368f;

struct SubTile {
  int tile, quad, x0, y0;
  float hx0, hx1, hy0, hy1;  // sample hull of the sub-tile
  bool empty;
};

__device__ __forceinline__ SubTile subtile_of(int item, const CamK &cam) {
  SubTile st;
  st.tile = item >> 2;
  st.quad = item & 3;
  const int tx = st.tile % cam.tiles_x, ty = st.tile / cam.tiles_x;
  st.x0 = tx * 16 + (st.quad & 1) * 8;
  st.y0 = ty * 16 + (st.quad >> 1) * 8;
  st.empty = st.x0 >= cam.width || st.y0 >= cam.height;
  st.hx0 = (float)st.x0 + 0.5f;
  st.hx1 = (float)min(st.x0 + 7, cam.width - 1) + 0.5f;
  st.hy0 = (float)st.y0 + 0.5f;
  st.hy1 = (float)min(st.y0 + 7, cam.height - 1) + 0.5f;
  return st;
}

__global__ void __launch_bounds__(GS_WAVE) k_render_fwd(
    const Splat *__restrict__ splats, const int32_t *__restrict__ sorted_ids,
    const int2 *__restrict__ ranges, CamK cam, float *__restrict__ rgb, float *__restrict__ Tout,
    int32_t *__restrict__ last, int32_t *__restrict__ sub_last,
    unsigned long long *__restrict__ stats) {
  __shared__ Splat sbuf[GS_WAVE];
  const int item = blockIdx.x;
  const SubTile st = subtile_of(item, cam);
  if (st.empty) {
    if (threadIdx.x == 0) sub_last[item] = 0;
    return;
  }
  const int lane = threadIdx.x;
  const int px = st.x0 + (lane & 7), py = st.y0 + (lane >> 3);
  const bool inside = px < cam.width && py < cam.height;
  const int2 rg = ranges[st.tile];
  const int start = rg.x, end = rg.y;
  const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
  float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
  int lastv = end - start;
  bool alive = inside;
  uint64_t live = __ballot(alive);
  int wlast = 0;
  unsigned long long nhits = 0, nsteps = 0;

  // prefetch the first batch; each batch's loads are issued one batch ahead
  int pid = -1;
  Splat pre;
  if (start + lane < end) {
    pid = sorted_ids[start + lane];
    pre = splats[pid];
  }
  for (int b = start; b < end && live; b += GS_WAVE) {
    bool cand = false;
    if (pid >= 0) {
      Splat s = pre;
      cand = rect_may_hit(s.p0.x, s.p0.y, s.p0.z, s.p0.w, s.p1.x, s.p2.y, st.hx0, st.hx1, st.hy0,
                          st.hy1);
      s.p0.w = 2.0f * s.p0.w;          // 2b, exact
      s.p2.w = __log2f(s.p1.y);        // log2(o) for the folded exponent
      sbuf[lane] = s;
    }
    uint64_t work = __ballot(cand);
    const int nb = b + GS_WAVE;
    pid = -1;
    if (nb + lane < end) {
      pid = sorted_ids[nb + lane];
      pre = splats[pid];
    }
    __syncthreads();
    while (work) {
      const int j = __builtin_ctzll(work);
      work &= work - 1;
      const Splat s = sbuf[j];
      const float dx = fx - s.p0.x, dy = fy - s.p0.y;
      const float q = canon_q(s.p0.z, s.p0.w, s.p1.x, dx, dy);
      const bool hit = alive && (q <= s.p2.y);
      const uint64_t hm = __ballot(hit);
      nsteps++;
      if (hm == 0) continue;
      nhits += __popcll(hm);
      wlast = b + j - start + 1;
      // branchless: a missed pixel blends with alpha = 0
      const float ex = __builtin_amdgcn_exp2f(__builtin_fmaf(q, NEG_HALF_LOG2E, s.p2.w));
      const float al = hit ? fminf(0.99f, ex) : 0.0f;
      const float w = al * T;
      C0 = __builtin_fmaf(w, s.p1.z, C0);
      C1 = __builtin_fmaf(w, s.p1.w, C1);
      C2 = __builtin_fmaf(w, s.p2.x, C2);
      T = T - w;
      const bool stop = hit && (T < 1e-4f);
      if (__ballot(stop)) {
        if (stop) {
          alive = false;
          lastv = b + j - start + 1;
        }
        live = __ballot(alive);
        if (!live) break;
      }
    }
    __syncthreads();
  }
  if (inside) {
    const int64_t P = (int64_t)cam.width * cam.height;
    const int64_t p = (int64_t)py * cam.width + px;
    rgb[p] = C0;
    rgb[P + p] = C1;
    rgb[2 * P + p] = C2;
    Tout[p] = T;
    last[p] = lastv;
  }
  if (lane == 0) {
    sub_last[item] = wlast;
    if (stats) {
      atomicAdd(&stats[0], nhits);
      atomicAdd(&stats[1], nsteps * (unsigned long long)GS_WAVE);
      atomicAdd(&stats[2], nsteps);
    }
  }
}

}  // namespace

hipError_t gs_launch_render_fwd(const float *splats, const int32_t *sorted_ids,
                                const int32_t *ranges, const CamK &cam, float *rgb, float *T,
                                int32_t *last, int32_t *sub_last, int64_t *stats, hipStream_t st) {
  const int items = cam.tiles_x * cam.tiles_y * 4;
  hipLaunchKernelGGL(k_render_fwd, dim3(items), dim3(GS_WAVE), 0, st,
                     reinterpret_cast<const Splat *>(splats), sorted_ids,
                     reinterpret_cast<const int2 *>(ranges), cam, rgb, T, last, sub_last,
                     reinterpret_cast<unsigned long long *>(stats));
  return hipGetLastError();
}
