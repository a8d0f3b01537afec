// gs_render_bwd: gradients of the blended image with respect to the 9
// screen-space splat parameters (centre x/y, conic a/b/c, opacity, r/g/b).
//
// "What the 3DGS Literature Left on the Table": Step 1 (a) per-pixel
// derivatives summed over a wave before global atomics; Step 1 (e) the scalar
// accumulator accum = c_behind . dL/dC; Step 2 the reduce-scatter that leaves
// the 9 sums on 9 lanes for one atomic instruction; Step 4 the walk from the
// last contributor back to the front; Step 5 branchless alpha = 0 predication
// for missed pixels and one canonical q shared with the forward pass; Step 6.3
// the per-splat term alpha T (c . dL/dC - accum), with log2(o) folded into the
// exponent and o divided back out once after the sum.
//
// gfx950 mapping: one wavefront per 8x8 sub-tile, LDS-staged batches of 64
// splats walked back to front; the next batch's records are fetched while the
// current one is processed; the per-wave cull ballot skips splats that miss the
// sub-tile and a second ballot skips splats no live pixel hits.
#include "gs_common.h"
#include "wave_reduce.h"

namespace {

constexpr float NEG_HALF_LOG2E = -0.72134752044448170368f;

__global__ void __launch_bounds__(256) k_zero(float *__restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n4 = n / 4;
  if (i < n4) reinterpret_cast<float4 *>(p)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i < n - 4 * n4) p[4 * n4 + i] = 0.0f;
}

__global__ void __launch_bounds__(GS_WAVE) k_render_bwd(
    const Splat *__restrict__ splats, const int32_t *__restrict__ sorted_ids,
    const int2 *__restrict__ ranges, CamK cam, const float *__restrict__ Tfin,
    const int32_t *__restrict__ last, const int32_t *__restrict__ sub_last,
    const float *__restrict__ dL, float *__restrict__ grads) {
  __shared__ Splat sbuf[GS_WAVE];
  __shared__ int sid[GS_WAVE];
  const int item = blockIdx.x;
  const int tile = item >> 2, quad = item & 3;
  const int tx = tile % cam.tiles_x, ty = tile / cam.tiles_x;
  const int x0 = tx * 16 + (quad & 1) * 8, y0 = ty * 16 + (quad >> 1) * 8;
  if (x0 >= cam.width || y0 >= cam.height) return;
  const float hx0 = (float)x0 + 0.5f, hx1 = (float)min(x0 + 7, cam.width - 1) + 0.5f;
  const float hy0 = (float)y0 + 0.5f, hy1 = (float)min(y0 + 7, cam.height - 1) + 0.5f;
  const int lane = threadIdx.x;
  const int px = x0 + (lane & 7), py = y0 + (lane >> 3);
  const bool inside = px < cam.width && py < cam.height;
  const int start = ranges[tile].x;
  const int64_t P = (int64_t)cam.width * cam.height;
  const int64_t p = (int64_t)py * cam.width + px;
  float T = 1.0f, g0 = 0.f, g1 = 0.f, g2 = 0.f;
  int lastp = 0;
  if (inside) {
    T = Tfin[p];
    lastp = last[p];
    g0 = dL[p];
    g1 = dL[P + p];
    g2 = dL[2 * P + p];
  }
  // walk back only from the last splat any lane of this sub-tile blended
  int kmax = lastp;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) kmax = max(kmax, __shfl_xor(kmax, d, GS_WAVE));
  kmax = min(kmax, sub_last[item]);
  const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
  const int comp = comp_of_lane(lane);
  float accum = 0.0f;

  // prefetch the first (highest) batch
  int hiE = start + kmax;
  int lo = max(start, hiE - GS_WAVE);
  int pid = -1;
  Splat pre;
  if (lo + lane < hiE) {
    pid = sorted_ids[lo + lane];
    pre = splats[pid];
  }
  while (hiE > start) {
    // stage the prefetched batch [lo, hiE)
    const Splat s_in = pre;
    const int id_in = pid;
    bool cand = false;
    if (id_in >= 0) {
      cand = rect_may_hit(s_in.p0.x, s_in.p0.y, s_in.p0.z, s_in.p0.w, s_in.p1.x, s_in.p2.y, hx0,
                          hx1, hy0, hy1);
      Splat s = s_in;
      s.p2.w = __log2f(s.p1.y);  // the forward pass folds log2(o) the same way
      sbuf[lane] = s;
      sid[lane] = id_in;
    }
    uint64_t work = __ballot(cand);
    // issue the loads of the next (lower) batch
    const int nhi = lo, nlo = max(start, lo - GS_WAVE);
    pid = -1;
    if (nlo + lane < nhi) {
      pid = sorted_ids[nlo + lane];
      pre = splats[pid];
    }
    __syncthreads();
    while (work) {
      const int j = 63 - __builtin_clzll(work);  // back to front
      work &= ~(1ull << j);
      const Splat s = sbuf[j];
      const int rel = lo + j - start;
      const float a = s.p0.z, b = s.p0.w, c = s.p1.x;
      const float dx = fx - s.p0.x, dy = fy - s.p0.y;
      const float adx = a * dx, cdy = c * dy;
      const float q = __builtin_fmaf(cdy, dy, __builtin_fmaf((2.0f * b) * dx, dy, adx * dx));
      const bool hit = inside && rel < lastp && (q <= s.p2.y);
      if (__ballot(hit) == 0) continue;
      // branchless: a missed pixel takes alpha = 0, which leaves T and accum
      // unchanged and contributes zero to every sum
      const float ex = __builtin_amdgcn_exp2f(__builtin_fmaf(q, NEG_HALF_LOG2E, s.p2.w));
      const float oG = hit ? ex : 0.0f;                 // o G
      const float al = fminf(0.99f, oG);
      T = T * __builtin_amdgcn_rcpf(1.0f - al);        // T before this splat
      const float cg = __builtin_fmaf(s.p1.z, g0, __builtin_fmaf(s.p1.w, g1, s.p2.x * g2));
      const float diff = cg - accum;
      const float dal = T * diff;                       // dL/dalpha
      accum = __builtin_fmaf(al, diff, accum);
      const float w = al * T;
      const bool live_g = oG < 0.99f;                   // clamped alpha passes no gradient
      const float m = live_g ? al * dal : 0.0f;         // -2 dL/dq
      float gr[9];
      gr[0] = m * __builtin_fmaf(b, dy, adx);           // dq/dmx = -2 (a dx + b dy)
      gr[1] = m * __builtin_fmaf(b, dx, cdy);
      gr[2] = (-0.5f * m) * (dx * dx);
      gr[3] = -(m * (dx * dy));
      gr[4] = (-0.5f * m) * (dy * dy);
      gr[5] = live_g ? oG * dal : 0.0f;                 // o G dL/dalpha
      gr[6] = w * g0;
      gr[7] = w * g1;
      gr[8] = w * g2;
      float out = reduce_scatter9(gr);
      if (comp == 5) out *= __builtin_amdgcn_rcpf(s.p1.y);
      if (comp >= 0) unsafeAtomicAdd(&grads[9 * (int64_t)sid[j] + comp], out);
    }
    __syncthreads();
    hiE = nhi;
    lo = nlo;
  }
}

}  // namespace

hipError_t gs_launch_render_bwd(const float *splats, const int32_t *sorted_ids,
                                const int32_t *ranges, const CamK &cam, const float *T,
                                const int32_t *last, const int32_t *sub_last, const float *dL,
                                float *grads, int n, hipStream_t st) {
  const int64_t ng = 9 * (int64_t)n;
  if (ng > 0)
    hipLaunchKernelGGL(k_zero, dim3(gs_div_up(ng / 4 + 4, 256)), dim3(256), 0, st, grads, ng);
  const int items = cam.tiles_x * cam.tiles_y * 4;
  hipLaunchKernelGGL(k_render_bwd, dim3(items), dim3(GS_WAVE), 0, st,
                     reinterpret_cast<const Splat *>(splats), sorted_ids,
                     reinterpret_cast<const int2 *>(ranges), cam, T, last, sub_last, dL, grads);
  return hipGetLastError();
}
