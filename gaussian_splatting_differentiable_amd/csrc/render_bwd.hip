// gs_render_bwd: gradients of the blended image with respect to the 9
// screen-space splat parameters (centre x/y, conic a/b/c, opacity, r/g/b).
//
// "What the 3DGS Literature Left on the Table": Step 1 (a) the 9 per-pixel
// derivatives summed over a wave before global atomics; Step 1 (e) the scalar
// accumulator accum = c_behind . dL/dC; Step 4 the walk from the last
// contributor back to the front; Step 5 the same canonical q as the forward
// pass, so both passes take the same hit decisions; Step 6.3 the per-splat
// gradient alpha T (c . dL/dC - accum) and recovery of T by division by (1-alpha).
//
// gfx950 mapping: one wavefront per 8x8 sub-tile, LDS-staged batches of 64
// splats walked back to front; the per-wave cull ballot skips splats that miss
// the sub-tile; per splat with any hit, the 9 values are summed over the 64
// lanes and 9 lanes issue one float atomic add each.
#include "gs_common.h"

namespace {

constexpr float NEG_HALF_LOG2E = -0.72134752044448170368f;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, GS_WAVE);
  return v;
}

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
  const int2 rg = ranges[tile];
  const int start = rg.x;
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
  // walk only as far back as the last splat any lane of this sub-tile blended
  int kmax = lastp;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) kmax = max(kmax, __shfl_xor(kmax, d, GS_WAVE));
  kmax = min(kmax, sub_last[item]);
  const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
  float accum = 0.0f;

  for (int hiE = start + kmax; hiE > start; hiE -= GS_WAVE) {
    const int lo = max(start, hiE - GS_WAVE);
    const int k = lo + lane;
    bool cand = false;
    if (k < hiE) {
      const int id = sorted_ids[k];
      Splat s = splats[id];
      cand = rect_may_hit(s.p0.x, s.p0.y, s.p0.z, s.p0.w, s.p1.x, s.p2.y, hx0, hx1, hy0, hy1);
      s.p2.w = __log2f(s.p1.y);  // the forward pass folds log2(o) the same way
      sbuf[lane] = s;
      sid[lane] = id;
    }
    uint64_t work = __ballot(cand);
    __syncthreads();
    while (work) {
      const int j = 63 - __builtin_clzll(work);  // back to front
      work &= ~(1ull << j);
      const Splat s = sbuf[j];
      const int rel = lo + j - start;
      const float a = s.p0.z, b = s.p0.w, c = s.p1.x;
      const float dx = fx - s.p0.x, dy = fy - s.p0.y;
      const float q = canon_q(a, 2.0f * b, c, dx, dy);
      const bool hit = inside && rel < lastp && (q <= s.p2.y);
      if (__ballot(hit) == 0) continue;
      float gr[9] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (hit) {
        // same alpha as the forward pass: o G = 2^(q (-log2(e)/2) + log2 o)
        const float oG = __builtin_amdgcn_exp2f(fmaf(q, NEG_HALF_LOG2E, s.p2.w));
        const float al = fminf(0.99f, oG);
        T = T * __builtin_amdgcn_rcpf(1.0f - al);
        const float cg = fmaf(s.p1.z, g0, fmaf(s.p1.w, g1, s.p2.x * g2));
        const float diff = cg - accum;
        const float dal = T * diff;
        accum = fmaf(al, diff, accum);
        const float w = al * T;
        gr[6] = w * g0;
        gr[7] = w * g1;
        gr[8] = w * g2;
        if (oG < 0.99f) {
          const float dq = -0.5f * al * dal;
          gr[5] = oG * dal;  // o G dL/dalpha; divided by o once after the sum
          const float m = -2.0f * dq;
          gr[0] = m * fmaf(a, dx, b * dy);
          gr[1] = m * fmaf(b, dx, c * dy);
          gr[2] = dq * (dx * dx);
          gr[3] = 2.0f * dq * (dx * dy);
          gr[4] = dq * (dy * dy);
        }
      }
      float out = 0.0f;
#pragma unroll
      for (int c9 = 0; c9 < 9; c9++) {
        const float sum = wave_sum(gr[c9]);
        out = (lane == c9) ? sum : out;
      }
      if (lane == 5) out *= __builtin_amdgcn_rcpf(s.p1.y);
      if (lane < 9) unsafeAtomicAdd(&grads[9 * (int64_t)sid[j] + lane], out);
    }
    __syncthreads();
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
