/* Oracle: forward blending and analytic backward. TEST INFRASTRUCTURE ONLY.
 *
 * [LOAD-IMB] section 2.1, Eq. 2-3: alpha_i = o_i exp(-q_i/2) with
 * q_i = (x - mu')^T Sigma'^-1 (x - mu'); the pixel colour is
 * C = sum_i c_i alpha_i T_i with T_i = prod_{j<i} (1 - alpha_j), and a pixel
 * stops blending once its transmittance falls below 1e-4.
 * [3DGS-CUDA] Step 1 (b): the alpha cutoff 1/255 is the test q <= tau with
 * tau = 2 ln(255 o). Step 5: forward and backward must take the same hit
 * decision, which is why q has one canonical fp32 form (below).
 * [3DGS-CUDA] Step 1 (a): the 9 screen-space gradients per splat are the 2D
 * centre (x, y), the conic (a, b, c), the opacity and the colour (r, g, b).
 *
 * Readings: pixel (px, py) is sampled at (px + 0.5, py + 0.5); q = a dx^2 +
 * 2 b dx dy + c dy^2; alpha is clamped to 0.99; the stop test T < 1e-4 comes
 * after the blend, so the splat that crosses is blended.
 *
 * Background (not on the pages; the usual completion of Eq. 3): the light that
 * passes every blended splat shows a background colour bg, so
 * C = sum_i c_i alpha_i T_i + T_final bg, with T_final the transmittance after
 * the last blended splat (the T output). A NULL bg is black. The backward also
 * takes an optional per-pixel dL/dT_final.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include "oracle.h"

#define T_STOP 1e-4f
#define ALPHA_MAX 0.99f

/* canonical fp32 quadratic form; fmaf as written, every other op rounded */
static inline float canon_q(const float *s, float dx, float dy) {
  return fmaf(s[4] * dy, dy, fmaf((2.0f * s[3]) * dx, dy, (s[2] * dx) * dx));
}

void or_render_fwd(const float *splats, const int32_t *sorted_ids, const int32_t *ranges,
                   int width, int height, const uint8_t *tile_mask, const float *bg, float *rgb,
                   float *T_final, int32_t *last, uint8_t *knife, int64_t *stats,
                   int32_t *pixel_hits, uint8_t *pair_quarters) {
  const float b0 = bg ? bg[0] : 0.0f, b1 = bg ? bg[1] : 0.0f, b2 = bg ? bg[2] : 0.0f;
  const int tiles_x = (width + 15) / 16;
  const int64_t P = (int64_t)width * height;
  int64_t hits = 0, evals = 0;
#pragma omp parallel for schedule(dynamic, 256) reduction(+ : hits, evals)
  for (int64_t p = 0; p < P; p++) {
    const int px = (int)(p % width), py = (int)(p / width);
    const int t = (py / 16) * tiles_x + px / 16;
    if (tile_mask && !tile_mask[t]) continue;
    const int start = ranges[2 * t], end = ranges[2 * t + 1];
    const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
    float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
    int consumed = end - start;
    int32_t nh = 0;
    uint8_t kn = 0;
    for (int k = start; k < end; k++) {
      const float *s = splats + 12 * (int64_t)sorted_ids[k];
      const float dx = fx - s[0], dy = fy - s[1];
      const float q = canon_q(s, dx, dy);
      evals++;
      if (!(q <= s[9])) continue;
      hits++;
      nh++;
      if (pair_quarters) {
        /* quarter of the tile: bit 0/1 left/right half, bit 1 of the index the lower half */
        const uint8_t bit = (uint8_t)(1u << (((px & 15) >> 3) | (((py & 15) >> 3) << 1)));
#pragma omp atomic
        pair_quarters[k] |= bit;
      }
      const float G = expf(-0.5f * q);
      const float alpha = fminf(ALPHA_MAX, s[5] * G);
      const float w = alpha * T;
      C0 = C0 + w * s[6];
      C1 = C1 + w * s[7];
      C2 = C2 + w * s[8];
      T = T * (1.0f - alpha);
      if (fabsf(T - T_STOP) <= T_STOP * 0x1p-12f) kn = 1;
      if (T < T_STOP) {
        consumed = k - start + 1;
        break;
      }
    }
    rgb[p] = C0 + T * b0;
    rgb[P + p] = C1 + T * b1;
    rgb[2 * P + p] = C2 + T * b2;
    T_final[p] = T;
    last[p] = consumed;
    if (knife) knife[p] = kn;
    if (pixel_hits) pixel_hits[p] = nh;
  }
  if (stats) {
    stats[0] += hits;
    stats[1] += evals;
  }
}

typedef struct {
  uint32_t depth_bits;
  int32_t id;
} order_t;

static int cmp_order(const void *pa, const void *pb) {
  const order_t *a = (const order_t *)pa, *b = (const order_t *)pb;
  if (a->depth_bits != b->depth_bits) return a->depth_bits < b->depth_bits ? -1 : 1;
  return a->id < b->id ? -1 : (a->id > b->id);
}

void or_render_fwd_untiled(int n, const float *splats, int width, int height, float *rgb,
                           float *T_final, int32_t *pixel_hits) {
  order_t *ord = (order_t *)malloc(sizeof(order_t) * (size_t)(n > 0 ? n : 1));
  int m = 0;
  for (int i = 0; i < n; i++) {
    const float *s = splats + 12 * (int64_t)i;
    if (!(s[9] > 0.0f)) continue;
    union { float f; uint32_t u; } db;
    db.f = s[10];
    ord[m].depth_bits = db.u;
    ord[m].id = i;
    m++;
  }
  qsort(ord, (size_t)m, sizeof(order_t), cmp_order);
  const int64_t P = (int64_t)width * height;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t p = 0; p < P; p++) {
    const float fx = (float)(p % width) + 0.5f, fy = (float)(p / width) + 0.5f;
    float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
    int32_t nh = 0;
    for (int k = 0; k < m; k++) {
      const float *s = splats + 12 * (int64_t)ord[k].id;
      const float dx = fx - s[0], dy = fy - s[1];
      const float q = canon_q(s, dx, dy);
      if (!(q <= s[9])) continue;
      nh++;
      const float G = expf(-0.5f * q);
      const float alpha = fminf(ALPHA_MAX, s[5] * G);
      const float w = alpha * T;
      C0 = C0 + w * s[6];
      C1 = C1 + w * s[7];
      C2 = C2 + w * s[8];
      T = T * (1.0f - alpha);
      if (T < T_STOP) break;
    }
    rgb[p] = C0;
    rgb[P + p] = C1;
    rgb[2 * P + p] = C2;
    T_final[p] = T;
    if (pixel_hits) pixel_hits[p] = nh;
  }
  free(ord);
}

void or_render_fwd_values(const float *splats_dec, const double *splats_val,
                          const int32_t *sorted_ids, const int32_t *ranges, int width, int height,
                          const int32_t *last, const double *bg, double *rgb, double *T_final) {
  const int tiles_x = (width + 15) / 16;
  const int64_t P = (int64_t)width * height;
#pragma omp parallel for schedule(dynamic, 64)
  for (int64_t p = 0; p < P; p++) {
    const int px = (int)(p % width), py = (int)(p / width);
    const int t = (py / 16) * tiles_x + px / 16;
    const int start = ranges[2 * t];
    const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
    double T = 1.0, C[3] = {0, 0, 0};
    for (int k = start; k < start + last[p]; k++) {
      const int64_t id = sorted_ids[k];
      const float *sd = splats_dec + 12 * id;
      if (!(canon_q(sd, fx - sd[0], fy - sd[1]) <= sd[9])) continue;
      const double *s = splats_val + 12 * id;
      const double dx = (px + 0.5) - s[0], dy = (py + 0.5) - s[1];
      const double q = s[2] * dx * dx + 2.0 * s[3] * dx * dy + s[4] * dy * dy;
      const double alpha = fmin(0.99, s[5] * exp(-0.5 * q));
      for (int ch = 0; ch < 3; ch++) C[ch] += s[6 + ch] * alpha * T;
      T *= (1.0 - alpha);
    }
    for (int ch = 0; ch < 3; ch++) rgb[ch * P + p] = C[ch] + (bg ? T * bg[ch] : 0.0);
    T_final[p] = T;
  }
}

typedef struct {
  int64_t k;  /* list position of the hit */
  double dx, dy, alpha, G, T, cg;
  int clamped;
} hit_t;

/* The backward, deterministically: every tile is one task (tiles own disjoint
 * list ranges), its pixels run in row-major order and each hit's 9 terms are
 * summed into the fp64 accumulator of its list position; the per-position
 * sums are then added into their splat's row in list order. The result does
 * not depend on the number of threads or their timing. */
void or_render_bwd(const float *splats, const int32_t *sorted_ids, const int32_t *ranges,
                   int width, int height, const int32_t *last, const float *dL_drgb,
                   const float *bg, const float *dL_dT, int n, double *grads) {
  const int tiles_x = (width + 15) / 16, tiles_y = (height + 15) / 16;
  const int ntiles = tiles_x * tiles_y;
  const int64_t P = (int64_t)width * height;
  const int64_t npairs = ntiles > 0 ? ranges[2 * (ntiles - 1) + 1] : 0;
  int maxlen = 1;
  for (int t = 0; t < ntiles; t++) {
    int len = ranges[2 * t + 1] - ranges[2 * t];
    if (len > maxlen) maxlen = len;
  }
  double *pg = (double *)calloc((size_t)(npairs > 0 ? npairs : 1) * 9, sizeof(double));
  memset(grads, 0, sizeof(double) * 9 * (size_t)n);
#pragma omp parallel
  {
    hit_t *H = (hit_t *)malloc(sizeof(hit_t) * (size_t)maxlen);
#pragma omp for schedule(dynamic, 1)
    for (int t = 0; t < ntiles; t++) {
      const int start = ranges[2 * t];
      const int tx = t % tiles_x, ty = t / tiles_x;
      for (int py = 16 * ty; py < 16 * ty + 16 && py < height; py++) {
        for (int px = 16 * tx; px < 16 * tx + 16 && px < width; px++) {
          const int64_t p = (int64_t)py * width + px;
          const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
          const double g[3] = {dL_drgb[p], dL_drgb[P + p], dL_drgb[2 * P + p]};
          /* forward in fp64 over the frozen hit set (no division) */
          int m = 0;
          double T = 1.0;
          for (int k = start; k < start + last[p]; k++) {
            const float *s = splats + 12 * (int64_t)sorted_ids[k];
            if (!(canon_q(s, fx - s[0], fy - s[1]) <= s[9])) continue;
            hit_t *h = &H[m++];
            h->k = k;
            h->dx = (px + 0.5) - (double)s[0];
            h->dy = (py + 0.5) - (double)s[1];
            const double q = (double)s[2] * h->dx * h->dx + 2.0 * (double)s[3] * h->dx * h->dy +
                             (double)s[4] * h->dy * h->dy;
            h->G = exp(-0.5 * q);
            const double oG = (double)s[5] * h->G;
            h->clamped = !(oG < 0.99);
            h->alpha = h->clamped ? 0.99 : oG;
            h->T = T;
            h->cg = (double)s[6] * g[0] + (double)s[7] * g[1] + (double)s[8] * g[2];
            T *= (1.0 - h->alpha);
          }
          /* dC/dalpha_k = T_k c_k - (sum_{j>k} alpha_j T_j c_j + T_final bg) / (1 - alpha_k)
           * and dT_final/dalpha_k = -T_final / (1 - alpha_k): both behind-terms start the
           * suffix (T holds T_final here) */
          const double bgg =
              bg ? (double)bg[0] * g[0] + (double)bg[1] * g[1] + (double)bg[2] * g[2] : 0.0;
          double suffix = T * (bgg + (dL_dT ? (double)dL_dT[p] : 0.0));
          for (int j = m - 1; j >= 0; j--) {
            const hit_t *h = &H[j];
            const float *s = splats + 12 * (int64_t)sorted_ids[h->k];
            const double dalpha = h->T * h->cg - suffix / (1.0 - h->alpha);
            suffix += h->cg * h->alpha * h->T;
            double gr[9];
            const double wT = h->alpha * h->T;
            gr[6] = wT * g[0];
            gr[7] = wT * g[1];
            gr[8] = wT * g[2];
            double dq = 0.0;
            gr[5] = 0.0;
            if (!h->clamped) {
              gr[5] = h->G * dalpha;
              dq = -0.5 * h->alpha * dalpha;
            }
            const double a = s[2], b = s[3], c = s[4];
            /* q = a dx^2 + 2 b dx dy + c dy^2 with dx = px + 0.5 - mx */
            gr[0] = -2.0 * dq * (a * h->dx + b * h->dy);
            gr[1] = -2.0 * dq * (b * h->dx + c * h->dy);
            gr[2] = dq * h->dx * h->dx;
            gr[3] = 2.0 * dq * h->dx * h->dy;
            gr[4] = dq * h->dy * h->dy;
            double *acc = pg + 9 * h->k;
            for (int i = 0; i < 9; i++) acc[i] += gr[i];
          }
        }
      }
    }
    free(H);
  }
  for (int64_t k = 0; k < npairs; k++) {
    double *row = grads + 9 * (int64_t)sorted_ids[k];
    for (int i = 0; i < 9; i++) row[i] += pg[9 * k + i];
  }
  free(pg);
}
