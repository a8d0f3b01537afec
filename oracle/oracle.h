/* CPU oracle for the tile-based differentiable Gaussian-splatting rasterizer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The HIP product path
 * neither includes this header nor links this code, and this code includes
 * nothing from the product path.
 *
 * Sources (titles of the pages the method comes from):
 *   [3DGS-CUDA]  "What the 3DGS Literature Left on the Table" (rasterizer
 *                optimisation blog: Steps 1-6, Figures 3-10)
 *   [LOAD-IMB]   "Mitigating SM-Level Load Imbalance in 3D Gaussian
 *                Splatting on GPUs" (section 2.1 Eq. 1-3, section 4 Eq. 4-6)
 *
 * Arithmetic modes
 *   mirror : IEEE fp32, round-to-nearest-even, no contraction (built with
 *            -ffp-contract=off); fmaf only where written. Every DECISION
 *            (tile emission, alpha cutoff, transmittance stop) is taken here.
 *   truth  : fp64 values with the mirror's decisions frozen; used for
 *            projection values and for the analytic backward.
 *
 * Splat record (12 floats): mx, my, a, b, c, o, r, g, b, tau, depth, 0.
 * Culled Gaussians carry tau = -1 and zeros elsewhere.
 * Gradient record (9 values): d mx, d my, d a, d b, d c, d o, d r, d g, d b.
 */
#ifndef GS_ORACLE_H
#define GS_ORACLE_H
#include <stdint.h>

typedef struct {
  int32_t width, height;
  double fx, fy, cx, cy;
  double w2c[12];  /* row-major [R | t] */
  double znear, lowpass;
} or_camera;

/* Real orthonormal SH basis (degree <= 3) at unit direction d; Y has (deg+1)^2 entries. */
void or_sh_basis(int degree, const double *d, double *Y);

/* Projection (EWA, Eq. 1 of [LOAD-IMB]) in fp64; writes fp32 records and,
   if splats64 != NULL, the unrounded fp64 records. */
void or_project(int n, const float *means, const float *log_scales, const float *quats,
                const float *opac, const float *sh, int degree, const or_camera *cam,
                float *splats, double *splats64);

/* The projection on fp64 inputs (fp64 records only): the reference for finite
   differences of or_project_bwd. */
void or_project64(int n, const double *means, const double *log_scales, const double *quats,
                  const double *opac, const double *sh, int degree, const or_camera *cam,
                  double *splats64);

/* The SH basis of or_sh_basis as polynomials of the direction, with their
   gradients dY[3k + j] = dY_k/dd_j (degree <= 3). */
void or_sh_cart(int degree, const double *d, double *Y, double *dY);

/* Backward of the projection: dL/d(mean, log-scales, quaternion, opacity, SH)
   from dL/d of the record's first nine entries (dsplat [n][9]), in fp64.
   Culled Gaussians get zeros. */
void or_project_bwd(int n, const float *means, const float *log_scales, const float *quats,
                    const float *opac, const float *sh, int degree, const or_camera *cam,
                    const double *dsplat, double *gmeans, double *gls, double *gquats,
                    double *gopac, double *gsh);

/* Opacity-aware exact conic-tile binning ([3DGS-CUDA] Step 1 (b), Figure 3). */
void or_bin_count(int n, const float *splats, int width, int height, int32_t *counts);
void or_bin_emit(int n, const float *splats, int width, int height, const int64_t *offsets,
                 uint64_t *keys, int32_t *ids);

/* Order pairs by (key, id) and cut the tile ranges. */
void or_sort_pairs(int64_t npairs, const uint64_t *keys, const int32_t *ids,
                   uint64_t *sorted_keys, int32_t *sorted_ids);
void or_tile_ranges(int64_t npairs, const uint64_t *sorted_keys, int ntiles, int32_t *ranges);

/* Forward blend, mirror mode (Eq. 2-3 of [LOAD-IMB]). last[p] = number of list
   entries consumed by the pixel (stop index + 1, or the full tile length).
   tile_mask (nullable) restricts the work to tiles with a nonzero byte; other
   pixels are left untouched. stats (nullable) += {hits, evaluations}.
   pixel_hits (nullable) <- the number of splats each pixel blended.
   pair_quarters (nullable, one byte per list position, zeroed by the caller)
   |= bit q for every 8x8 quarter q of the position's tile (q = 0 upper left,
   1 upper right, 2 lower left, 3 lower right) in which at least one pixel
   blended that splat ([3DGS-CUDA] Step 4: the forward pass records which
   splats contributed to which part of the tile). */
void or_render_fwd(const float *splats, const int32_t *sorted_ids, const int32_t *ranges,
                   int width, int height, const uint8_t *tile_mask, const float *bg, float *rgb,
                   float *T_final, int32_t *last, uint8_t *knife, int64_t *stats,
                   int32_t *pixel_hits, uint8_t *pair_quarters);

/* Untiled brute force: every pixel walks every visible splat in (depth, id) order.
   pixel_hits (nullable) <- the number of splats each pixel blended. */
void or_render_fwd_untiled(int n, const float *splats, int width, int height,
                           float *rgb, float *T_final, int32_t *pixel_hits);

/* Forward values in fp64 with frozen decisions: hits from the fp32 records
   splats_dec, stop from last; values from splats_val (fp64 records). */
void or_render_fwd_values(const float *splats_dec, const double *splats_val,
                          const int32_t *sorted_ids, const int32_t *ranges, int width, int height,
                          const int32_t *last, const double *bg, double *rgb, double *T_final);

/* Analytic backward, truth mode: grads[n][9] (overwritten) of
   L = sum_p g_p . C_p + dL_dT_p T_final,p with C_p including T_final,p bg
   (bg, dL_dT: NULL for none). */
void or_render_bwd(const float *splats, const int32_t *sorted_ids, const int32_t *ranges,
                   int width, int height, const int32_t *last, const float *dL_drgb,
                   const float *bg, const float *dL_dT, int n, double *grads);

/* Per-frame chunking policy (Eq. 6 of [LOAD-IMB]). counts_desc: tile counts in
   descending order. Writes h (tiles to chunk) and k (chunks per tile; 1 when off);
   only candidates with h k <= max_items are considered. */
void or_chunk_policy(int ntiles, const int32_t *counts_desc, double workers, double lambda_,
                     double beta, double eps, int max_items, int32_t *h_out, int32_t *k_out);

/* OpenMP threads used by the parallel loops (for reporting). */
int or_num_threads(void);
/* Sets the OpenMP thread count of later parallel loops (n >= 1). */
void or_set_num_threads(int n);

#endif
