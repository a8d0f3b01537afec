/* gs.h - C ABI of the MI355X (gfx950) tile-based differentiable Gaussian-splatting
 * rasterizer.
 *
 * The method (sources by page title):
 *   "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on GPUs"
 *      section 2.1 Eq. 1 (projection), Eq. 2-3 (alpha and front-to-back
 *      blending with the 1e-4 transmittance stop), section 4 (persistent
 *      longest-first tile scheduling, depth-wise chunking with saturation
 *      signalling, Eq. 4-5 composition, Eq. 6 per-frame chunking policy).
 *   "What the 3DGS Literature Left on the Table" Step 1 (a)-(e): the 9
 *      screen-space gradients, exact opacity-aware conic-tile binning, the
 *      (tile, depth) key sort, 16x16 tiles, the scalar backward accumulator.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers owned by the caller unless marked (host).
 *     The library allocates nothing. Its global mutable state is the optional
 *     measurement timer (gs_timing_start / gs_timing_read), the probe limit of
 *     the bounded device-side waits (gs_set_wait_limit, for tests of the
 *     give-up path) and the static device array of gs_sort_keys_noalloc; apart
 *     from these, calls on different streams with their own buffers are
 *     independent.
 *   - `stream` is a hipStream_t (NULL = the default stream). Each call only
 *     enqueues kernels on it and returns; it never synchronises.
 *   - Synchronous errors (argument validation, HIP launch errors) return a
 *     negative gs_status; after an error nothing more is enqueued by that call,
 *     and outputs are undefined only if a launch error occurred mid-call.
 *   - Asynchronous errors go to the frame's device status word (int32, device
 *     memory, one per frame): gs_bin_tiles starts it at GS_OK (or
 *     GS_ERR_CAPACITY); gs_sort_keys, gs_render_fwd and gs_render_bwd take the
 *     same word, do nothing when it is not GS_OK on entry, and store the first
 *     error they find (a later error never overwrites an earlier one). The
 *     caller reads it once, after the frame; a frame whose word is not GS_OK
 *     has undefined rgb, T_final, last and ranges, and zero gradients.
 *   - All floating-point arithmetic is fp32. Keys, ids, counts and ranges are
 *     integers. Splat counts n and pair capacities must be below 2^30
 *     (GS_ERR_UNSUPPORTED).
 *
 * Data layouts
 *   splat record (GS_SPLAT_FLOATS = 12 floats, 48 B, 16-B aligned):
 *       mx, my, a, b, c, o, r, g, b, tau, depth, view
 *     (mx, my) centre in pixels; (a, b, c) the conic Sigma'^-1 = [[a,b],[b,c]];
 *     o opacity; (r, g, b) colour; tau = 2 ln(255 o), the alpha >= 1/255
 *     cutoff as a bound on q; depth = camera-space z; view: the record's view
 *     in a batch of views, as int bits (0, i.e. 0.0f, outside batches; a record
 *     whose view is not in the batch emits no pairs). Culled: tau = -1, the
 *     others 0 but view.
 *   pixel (px, py) is sampled at (px + 0.5, py + 0.5);
 *     q = a dx^2 + 2 b dx dy + c dy^2, evaluated in the canonical fp32 form
 *     fma(c*dy, dy, fma((2b)*dx, dy, (a*dx)*dx)); a pixel is hit iff q <= tau.
 *   tiles are 16x16 pixels; tiles_x = ceil(W/16), tiles_y = ceil(H/16),
 *     tile id = ty * tiles_x + tx.
 *   images are planar: rgb / dL_drgb [3][H][W]; T_final, last [H][W].
 *   gradient record (GS_GRAD_FLOATS = 9): d/d (mx, my, a, b, c, o, r, g, b).
 */
#ifndef GS_H
#define GS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GS_OK = 0,
  GS_ERR_INVALID_ARGUMENT = -1, /* bad size, NULL pointer, degree outside 0..3 */
  GS_ERR_CAPACITY = -2,         /* pair buffer too small (reported on the device) */
  GS_ERR_WORKSPACE = -3,        /* workspace or fwd_state smaller than required */
  GS_ERR_HIP = -4,              /* a HIP runtime call or kernel launch failed */
  GS_ERR_UNSUPPORTED = -5,      /* image too large (> 65535 tiles), n or capacity >= 2^30 */
  GS_ERR_TIMEOUT = -6           /* a bounded device-side wait gave up (reported on the
                                   device; never expected): the frame's results are invalid */
} gs_status;

#define GS_TILE 16
#define GS_SPLAT_FLOATS 12
#define GS_GRAD_FLOATS 9
#define GS_MAX_VIEWS 16 /* views in one batch (the *_views calls) */

/* Pinhole camera, passed by HOST pointer. world_to_cam is row-major [R | t]
 * (camera: +x right, +y down, +z forward). Gaussians with t_z <= znear are
 * culled. lowpass (px^2) is added to both diagonal entries of Sigma'. */
typedef struct {
  int32_t width, height;
  float fx, fy, cx, cy;
  float world_to_cam[12];
  float znear;
  float lowpass;
} gs_camera;

/* Tile scheduling knobs, passed by HOST pointer (NULL = defaults:
 * chunk_mode 1, lambda 131072, beta 0.25, eps 0.10). The page prints neither
 * lambda (fixed cost of one chunk, in pair units) nor beta; these values come
 * from timing forced (h, k) plans on MI355X: with them the policy leaves
 * scenes whose tiles saturate early unchunked and splits the outliers of
 * scenes with long unsaturated lists.
 *   chunk_mode 0: no depth chunking (persistent longest-first queue only)
 *              1: automatic (Eq. 6 policy, evaluated on the device per frame)
 *              2: force chunking of the force_h heaviest tiles into force_k chunks
 *                 (force_h <= 0 means every tile), force_k in {2,4,8,16}. */
typedef struct {
  int32_t chunk_mode;
  int32_t force_k;
  int32_t force_h;
  float lambda_;
  float beta;
  float eps;
  /* 1: the caller built this frame's plan ahead with gs_plan_tiles (same
   * knobs) on a stream this call's stream waits for; gs_render_fwd then checks
   * it inside its own launch instead of launching the hand-over first, and a
   * frame without a matching plan fails with GS_ERR_WORKSPACE. 0: gs_render_fwd
   * takes a plan built ahead if one waits, else builds it. gs_plan_tiles
   * ignores this field. */
  int32_t planned;
} gs_sched;

/* Human-readable name of a status (host). */
const char *gs_strerror(int32_t status);

/* Bytes of scratch the calls below need for n Gaussians, a W x H image and a
 * pair buffer of pair_capacity entries (host). One workspace may serve all
 * calls of a frame on one stream; it must not be shared by concurrent calls. */
size_t gs_workspace_size(int32_t n, int32_t width, int32_t height, int64_t pair_capacity);

/* Bytes of the opaque per-frame state that gs_render_fwd writes and
 * gs_render_bwd reads: the schedule (LPT order, chunk plan, work queues), the
 * per-sub-tile walk bounds, the chunk partials, and the contributor record
 * (Step 4 of the literature page: which list entries blended into which 8x8
 * quarter of their tile, one bit per entry and quarter), which needs room for
 * pair_capacity entries. 0 on invalid arguments. */
size_t gs_fwd_state_size(int32_t width, int32_t height, int64_t pair_capacity);

/* Projection (Eq. 1 of the load-imbalance page) and SH colour.
 *   means [n][3], log_scales [n][3], quats [n][4] (w,x,y,z; need not be unit),
 *   opacities [n] (activated, in (0,1)), sh [n][(deg+1)^2][3] (sh_degree 0..3)
 *   -> splats [n][12] (record above; every row written).
 * Colour = sum_k Y_k(d) sh[k] with d the unit direction from the camera centre
 * to the mean and Y_k the real orthonormal SH basis (no offset, no clamp). */
int32_t gs_project(int32_t n, const float *means, const float *log_scales, const float *quats,
                   const float *opacities, const float *sh, int32_t sh_degree,
                   const gs_camera *cam, float *splats, void *stream);

/* Backward of gs_project: the 9 screen-space gradients of each record chained
 * to the Gaussian's parameters (Eq. 1 of the load-imbalance page differentiated
 * through Lambda = Sigma'^-1, the Jacobian J(t), the view transform and
 * Sigma = Rq diag(exp(2 s)) Rq^T; Step 3 of the literature page for the colour:
 * dL/ds_k = Y_k(d) dL/dc, plus the view direction's share of dL/dmean).
 *   means, log_scales, quats, opacities, sh, sh_degree, cam: as for gs_project
 *   dL_dsplat [n][9] <- read: dL/d(mx, my, a, b, c, o, r, g, b) (gs_render_bwd's
 *     output); tau and depth pass no gradient (a threshold and a sort key)
 *   dL_dmeans [n][3], dL_dlog_scales [n][3], dL_dquats [n][4] (with respect to
 *     the quaternion as given, not normalised), dL_dopacities [n],
 *     dL_dsh [n][(deg+1)^2][3] <- fully overwritten; rows of Gaussians that
 *     gs_project culls are 0.
 * quats and dL_dquats 16-byte aligned; sh and dL_dsh 16-byte aligned for SH
 * degrees 1 and 3 (rows of 12 and 48 floats, read and written as vectors),
 * 4-byte aligned otherwise. */
int32_t gs_project_bwd(int32_t n, const float *means, const float *log_scales, const float *quats,
                       const float *opacities, const float *sh, int32_t sh_degree,
                       const gs_camera *cam, const float *dL_dsplat, float *dL_dmeans,
                       float *dL_dlog_scales, float *dL_dquats, float *dL_dopacities,
                       float *dL_dsh, void *stream);

/* gs_project and gs_project_bwd with the SH coefficients stored as bfloat16
 * (Step 3 and Step 6 of the literature page keep the SH parameters in bf16 to
 * halve their bytes): sh [n][(deg+1)^2][3] holds the upper 16 bits of each
 * fp32 value (bf16 bit patterns). Each value is widened exactly to fp32 in
 * registers and all arithmetic is fp32, so the results equal those of
 * gs_project / gs_project_bwd called with the widened coefficients, bit for
 * bit. dL_dsh stays fp32 (same layout and alignment as for gs_project_bwd).
 * sh 16-byte aligned for SH degree 3 (rows of 48 values, read as 16-byte
 * vectors), 8-byte aligned for degree 1 (rows of 12), 2-byte aligned for
 * degrees 0 and 2. Other arguments, outputs and errors as for the fp32 calls. */
int32_t gs_project_bf16sh(int32_t n, const float *means, const float *log_scales,
                          const float *quats, const float *opacities, const uint16_t *sh,
                          int32_t sh_degree, const gs_camera *cam, float *splats, void *stream);
int32_t gs_project_bwd_bf16sh(int32_t n, const float *means, const float *log_scales,
                              const float *quats, const float *opacities, const uint16_t *sh,
                              int32_t sh_degree, const gs_camera *cam, const float *dL_dsplat,
                              float *dL_dmeans, float *dL_dlog_scales, float *dL_dquats,
                              float *dL_dopacities, float *dL_dsh, void *stream);

/* Exact opacity-aware conic-tile binning (Step 1 (b) of the literature page).
 * A tile is emitted for splat i when the ellipse q <= tau (1 + 2^-10) meets the
 * tile's pixel-sample hull widened by 2^-8 px; spans are solved per tile row
 * in closed form with the canonical fp32 operation sequence (bit-exact).
 *   offsets [n+1] <- exclusive prefix sum of per-splat pair counts;
 *                    offsets[n] = I, the number of pairs (always written).
 *   tile_counts [T] or NULL <- the number of pairs of every tile (T = tiles_x
 *     x tiles_y, row-major), for gs_plan_tiles; gs_sort_keys does not read it
 *     (it recomputes the counts from its own record in the workspace).
 *   keys, ids [pair_capacity] or both NULL <- (tile << 32) | float_bits(depth)
 *     and the splat id of every pair, in splat-id order, tiles of one splat
 *     ascending. The frame does not need them (gs_sort_keys emits the pairs
 *     again, directly in depth order); they expose the emission for checking.
 *   device_status [1] <- GS_OK, or GS_ERR_CAPACITY when I > pair_capacity; in
 *     that case nothing is emitted and the later calls of the frame do nothing.
 *     The caller reads it after the frame, grows its pair buffers to at least
 *     offsets[n] and runs the frame again.
 *   workspace <- also receives, from the same pass over the splat records, what
 *     gs_sort_keys needs: each splat's depth key, the depth-digit and per-tile
 *     pair histograms, and cleared radix look-back words. Pass the same
 *     workspace, untouched, to the gs_sort_keys call of the same frame. */
int32_t gs_bin_tiles(int32_t n, const float *splats, const gs_camera *cam, int64_t pair_capacity,
                     int32_t *offsets, int32_t *tile_counts, uint64_t *keys, int32_t *ids,
                     int32_t *device_status, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Order the pairs by (tile, depth, splat id) and cut the per-tile ranges
 * (Step 1 (d), Figure 5 of the literature page): stable radix sort of the
 * visible splats (those with offsets[i+1] > offsets[i]) by fp32 depth bits,
 * emission of their tile keys in that order (the same canonical spans as
 * gs_bin_tiles), then a stable radix sort by tile id.
 * Reads the state gs_bin_tiles of the same frame left in `workspace` (so it
 * takes no key, id or per-tile count arrays: the pairs are emitted again, in
 * depth order, inside the first tile pass, and the per-tile counts come from
 * the binning pass's row histogram; a tile's count is
 * tile_ranges[t][1] - tile_ranges[t][0]). Call it once after every
 * gs_bin_tiles, with the same workspace, n, splats, offsets, camera and
 * pair_capacity: the binning pass tags the workspace with n, the capacity and
 * the tile grid, and this call uses the tag up; a workspace without a
 * matching tag sets device_status to GS_ERR_WORKSPACE and sorts nothing.
 *   sorted_ids [pair_capacity] <- splat ids in that order
 *   sorted_keys [pair_capacity] or NULL <- (tile << 32) | float_bits(depth)
 *   tile_ranges [T][2] <- [start, end) of every tile (empty tiles: start = end
 *     = number of pairs of lower tiles; all zero when the frame failed)
 *   device_status [1]: the frame's status word (conventions above); a radix
 *     pass whose bounded look-back wait gives up stores GS_ERR_TIMEOUT. */
int32_t gs_sort_keys(int32_t n, const float *splats, const int32_t *offsets, int64_t pair_capacity,
                     const gs_camera *cam, uint64_t *sorted_keys, int32_t *sorted_ids,
                     int32_t *tile_ranges, int32_t *device_status, void *workspace,
                     size_t workspace_bytes, void *stream);

/* gs_sort_keys that also builds the frame's tile schedule (as gs_plan_tiles
 * would, from the per-tile counts the sort itself holds) into fwd_state: a
 * frame of 257 to 8192 tiles builds it in one more workgroup of its last tile
 * pass, beside that pass's partitions, any other after the sort in a launch of
 * its own. The plan waits for a gs_render_fwd with sched->planned = 1 on the
 * same stream, which needs no event between the streams and no hand-over
 * launch.
 *   sched (NULL = defaults; `planned` ignored), fwd_state, fwd_state_bytes: as
 *   for gs_plan_tiles; everything else as for gs_sort_keys. */
int32_t gs_sort_keys_plan(int32_t n, const float *splats, const int32_t *offsets,
                          int64_t pair_capacity, const gs_camera *cam, uint64_t *sorted_keys,
                          int32_t *sorted_ids, int32_t *tile_ranges, const gs_sched *sched,
                          void *fwd_state, size_t fwd_state_bytes, int32_t *device_status,
                          void *workspace, size_t workspace_bytes, void *stream);

/* The frame's tile schedule, built ahead of gs_render_fwd from the per-tile
 * counts of gs_bin_tiles (section 4 of the load-imbalance page: the
 * longest-first order of the tiles by pair count, the Eq. 6 chunking policy and
 * the work queues). Only the counts feed the schedule, so it can be built
 * while gs_sort_keys runs, on a second stream that waits for gs_bin_tiles;
 * the stream of gs_render_fwd then waits for this call. gs_render_fwd finds
 * the plan in fwd_state and uses it in place of building its own (it checks
 * the tile grid and that the pair total matches its tile_ranges; a mismatch
 * sets device_status to GS_ERR_WORKSPACE). Without this call gs_render_fwd
 * builds the same plan itself.
 *   tile_counts [T]: as written by gs_bin_tiles for this frame.
 *   sched: as for gs_render_fwd (NULL = defaults); pass the same to both.
 *   fwd_state <- the plan; the state must not be in use by a gs_render_bwd of
 *     an earlier frame while this runs (order the streams accordingly).
 *   device_status [1]: read when the call starts (a frame that already failed
 *     gets no plan, and gs_render_fwd then plans and skips it itself);
 *     GS_ERR_WORKSPACE when the pairs exceed the state's capacity. */
int32_t gs_plan_tiles(const int32_t *tile_counts, const gs_camera *cam, const gs_sched *sched,
                      void *fwd_state, size_t fwd_state_bytes, int32_t *device_status,
                      void *stream);

/* Forward blend (Eq. 2-3): per pixel, front to back over its tile's list;
 * alpha = min(0.99, o exp(-q/2)) on hits (q <= tau); C += alpha T c;
 * T *= (1 - alpha); the pixel stops after the splat that takes T below 1e-4.
 * Tiles are served by a persistent longest-first queue; heavy tiles may be
 * split into depth chunks (Eq. 4-5) with saturation signalling, exactly:
 * results do not depend on the schedule beyond fp32 rounding. The schedule is
 * the one gs_plan_tiles built ahead for this frame, if it did, else the call
 * builds it first.
 *   rgb [3][H][W], T_final [H][W] <- colour and final transmittance
 *   last [H][W] <- list entries the pixel consumed (stop index + 1, or the
 *                  tile's full length when it never stopped)
 *   fwd_state <- opaque, gs_fwd_state_size(W, H, capacity) bytes (256-byte
 *     aligned), consumed by gs_render_bwd; a frame with more pairs than the
 *     capacity it was sized for sets device_status to GS_ERR_WORKSPACE
 *   stats [4] or NULL <- += {hits: (pixel, splat) pairs blended; lane evaluations:
 *                          64 x (8x8 sub-tile, splat) pairs tested; sub-tile hits:
 *                          (8x8 sub-tile, splat) pairs with at least one hit;
 *                          chunked tiles h}
 *   pixel_hits [H][W] or NULL <- += the number of splats each pixel blended
 *     (for checking; with stats or pixel_hits the forward runs a counting
 *     instantiation of its kernel, which gives the same images bit for bit)
 *   device_status [1]: the frame's status word (conventions above); a chunk
 *     whose bounded wait for the chunks in front of it gives up stores
 *     GS_ERR_TIMEOUT. Ids in sorted_ids outside [0, n) are skipped. */
int32_t gs_render_fwd(int32_t n, const float *splats, const int32_t *sorted_ids,
                      const int32_t *tile_ranges, const gs_camera *cam, const gs_sched *sched,
                      float *rgb, float *T_final, int32_t *last, void *fwd_state,
                      size_t fwd_state_bytes, int64_t *stats, int32_t *pixel_hits,
                      int32_t *device_status, void *stream);

/* Backward of the forward blend with respect to the 9 screen-space splat
 * parameters (Step 1 (a), (e) of the literature page), given dL/dC per pixel.
 * Each pixel walks the list entries the forward pass recorded as contributors
 * of its quarter (Step 4) back from `last`, recovers T by division by
 * (1 - alpha), keeps the scalar accumulator accum = c_behind . dL/dC, and
 * forms dL/dalpha = T (c . dL/dC - accum). Per-wave sums go to the output
 * with float atomics, so low-order bits depend on the atomic order.
 *   fwd_state: the state gs_render_fwd left for this frame (same size). The
 *     backward keeps its own work queue in it, so it is not const: a frame's
 *     state is the forward-to-backward record of that frame, and the backward
 *     may run again on it.
 *   dL_dsplat [n][9] <- fully overwritten (rows of culled splats are 0; all
 *     rows 0 when device_status is not GS_OK on entry).
 *   device_status [1]: the frame's status word (conventions above). */
int32_t gs_render_bwd(int32_t n, const float *splats, const int32_t *sorted_ids,
                      const int32_t *tile_ranges, const gs_camera *cam, const float *T_final,
                      const int32_t *last, void *fwd_state, size_t fwd_state_bytes,
                      const float *dL_drgb, float *dL_dsplat, int32_t *device_status,
                      void *stream);

/* gs_render_fwd and gs_render_bwd with a background colour and a gradient of
 * the final transmittance (not on the pages, which blend onto black; the usual
 * completion of Eq. 3): the light that passes every blended splat shows the
 * background, C = sum_i c_i alpha_i T_i + T_final bg. In the backward both
 * terms sit behind the last blended splat, so each pixel's accumulator starts
 * at bg . dL/dC + dL/dT_final instead of 0 (and a chunk's at the later chunks'
 * colour plus T_final (bg . dL/dC + dL/dT_final), over its own T_end).
 *   background: host pointer to 3 floats (read during the call; finite), or
 *     NULL for black. The two calls of a frame take the same colour.
 *   dL_dT [H][W] or NULL: dL/dT_final per pixel (device, 4-byte aligned).
 * With NULL for both the results are those of gs_render_fwd / gs_render_bwd,
 * bit for bit. Other arguments, outputs and errors as for those calls. */
int32_t gs_render_fwd_bg(int32_t n, const float *splats, const int32_t *sorted_ids,
                         const int32_t *tile_ranges, const gs_camera *cam,
                         const gs_sched *sched, float *rgb, float *T_final, int32_t *last,
                         void *fwd_state, size_t fwd_state_bytes, int64_t *stats,
                         int32_t *pixel_hits, int32_t *device_status, const float *background,
                         void *stream);
int32_t gs_render_bwd_bg(int32_t n, const float *splats, const int32_t *sorted_ids,
                         const int32_t *tile_ranges, const gs_camera *cam, const float *T_final,
                         const int32_t *last, void *fwd_state, size_t fwd_state_bytes,
                         const float *dL_drgb, float *dL_dsplat, int32_t *device_status,
                         const float *background, const float *dL_dT, void *stream);

/* gs_render_fwd_bg that also sets zero_out[0 .. zero_count) to zero: each of
 * the frame's workers clears its own slice once no tile is left for it, so the
 * clearing fills the idle end of the persistent launch instead of a launch of
 * its own before the backward. Meant for the gradient array that a
 * gs_render_bwd_accumulate of the same frame then adds into (together the
 * results of gs_render_bwd_bg, up to the order of the float additions).
 *   zero_out: device, 16-byte aligned, zero_count floats (0 and NULL: none);
 *     cleared whatever the frame's device_status (a failed frame clears only).
 * Other arguments, outputs and errors as for gs_render_fwd_bg. */
int32_t gs_render_fwd_zero(int32_t n, const float *splats, const int32_t *sorted_ids,
                           const int32_t *tile_ranges, const gs_camera *cam,
                           const gs_sched *sched, float *rgb, float *T_final, int32_t *last,
                           void *fwd_state, size_t fwd_state_bytes, int64_t *stats,
                           int32_t *pixel_hits, int32_t *device_status, const float *background,
                           float *zero_out, int64_t zero_count, void *stream);

/* gs_render_bwd_bg (n_views 1) or gs_render_bwd_views (n_views > 1) adding
 * the gradients into dL_dsplat instead of overwriting it: the caller
 * initialises the array (zeros for one frame's gradients, or the sums of
 * earlier calls to accumulate over frames or batches). For callers that clear
 * the array elsewhere, e.g. on another stream while the frame is sorted, so
 * the call itself writes only the splats the frame touches. A frame whose
 * device_status is not GS_OK on entry adds nothing. Float atomics make the
 * low-order bits depend on the order of the additions. Other arguments,
 * outputs and errors as for gs_render_bwd_views. */
int32_t gs_render_bwd_accumulate(int32_t n, const float *splats, const int32_t *sorted_ids,
                                 const int32_t *tile_ranges, const gs_camera *cam,
                                 int32_t n_views, const float *T_final, const int32_t *last,
                                 void *fwd_state, size_t fwd_state_bytes, const float *dL_drgb,
                                 float *dL_dsplat, int32_t *device_status,
                                 const float *background, const float *dL_dT, void *stream);

/* Batches of views: n_views cameras of one size (1 <= n_views <= GS_MAX_VIEWS)
 * rendered as one image, so that binning, sorting and each of the two
 * persistent raster kernels run once for the whole batch (one schedule, one
 * longest-first queue over every view's tiles). Not on the pages; each view's
 * results are those of the single-view calls on that view.
 *   Layout: view v's splat records are rows [v n, (v + 1) n) of splats (n
 *   Gaussians per view; the record's pad word holds v as int bits; the bin,
 *   sort and render calls take the record count n_views n as their n); its tiles
 *   are tile rows [v ty, (v + 1) ty) of the batch (ty = ceil(height / 16)),
 *   so tile ids run over tiles_x x (n_views ty) tiles; its pixels are rows
 *   [v height, (v + 1) height) of rgb [3][n_views height][width], T_final and
 *   last [n_views height][width], and of dL_drgb and dL_dT.
 *   cam (bin, sort, plan, render): any camera of the batch (only its size is
 *   used).
 *   Sizes: gs_workspace_size_views and gs_fwd_state_size_views (0 on invalid
 *   arguments or more than 65535 tiles in the batch).
 *   gs_project_views: splats [n_views n][12] <- gs_project with cams[v] for
 *     rows of view v. cams[n_views], all of one width and height.
 *   gs_project_bwd_views: dL_dsplat [n_views n][9] -> the per-Gaussian outputs
 *     of gs_project_bwd, summed over the views (fully overwritten).
 *   Everything else as for the single-view calls (the render calls take the
 *   background and dL/dT_final arguments of gs_render_fwd_bg/gs_render_bwd_bg). */
size_t gs_workspace_size_views(int32_t n, int32_t width, int32_t height, int32_t n_views,
                               int64_t pair_capacity);
size_t gs_fwd_state_size_views(int32_t width, int32_t height, int32_t n_views,
                               int64_t pair_capacity);
int32_t gs_project_views(int32_t n, const float *means, const float *log_scales,
                         const float *quats, const float *opacities, const float *sh,
                         int32_t sh_degree, const gs_camera *cams, int32_t n_views,
                         float *splats, void *stream);
int32_t gs_project_bwd_views(int32_t n, const float *means, const float *log_scales,
                             const float *quats, const float *opacities, const float *sh,
                             int32_t sh_degree, const gs_camera *cams, int32_t n_views,
                             const float *dL_dsplat, float *dL_dmeans, float *dL_dlog_scales,
                             float *dL_dquats, float *dL_dopacities, float *dL_dsh,
                             void *stream);
int32_t gs_bin_tiles_views(int32_t n, const float *splats, const gs_camera *cam, int32_t n_views,
                           int64_t pair_capacity, int32_t *offsets, int32_t *tile_counts,
                           uint64_t *keys, int32_t *ids, int32_t *device_status, void *workspace,
                           size_t workspace_bytes, void *stream);
int32_t gs_sort_keys_views(int32_t n, const float *splats, const int32_t *offsets,
                           int64_t pair_capacity, const gs_camera *cam, int32_t n_views,
                           uint64_t *sorted_keys, int32_t *sorted_ids, int32_t *tile_ranges,
                           int32_t *device_status, void *workspace, size_t workspace_bytes,
                           void *stream);
int32_t gs_plan_tiles_views(const int32_t *tile_counts, const gs_camera *cam, int32_t n_views,
                            const gs_sched *sched, void *fwd_state, size_t fwd_state_bytes,
                            int32_t *device_status, void *stream);
int32_t gs_render_fwd_views(int32_t n, const float *splats, const int32_t *sorted_ids,
                            const int32_t *tile_ranges, const gs_camera *cam, int32_t n_views,
                            const gs_sched *sched, float *rgb, float *T_final, int32_t *last,
                            void *fwd_state, size_t fwd_state_bytes, int64_t *stats,
                            int32_t *pixel_hits, int32_t *device_status,
                            const float *background, void *stream);
int32_t gs_render_bwd_views(int32_t n, const float *splats, const int32_t *sorted_ids,
                            const int32_t *tile_ranges, const gs_camera *cam, int32_t n_views,
                            const float *T_final, const int32_t *last, void *fwd_state,
                            size_t fwd_state_bytes, const float *dL_drgb, float *dL_dsplat,
                            int32_t *device_status, const float *background,
                            const float *dL_dT, void *stream);

/* Allocation-free sort, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): gs_bin_tiles (without the id-order keys and ids) followed by
 * gs_sort_keys, with both calls' workspace taken from the library's own static
 * device array of GS_NOALLOC_SCRATCH_BYTES per GPU instead of a caller's
 * buffer. The array belongs to the library, lives on every GPU the library
 * runs on until the process ends, and is shared by every call on that GPU: it
 * keeps the last call's contents, so calls that overlap on one GPU (on two
 * streams, or from two threads) race and must not be issued. The first call on
 * a device looks up that device's array address (hipGetSymbolAddress) with the
 * device current; no call allocates.
 *   Arguments and outputs: as for gs_bin_tiles and gs_sort_keys (offsets,
 *   device_status, sorted_keys or NULL, sorted_ids, tile_ranges).
 *   Limit: a frame whose workspace (gs_workspace_size(n, W, H, pair_capacity))
 *   exceeds GS_NOALLOC_SCRATCH_BYTES returns GS_ERR_WORKSPACE before any HIP
 *   call (about 1M Gaussians with a capacity of 2M pairs fit). */
#define GS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int32_t gs_sort_keys_noalloc(int32_t n, const float *splats, const gs_camera *cam,
                             int64_t pair_capacity, int32_t *offsets, uint64_t *sorted_keys,
                             int32_t *sorted_ids, int32_t *tile_ranges, int32_t *device_status,
                             void *stream);

/* Kernel timing, for measurement only (no paper passage: it lets a benchmark
 * divide algorithmic bytes by the raster kernel's own duration rather than by
 * the whole call's, which also zeroes the gradients and orders the backward's
 * items). Not thread-safe; one device per process while it is on.
 * gs_timing_start: the next up to 512 calls each of gs_render_fwd and
 *   gs_render_bwd record a pair of HIP events on their stream, just before and
 *   after their raster kernel (k_render_fwd / k_render_bwd). The events are
 *   created on the first call (current device) and kept until the process ends.
 *   Returns GS_OK or GS_ERR_HIP.
 * gs_timing_read(which, ms, cap): ends the recording, waits for the recorded
 *   launches of kernel `which` (0 forward, 1 backward) and writes up to cap of
 *   their durations in ms, in launch order, to the HOST array ms. Returns the
 *   number written, or GS_ERR_INVALID_ARGUMENT / GS_ERR_HIP. */
int32_t gs_timing_start(void);
int32_t gs_timing_read(int32_t which, float *ms, int32_t cap);

/* The bounded device-side waits (the sort's look-back over earlier partitions,
 * a chunk's wait for the chunks in front of it) give up after a number of
 * probes and store GS_ERR_TIMEOUT in the frame's status word; the frame's later
 * kernels then do nothing. For tests of that path (a caller that wants every
 * wait to give up at its first unsuccessful probe sets 0):
 *   probes >= 0: the limit for the calls enqueued from now on;
 *   probes < 0: each wait's own default (1 << 22 probes in the sort, 1 << 20 in
 *               the forward, seconds at the longest back-off).
 * Returns the previous setting (-1 for the defaults). Host-side state shared by
 * every device and thread of the process. */
int32_t gs_set_wait_limit(int32_t probes);

#ifdef __cplusplus
}
#endif
#endif /* GS_H */
