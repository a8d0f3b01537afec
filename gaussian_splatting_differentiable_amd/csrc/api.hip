// C-ABI entry points: argument validation, camera preparation, workspace and
// forward-state layout, and the kernel launches of each stage. The functions
// are declared (with their contracts) in include/gs.h.
#include <atomic>
#include <math.h>
#include <string.h>

#include <mutex>

#include "render_common.h"

hipError_t gs_launch_project(int n, const float *means, const float *log_scales, const float *quats,
                             const float *opac, const void *sh, bool sh_bf16, int degree,
                             const CamK &cam, float *splats, hipStream_t st);
hipError_t gs_launch_project_bwd(int n, const float *means, const float *log_scales,
                                 const float *quats, const float *opac, const void *sh,
                                 bool sh_bf16, int degree, const CamK &cam, const float *dsplat,
                                 float *gmeans, float *gls, float *gquats, float *gopac,
                                 float *gsh, bool accumulate, hipStream_t st);
hipError_t gs_launch_bin(int n, const float *splats, const CamK &cam, int64_t capacity,
                         int32_t *offsets, int32_t *tile_counts, uint64_t *keys, int32_t *ids,
                         int32_t *status, void *ws, hipStream_t st);
size_t gs_sort_ws_bytes(int n, int64_t cap, int tiles_x, int tiles_y);
hipError_t gs_launch_sort(int n, const float *splats, const int32_t *offsets, int64_t cap,
                          const CamK &cam, uint64_t *sorted_keys, int32_t *sorted_ids,
                          int32_t *ranges, int32_t *status, void *ws, const SortPlan *plan,
                          hipStream_t st);
hipError_t gs_launch_render_fwd(int n, const float *splats, const int32_t *sorted_ids,
                                const int32_t *ranges, const CamK &cam, const gs_sched &sched,
                                float *rgb, float *T, int32_t *last, void *fwd_state,
                                int64_t cap_pairs, int64_t *stats, int32_t *pixel_hits,
                                int32_t *status, int workers_waves, float *clear,
                                int64_t nclear, hipEvent_t ev0, hipEvent_t ev1, hipStream_t st);
hipError_t gs_launch_schedule(const int32_t *ranges, const int32_t *counts, const CamK &cam,
                              int chunk_mode, int force_k, int force_h, double lambda_,
                              double beta, double eps, int nblocks, void *fwd_state,
                              int64_t *stats, int32_t *status, int64_t cap_pairs,
                              hipStream_t st);
hipError_t gs_launch_render_bwd(int n, const float *splats, const int32_t *sorted_ids,
                                const int32_t *ranges, const CamK &cam, const float *T,
                                const int32_t *last, void *fwd_state, const float *dL,
                                const float *dT, float *grads, bool accumulate, int32_t *status,
                                int workers_waves, hipEvent_t ev0, hipEvent_t ev1, hipStream_t st);

// The probe limit of the device-side bounded waits (below 0: each wait's own
// default). Only tests of the give-up path change it.
static std::atomic<int32_t> g_wait_limit{-1};

int32_t gs_wait_limit(int32_t fallback) {
  const int32_t v = g_wait_limit.load(std::memory_order_relaxed);
  return v < 0 ? fallback : v;
}

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool finite_pos(float v) { return isfinite(v) && v > 0.0f; }

// Fills the kernel-side camera; false on invalid values.
bool prep_camera(const gs_camera *c, CamK *k) {
  if (!c || c->width <= 0 || c->height <= 0) return false;
  if (!finite_pos(c->fx) || !finite_pos(c->fy) || !isfinite(c->cx) || !isfinite(c->cy)) return false;
  if (!isfinite(c->znear) || !isfinite(c->lowpass) || c->lowpass < 0.0f) return false;
  for (int i = 0; i < 12; i++)
    if (!isfinite(c->world_to_cam[i])) return false;
  k->width = c->width;
  k->height = c->height;
  k->tiles_x = (c->width + 15) / 16;
  k->tiles_y = (c->height + 15) / 16;
  k->fx = c->fx; k->fy = c->fy; k->cx = c->cx; k->cy = c->cy;
  const float *M = c->world_to_cam;
  for (int r = 0; r < 3; r++) {
    for (int j = 0; j < 3; j++) k->R[3 * r + j] = M[4 * r + j];
    k->t[r] = M[4 * r + 3];
  }
  for (int j = 0; j < 3; j++)
    k->centre[j] = -(k->R[j] * k->t[0] + k->R[3 + j] * k->t[1] + k->R[6 + j] * k->t[2]);
  k->znear = c->znear;
  k->lowpass = c->lowpass;
  k->bg[0] = k->bg[1] = k->bg[2] = 0.0f;
  k->bg_on = 0;
  k->views = 1;
  k->vty = k->tiles_y;
  k->view = 0;
  return true;
}

// A batch of n_views views of cam's size, stacked: tile rows and output pixel
// rows of view v follow those of view v - 1.
bool prep_views(const gs_camera *c, int32_t n_views, CamK *k) {
  if (n_views < 1 || n_views > GS_MAX_VIEWS || !prep_camera(c, k)) return false;
  k->views = n_views;
  k->tiles_y = k->vty * n_views;
  return true;
}

int64_t batch_tiles(const CamK &k) { return (int64_t)k.tiles_x * k.tiles_y; }

// Background colour (host, 3 floats, or NULL for black) into the kernel camera.
bool set_background(const float *bg, CamK *k) {
  if (!bg) return true;
  for (int c = 0; c < 3; c++) {
    if (!isfinite(bg[c])) return false;
    k->bg[c] = bg[c];
    if (bg[c] != 0.0f) k->bg_on = 1;
  }
  return true;
}

// Per-launch timing of the raster kernels (measurement only): a ring of event
// pairs per kernel, filled by the render calls while timing is on.
constexpr int TIMING_SLOTS = 512;
struct Timing {
  bool on = false, made = false;
  int used[2] = {0, 0};
  hipEvent_t ev[2][TIMING_SLOTS][2] = {};
};
Timing g_timing;

// The event pair for the next launch of kernel `which` (0 forward, 1 backward),
// or nulls when timing is off or the ring is full.
void timing_slot(int which, hipEvent_t &a, hipEvent_t &b) {
  a = b = nullptr;
  if (!g_timing.on || g_timing.used[which] >= TIMING_SLOTS) return;
  const int i = g_timing.used[which]++;
  a = g_timing.ev[which][i][0];
  b = g_timing.ev[which][i][1];
}

int64_t num_tiles(int32_t w, int32_t h) { return (int64_t)((w + 15) / 16) * ((h + 15) / 16); }

// Splat counts and pair capacities from 2^30 up are refused: the radix passes'
// look-back words hold 30-bit counts.
constexpr int64_t GS_COUNT_LIMIT = (int64_t)1 << 30;

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

int32_t hip_status(hipError_t e) { return e == hipSuccess ? GS_OK : GS_ERR_HIP; }

// Persistent workers to launch on the current device, 0 on error.
int worker_waves() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  // one workgroup of 16 persistent worker waves per CU (4 per SIMD): fewer
  // co-resident waves let each item finish sooner, which shortens the tail of
  // the launch more than the latency hiding of 8 waves per SIMD gains (measured)
  return cus > 0 ? cus * 16 : 0;
}

gs_sched default_sched() {
  gs_sched s;
  s.chunk_mode = 1;
  s.force_k = 0;
  s.force_h = 0;
  s.lambda_ = 131072.0f;  // measured on MI355X (see gs_sched in gs.h)
  s.beta = 0.25f;
  s.eps = 0.10f;
  s.planned = 0;
  return s;
}

// Byte alignment the SH rows of one Gaussian are read with: fp32 rows of 12 or
// 48 floats (degrees 1, 3) as 16-byte vectors; bf16 rows of 48 values
// (degree 3) as 16-byte and of 12 (degree 1) as 8-byte vectors; else scalars.
size_t sh_align(int degree, bool bf16) {
  const int e = 3 * (degree + 1) * (degree + 1);
  if (!bf16) return e % 4 == 0 ? 16 : 4;
  return e % 8 == 0 ? 16 : e % 4 == 0 ? 8 : 2;
}

int32_t project_impl(int32_t n, const float *means, const float *log_scales, const float *quats,
                     const float *opacities, const void *sh, bool bf16, int32_t sh_degree,
                     const gs_camera *cam, float *splats, void *stream) {
  CamK k;
  if (n < 0 || sh_degree < 0 || sh_degree > 3 || !prep_camera(cam, &k)) return GS_ERR_INVALID_ARGUMENT;
  if (n == 0) return GS_OK;
  if (!means || !log_scales || !quats || !opacities || !sh || !splats) return GS_ERR_INVALID_ARGUMENT;
  if (!aligned(quats, 16) || !aligned(splats, 16) || !aligned(sh, sh_align(sh_degree, bf16)))
    return GS_ERR_INVALID_ARGUMENT;
  return hip_status(gs_launch_project(n, means, log_scales, quats, opacities, sh, bf16, sh_degree,
                                      k, splats, (hipStream_t)stream));
}

int32_t project_bwd_impl(int32_t n, const float *means, const float *log_scales,
                         const float *quats, const float *opacities, const void *sh, bool bf16,
                         int32_t sh_degree, const gs_camera *cam, const float *dL_dsplat,
                         float *dL_dmeans, float *dL_dlog_scales, float *dL_dquats,
                         float *dL_dopacities, float *dL_dsh, void *stream) {
  CamK k;
  if (n < 0 || sh_degree < 0 || sh_degree > 3 || !prep_camera(cam, &k)) return GS_ERR_INVALID_ARGUMENT;
  if (n == 0) return GS_OK;
  if (!means || !log_scales || !quats || !opacities || !sh || !dL_dsplat || !dL_dmeans ||
      !dL_dlog_scales || !dL_dquats || !dL_dopacities || !dL_dsh)
    return GS_ERR_INVALID_ARGUMENT;
  if (!aligned(quats, 16) || !aligned(dL_dquats, 16) || !aligned(sh, sh_align(sh_degree, bf16)) ||
      !aligned(dL_dsh, sh_align(sh_degree, false)))
    return GS_ERR_INVALID_ARGUMENT;
  return hip_status(gs_launch_project_bwd(n, means, log_scales, quats, opacities, sh, bf16,
                                          sh_degree, k, dL_dsplat, dL_dmeans, dL_dlog_scales,
                                          dL_dquats, dL_dopacities, dL_dsh, false,
                                          (hipStream_t)stream));
}

}  // namespace

extern "C" {

const char *gs_strerror(int32_t s) {
  switch (s) {
    case GS_OK: return "ok";
    case GS_ERR_INVALID_ARGUMENT: return "invalid argument";
    case GS_ERR_CAPACITY: return "pair buffer capacity exceeded";
    case GS_ERR_WORKSPACE: return "workspace or forward state too small";
    case GS_ERR_HIP: return "HIP runtime error";
    case GS_ERR_UNSUPPORTED: return "unsupported size";
    case GS_ERR_TIMEOUT: return "a bounded device-side wait gave up: the frame's results are invalid";
    default: return "unknown status";
  }
}

size_t gs_fwd_state_size(int32_t width, int32_t height, int64_t pair_capacity) {
  if (width <= 0 || height <= 0 || num_tiles(width, height) > GS_MAX_TILES) return 0;
  if (pair_capacity < 0 || pair_capacity >= GS_COUNT_LIMIT) return 0;
  return fwd_layout((int)num_tiles(width, height), pair_capacity).total;
}

size_t gs_workspace_size(int32_t n, int32_t width, int32_t height, int64_t pair_capacity) {
  if (n < 0 || width <= 0 || height <= 0 || pair_capacity < 0) return 0;
  return gs_sort_ws_bytes(n, pair_capacity, (width + 15) / 16, (height + 15) / 16);
}

int32_t gs_project(int32_t n, const float *means, const float *log_scales, const float *quats,
                   const float *opacities, const float *sh, int32_t sh_degree, const gs_camera *cam,
                   float *splats, void *stream) {
  return project_impl(n, means, log_scales, quats, opacities, sh, false, sh_degree, cam, splats,
                      stream);
}

int32_t gs_project_bf16sh(int32_t n, const float *means, const float *log_scales,
                          const float *quats, const float *opacities, const uint16_t *sh,
                          int32_t sh_degree, const gs_camera *cam, float *splats, void *stream) {
  return project_impl(n, means, log_scales, quats, opacities, sh, true, sh_degree, cam, splats,
                      stream);
}

int32_t gs_project_bwd(int32_t n, const float *means, const float *log_scales, const float *quats,
                       const float *opacities, const float *sh, int32_t sh_degree,
                       const gs_camera *cam, const float *dL_dsplat, float *dL_dmeans,
                       float *dL_dlog_scales, float *dL_dquats, float *dL_dopacities,
                       float *dL_dsh, void *stream) {
  return project_bwd_impl(n, means, log_scales, quats, opacities, sh, false, sh_degree, cam,
                          dL_dsplat, dL_dmeans, dL_dlog_scales, dL_dquats, dL_dopacities, dL_dsh,
                          stream);
}

int32_t gs_project_bwd_bf16sh(int32_t n, const float *means, const float *log_scales,
                              const float *quats, const float *opacities, const uint16_t *sh,
                              int32_t sh_degree, const gs_camera *cam, const float *dL_dsplat,
                              float *dL_dmeans, float *dL_dlog_scales, float *dL_dquats,
                              float *dL_dopacities, float *dL_dsh, void *stream) {
  return project_bwd_impl(n, means, log_scales, quats, opacities, sh, true, sh_degree, cam,
                          dL_dsplat, dL_dmeans, dL_dlog_scales, dL_dquats, dL_dopacities, dL_dsh,
                          stream);
}

}  // extern "C"

namespace {

int32_t bin_impl(int32_t n, const float *splats, const CamK &k, int64_t pair_capacity,
                 int32_t *offsets, int32_t *tile_counts, uint64_t *keys, int32_t *ids,
                 int32_t *device_status, void *workspace, size_t workspace_bytes, void *stream) {
  if (n < 0 || pair_capacity < 0) return GS_ERR_INVALID_ARGUMENT;
  if (batch_tiles(k) > GS_MAX_TILES || n >= GS_COUNT_LIMIT || pair_capacity >= GS_COUNT_LIMIT)
    return GS_ERR_UNSUPPORTED;
  if (!offsets || !device_status || !workspace || (n > 0 && !splats)) return GS_ERR_INVALID_ARGUMENT;
  if ((keys == nullptr) != (ids == nullptr)) return GS_ERR_INVALID_ARGUMENT;
  if ((splats && !aligned(splats, 16)) || (keys && !aligned(keys, 8)) ||
      (tile_counts && !aligned(tile_counts, 4)))
    return GS_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < gs_sort_ws_bytes(n, pair_capacity, k.tiles_x, k.tiles_y))
    return GS_ERR_WORKSPACE;
  return hip_status(gs_launch_bin(n, splats, k, pair_capacity, offsets, tile_counts, keys, ids,
                                  device_status, workspace, (hipStream_t)stream));
}

int32_t sort_impl(int32_t n, const float *splats, const int32_t *offsets, int64_t pair_capacity,
                  const CamK &k, uint64_t *sorted_keys, int32_t *sorted_ids, int32_t *tile_ranges,
                  int32_t *device_status, void *workspace, size_t workspace_bytes, void *stream,
                  const SortPlan *plan = nullptr) {
  if (n < 0 || pair_capacity < 0) return GS_ERR_INVALID_ARGUMENT;
  if (batch_tiles(k) > GS_MAX_TILES || n >= GS_COUNT_LIMIT || pair_capacity >= GS_COUNT_LIMIT)
    return GS_ERR_UNSUPPORTED;
  if (!offsets || !tile_ranges || !workspace || !device_status || (n > 0 && !splats))
    return GS_ERR_INVALID_ARGUMENT;
  if (pair_capacity > 0 && !sorted_ids) return GS_ERR_INVALID_ARGUMENT;
  if ((splats && !aligned(splats, 16)) || (sorted_keys && !aligned(sorted_keys, 8)) ||
      !aligned(tile_ranges, 8))
    return GS_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < gs_sort_ws_bytes(n, pair_capacity, k.tiles_x, k.tiles_y))
    return GS_ERR_WORKSPACE;
  return hip_status(gs_launch_sort(n, splats, offsets, pair_capacity, k, sorted_keys, sorted_ids,
                                   tile_ranges, device_status, workspace, plan,
                                   (hipStream_t)stream));
}

int32_t fwd_impl(int32_t n, const float *splats, const int32_t *sorted_ids,
                 const int32_t *tile_ranges, CamK k, const gs_sched *sched, float *rgb,
                 float *T_final, int32_t *last, void *fwd_state, size_t fwd_state_bytes,
                 int64_t *stats, int32_t *pixel_hits, int32_t *device_status,
                 const float *background, float *clear, int64_t nclear, void *stream) {
  if (n < 0 || !set_background(background, &k)) return GS_ERR_INVALID_ARGUMENT;
  if (nclear < 0 || (nclear > 0 && (!clear || !aligned(clear, 16))))
    return GS_ERR_INVALID_ARGUMENT;
  if (batch_tiles(k) > GS_MAX_TILES || n >= GS_COUNT_LIMIT) return GS_ERR_UNSUPPORTED;
  if (!tile_ranges || !rgb || !T_final || !last || !fwd_state || !device_status)
    return GS_ERR_INVALID_ARGUMENT;
  if (n > 0 && (!splats || !sorted_ids)) return GS_ERR_INVALID_ARGUMENT;
  if ((splats && !aligned(splats, 16)) || !aligned(tile_ranges, 8) ||
      (pixel_hits && !aligned(pixel_hits, 4)))
    return GS_ERR_INVALID_ARGUMENT;
  // the pairs the state's contributor bitmap can hold; the schedule reports a
  // frame with more through device_status
  const int64_t cap_pairs = fwd_state_capacity((int)batch_tiles(k), fwd_state_bytes);
  if (cap_pairs < 0) return GS_ERR_WORKSPACE;
  if (!aligned(fwd_state, 256)) return GS_ERR_INVALID_ARGUMENT;
  const gs_sched sc = sched ? *sched : default_sched();
  if (sc.chunk_mode < 0 || sc.chunk_mode > 2 || !(sc.eps >= 0.0f) || !(sc.lambda_ >= 0.0f) ||
      !(sc.beta >= 0.0f) || (sc.planned != 0 && sc.planned != 1))
    return GS_ERR_INVALID_ARGUMENT;
  const int workers = worker_waves();
  if (workers <= 0) return GS_ERR_HIP;
  hipEvent_t e0, e1;
  timing_slot(0, e0, e1);
  return hip_status(gs_launch_render_fwd(n, splats, sorted_ids, tile_ranges, k, sc, rgb, T_final,
                                         last, fwd_state, cap_pairs, stats, pixel_hits,
                                         device_status, workers, nclear > 0 ? clear : nullptr,
                                         nclear, e0, e1, (hipStream_t)stream));
}

int32_t plan_impl(const int32_t *tile_counts, const CamK &k, const gs_sched *sched,
                  void *fwd_state, size_t fwd_state_bytes, int32_t *device_status, void *stream) {
  if (batch_tiles(k) > GS_MAX_TILES) return GS_ERR_UNSUPPORTED;
  if (!tile_counts || !fwd_state || !device_status) return GS_ERR_INVALID_ARGUMENT;
  if (!aligned(tile_counts, 4) || !aligned(fwd_state, 256)) return GS_ERR_INVALID_ARGUMENT;
  const int64_t cap_pairs = fwd_state_capacity((int)batch_tiles(k), fwd_state_bytes);
  if (cap_pairs < 0) return GS_ERR_WORKSPACE;
  const gs_sched sc = sched ? *sched : default_sched();
  if (sc.chunk_mode < 0 || sc.chunk_mode > 2 || !(sc.eps >= 0.0f) || !(sc.lambda_ >= 0.0f) ||
      !(sc.beta >= 0.0f))
    return GS_ERR_INVALID_ARGUMENT;
  const int workers = worker_waves();
  if (workers <= 0) return GS_ERR_HIP;
  return hip_status(gs_launch_schedule(nullptr, tile_counts, k, sc.chunk_mode, sc.force_k,
                                       sc.force_h, sc.lambda_, sc.beta, sc.eps,
                                       workers / GS_WAVES_PER_BLOCK, fwd_state, nullptr,
                                       device_status, cap_pairs, (hipStream_t)stream));
}

int32_t bwd_impl(int32_t n, const float *splats, const int32_t *sorted_ids,
                 const int32_t *tile_ranges, CamK k, const float *T_final, const int32_t *last,
                 void *fwd_state, size_t fwd_state_bytes, const float *dL_drgb, float *dL_dsplat,
                 int32_t *device_status, const float *background, const float *dL_dT,
                 bool accumulate, void *stream) {
  if (n < 0 || !set_background(background, &k)) return GS_ERR_INVALID_ARGUMENT;
  if (dL_dT) k.bg_on = 1;
  if (batch_tiles(k) > GS_MAX_TILES || n >= GS_COUNT_LIMIT) return GS_ERR_UNSUPPORTED;
  if (!tile_ranges || !T_final || !last || !fwd_state || !dL_drgb || !device_status)
    return GS_ERR_INVALID_ARGUMENT;
  if (n > 0 && (!splats || !sorted_ids || !dL_dsplat)) return GS_ERR_INVALID_ARGUMENT;
  if ((splats && !aligned(splats, 16)) || !aligned(tile_ranges, 8) ||
      (dL_dsplat && !aligned(dL_dsplat, 16)) || (dL_dT && !aligned(dL_dT, 4)))
    return GS_ERR_INVALID_ARGUMENT;
  if (fwd_state_capacity((int)batch_tiles(k), fwd_state_bytes) < 0) return GS_ERR_WORKSPACE;
  if (!aligned(fwd_state, 256)) return GS_ERR_INVALID_ARGUMENT;
  const int workers = worker_waves();
  if (workers <= 0) return GS_ERR_HIP;
  hipEvent_t e0, e1;
  timing_slot(1, e0, e1);
  return hip_status(gs_launch_render_bwd(n, splats, sorted_ids, tile_ranges, k, T_final, last,
                                         fwd_state, dL_drgb, dL_dT, dL_dsplat, accumulate,
                                         device_status, workers, e0, e1, (hipStream_t)stream));
}

// The camera of view 0 of a batch, with every view checked to be valid and of
// its size.
bool prep_batch_cams(const gs_camera *cams, int32_t n_views) {
  if (!cams || n_views < 1 || n_views > GS_MAX_VIEWS) return false;
  CamK k;
  for (int v = 0; v < n_views; v++) {
    if (!prep_camera(&cams[v], &k)) return false;
    if (cams[v].width != cams[0].width || cams[v].height != cams[0].height) return false;
  }
  return true;
}

}  // namespace

extern "C" {

int32_t gs_bin_tiles(int32_t n, const float *splats, const gs_camera *cam, int64_t pair_capacity,
                     int32_t *offsets, int32_t *tile_counts, uint64_t *keys, int32_t *ids,
                     int32_t *device_status, void *workspace, size_t workspace_bytes,
                     void *stream) {
  CamK k;
  if (!prep_camera(cam, &k)) return GS_ERR_INVALID_ARGUMENT;
  return bin_impl(n, splats, k, pair_capacity, offsets, tile_counts, keys, ids, device_status,
                  workspace, workspace_bytes, stream);
}

int32_t gs_sort_keys(int32_t n, const float *splats, const int32_t *offsets, int64_t pair_capacity,
                     const gs_camera *cam, uint64_t *sorted_keys, int32_t *sorted_ids,
                     int32_t *tile_ranges, int32_t *device_status, void *workspace,
                     size_t workspace_bytes, void *stream) {
  CamK k;
  if (!prep_camera(cam, &k)) return GS_ERR_INVALID_ARGUMENT;
  return sort_impl(n, splats, offsets, pair_capacity, k, sorted_keys, sorted_ids, tile_ranges,
                   device_status, workspace, workspace_bytes, stream);
}

int32_t gs_sort_keys_plan(int32_t n, const float *splats, const int32_t *offsets,
                          int64_t pair_capacity, const gs_camera *cam, uint64_t *sorted_keys,
                          int32_t *sorted_ids, int32_t *tile_ranges, const gs_sched *sched,
                          void *fwd_state, size_t fwd_state_bytes, int32_t *device_status,
                          void *workspace, size_t workspace_bytes, void *stream) {
  CamK k;
  if (!prep_camera(cam, &k)) return GS_ERR_INVALID_ARGUMENT;
  if (!fwd_state || !aligned(fwd_state, 256)) return GS_ERR_INVALID_ARGUMENT;
  const int64_t cap_pairs = fwd_state_capacity((int)batch_tiles(k), fwd_state_bytes);
  if (cap_pairs < 0) return GS_ERR_WORKSPACE;
  const gs_sched sc = sched ? *sched : default_sched();
  if (sc.chunk_mode < 0 || sc.chunk_mode > 2 || !(sc.eps >= 0.0f) || !(sc.lambda_ >= 0.0f) ||
      !(sc.beta >= 0.0f))
    return GS_ERR_INVALID_ARGUMENT;
  const int workers = worker_waves();
  if (workers <= 0) return GS_ERR_HIP;
  SortPlan plan;
  plan.fwd_state = fwd_state;
  plan.mode = sc.chunk_mode;
  plan.force_k = sc.force_k;
  plan.force_h = sc.force_h;
  plan.nblocks = workers / GS_WAVES_PER_BLOCK;
  plan.lambda_ = sc.lambda_;
  plan.beta = sc.beta;
  plan.eps = sc.eps;
  plan.cap = cap_pairs;
  return sort_impl(n, splats, offsets, pair_capacity, k, sorted_keys, sorted_ids, tile_ranges,
                   device_status, workspace, workspace_bytes, stream, &plan);
}

int32_t gs_plan_tiles(const int32_t *tile_counts, const gs_camera *cam, const gs_sched *sched,
                      void *fwd_state, size_t fwd_state_bytes, int32_t *device_status,
                      void *stream) {
  CamK k;
  if (!prep_camera(cam, &k)) return GS_ERR_INVALID_ARGUMENT;
  return plan_impl(tile_counts, k, sched, fwd_state, fwd_state_bytes, device_status, stream);
}

int32_t gs_render_fwd_bg(int32_t n, const float *splats, const int32_t *sorted_ids,
                         const int32_t *tile_ranges, const gs_camera *cam,
                         const gs_sched *sched, float *rgb, float *T_final, int32_t *last,
                         void *fwd_state, size_t fwd_state_bytes, int64_t *stats,
                         int32_t *pixel_hits, int32_t *device_status, const float *background,
                         void *stream) {
  CamK k;
  if (!prep_camera(cam, &k)) return GS_ERR_INVALID_ARGUMENT;
  return fwd_impl(n, splats, sorted_ids, tile_ranges, k, sched, rgb, T_final, last, fwd_state,
                  fwd_state_bytes, stats, pixel_hits, device_status, background, nullptr, 0,
                  stream);
}

int32_t gs_render_fwd_zero(int32_t n, const float *splats, const int32_t *sorted_ids,
                           const int32_t *tile_ranges, const gs_camera *cam,
                           const gs_sched *sched, float *rgb, float *T_final, int32_t *last,
                           void *fwd_state, size_t fwd_state_bytes, int64_t *stats,
                           int32_t *pixel_hits, int32_t *device_status, const float *background,
                           float *zero_out, int64_t zero_count, void *stream) {
  CamK k;
  if (!prep_camera(cam, &k)) return GS_ERR_INVALID_ARGUMENT;
  if (zero_count < 0 || (zero_count > 0 && !zero_out)) return GS_ERR_INVALID_ARGUMENT;
  return fwd_impl(n, splats, sorted_ids, tile_ranges, k, sched, rgb, T_final, last, fwd_state,
                  fwd_state_bytes, stats, pixel_hits, device_status, background, zero_out,
                  zero_count, stream);
}

int32_t gs_render_fwd(int32_t n, const float *splats, const int32_t *sorted_ids,
                      const int32_t *tile_ranges, const gs_camera *cam, const gs_sched *sched,
                      float *rgb, float *T_final, int32_t *last, void *fwd_state,
                      size_t fwd_state_bytes, int64_t *stats, int32_t *pixel_hits,
                      int32_t *device_status, void *stream) {
  return gs_render_fwd_bg(n, splats, sorted_ids, tile_ranges, cam, sched, rgb, T_final, last,
                          fwd_state, fwd_state_bytes, stats, pixel_hits, device_status, nullptr,
                          stream);
}

int32_t gs_render_bwd_bg(int32_t n, const float *splats, const int32_t *sorted_ids,
                         const int32_t *tile_ranges, const gs_camera *cam, const float *T_final,
                         const int32_t *last, void *fwd_state, size_t fwd_state_bytes,
                         const float *dL_drgb, float *dL_dsplat, int32_t *device_status,
                         const float *background, const float *dL_dT, void *stream) {
  CamK k;
  if (!prep_camera(cam, &k)) return GS_ERR_INVALID_ARGUMENT;
  return bwd_impl(n, splats, sorted_ids, tile_ranges, k, T_final, last, fwd_state,
                  fwd_state_bytes, dL_drgb, dL_dsplat, device_status, background, dL_dT, false,
                  stream);
}

int32_t gs_render_bwd(int32_t n, const float *splats, const int32_t *sorted_ids,
                      const int32_t *tile_ranges, const gs_camera *cam, const float *T_final,
                      const int32_t *last, void *fwd_state, size_t fwd_state_bytes,
                      const float *dL_drgb, float *dL_dsplat, int32_t *device_status,
                      void *stream) {
  return gs_render_bwd_bg(n, splats, sorted_ids, tile_ranges, cam, T_final, last, fwd_state,
                          fwd_state_bytes, dL_drgb, dL_dsplat, device_status, nullptr, nullptr,
                          stream);
}

// ---------------------------------------------------------------- batches of views

size_t gs_workspace_size_views(int32_t n, int32_t width, int32_t height, int32_t n_views,
                               int64_t pair_capacity) {
  if (n < 0 || width <= 0 || height <= 0 || pair_capacity < 0 || n_views < 1 ||
      n_views > GS_MAX_VIEWS)
    return 0;
  return gs_sort_ws_bytes(n, pair_capacity, (width + 15) / 16, ((height + 15) / 16) * n_views);
}

size_t gs_fwd_state_size_views(int32_t width, int32_t height, int32_t n_views,
                               int64_t pair_capacity) {
  if (width <= 0 || height <= 0 || n_views < 1 || n_views > GS_MAX_VIEWS) return 0;
  if (pair_capacity < 0 || pair_capacity >= GS_COUNT_LIMIT) return 0;
  const int64_t t = num_tiles(width, height) * n_views;
  if (t > GS_MAX_TILES) return 0;
  return fwd_layout((int)t, pair_capacity).total;
}

int32_t gs_project_views(int32_t n, const float *means, const float *log_scales,
                         const float *quats, const float *opacities, const float *sh,
                         int32_t sh_degree, const gs_camera *cams, int32_t n_views,
                         float *splats, void *stream) {
  if (n < 0 || sh_degree < 0 || sh_degree > 3 || !prep_batch_cams(cams, n_views))
    return GS_ERR_INVALID_ARGUMENT;
  if (n == 0) return GS_OK;
  if (!means || !log_scales || !quats || !opacities || !sh || !splats) return GS_ERR_INVALID_ARGUMENT;
  if (!aligned(quats, 16) || !aligned(splats, 16) || !aligned(sh, sh_align(sh_degree, false)))
    return GS_ERR_INVALID_ARGUMENT;
  for (int v = 0; v < n_views; v++) {
    CamK k;
    prep_camera(&cams[v], &k);
    k.view = v;
    const hipError_t e = gs_launch_project(n, means, log_scales, quats, opacities, sh, false,
                                           sh_degree, k, splats + (size_t)v * n * 12,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return GS_ERR_HIP;
  }
  return GS_OK;
}

int32_t gs_project_bwd_views(int32_t n, const float *means, const float *log_scales,
                             const float *quats, const float *opacities, const float *sh,
                             int32_t sh_degree, const gs_camera *cams, int32_t n_views,
                             const float *dL_dsplat, float *dL_dmeans, float *dL_dlog_scales,
                             float *dL_dquats, float *dL_dopacities, float *dL_dsh,
                             void *stream) {
  if (n < 0 || sh_degree < 0 || sh_degree > 3 || !prep_batch_cams(cams, n_views))
    return GS_ERR_INVALID_ARGUMENT;
  if (n == 0) return GS_OK;
  if (!means || !log_scales || !quats || !opacities || !sh || !dL_dsplat || !dL_dmeans ||
      !dL_dlog_scales || !dL_dquats || !dL_dopacities || !dL_dsh)
    return GS_ERR_INVALID_ARGUMENT;
  if (!aligned(quats, 16) || !aligned(dL_dquats, 16) ||
      !aligned(sh, sh_align(sh_degree, false)) || !aligned(dL_dsh, sh_align(sh_degree, false)))
    return GS_ERR_INVALID_ARGUMENT;
  for (int v = 0; v < n_views; v++) {
    CamK k;
    prep_camera(&cams[v], &k);
    k.view = v;
    const hipError_t e = gs_launch_project_bwd(
        n, means, log_scales, quats, opacities, sh, false, sh_degree, k,
        dL_dsplat + (size_t)v * n * 9, dL_dmeans, dL_dlog_scales, dL_dquats, dL_dopacities,
        dL_dsh, v > 0, (hipStream_t)stream);
    if (e != hipSuccess) return GS_ERR_HIP;
  }
  return GS_OK;
}

int32_t gs_bin_tiles_views(int32_t n, const float *splats, const gs_camera *cam, int32_t n_views,
                           int64_t pair_capacity, int32_t *offsets, int32_t *tile_counts,
                           uint64_t *keys, int32_t *ids, int32_t *device_status, void *workspace,
                           size_t workspace_bytes, void *stream) {
  CamK k;
  if (!prep_views(cam, n_views, &k)) return GS_ERR_INVALID_ARGUMENT;
  return bin_impl(n, splats, k, pair_capacity, offsets, tile_counts, keys, ids, device_status,
                  workspace, workspace_bytes, stream);
}

int32_t gs_sort_keys_views(int32_t n, const float *splats, const int32_t *offsets,
                           int64_t pair_capacity, const gs_camera *cam, int32_t n_views,
                           uint64_t *sorted_keys, int32_t *sorted_ids, int32_t *tile_ranges,
                           int32_t *device_status, void *workspace, size_t workspace_bytes,
                           void *stream) {
  CamK k;
  if (!prep_views(cam, n_views, &k)) return GS_ERR_INVALID_ARGUMENT;
  return sort_impl(n, splats, offsets, pair_capacity, k, sorted_keys, sorted_ids, tile_ranges,
                   device_status, workspace, workspace_bytes, stream);
}

int32_t gs_plan_tiles_views(const int32_t *tile_counts, const gs_camera *cam, int32_t n_views,
                            const gs_sched *sched, void *fwd_state, size_t fwd_state_bytes,
                            int32_t *device_status, void *stream) {
  CamK k;
  if (!prep_views(cam, n_views, &k)) return GS_ERR_INVALID_ARGUMENT;
  return plan_impl(tile_counts, k, sched, fwd_state, fwd_state_bytes, device_status, stream);
}

int32_t gs_render_fwd_views(int32_t n, const float *splats, const int32_t *sorted_ids,
                            const int32_t *tile_ranges, const gs_camera *cam, int32_t n_views,
                            const gs_sched *sched, float *rgb, float *T_final, int32_t *last,
                            void *fwd_state, size_t fwd_state_bytes, int64_t *stats,
                            int32_t *pixel_hits, int32_t *device_status,
                            const float *background, void *stream) {
  CamK k;
  if (!prep_views(cam, n_views, &k)) return GS_ERR_INVALID_ARGUMENT;
  return fwd_impl(n, splats, sorted_ids, tile_ranges, k, sched, rgb, T_final, last, fwd_state,
                  fwd_state_bytes, stats, pixel_hits, device_status, background, nullptr, 0,
                  stream);
}

int32_t gs_render_bwd_views(int32_t n, const float *splats, const int32_t *sorted_ids,
                            const int32_t *tile_ranges, const gs_camera *cam, int32_t n_views,
                            const float *T_final, const int32_t *last, void *fwd_state,
                            size_t fwd_state_bytes, const float *dL_drgb, float *dL_dsplat,
                            int32_t *device_status, const float *background,
                            const float *dL_dT, void *stream) {
  CamK k;
  if (!prep_views(cam, n_views, &k)) return GS_ERR_INVALID_ARGUMENT;
  return bwd_impl(n, splats, sorted_ids, tile_ranges, k, T_final, last, fwd_state,
                  fwd_state_bytes, dL_drgb, dL_dsplat, device_status, background, dL_dT, false,
                  stream);
}

int32_t gs_render_bwd_accumulate(int32_t n, const float *splats, const int32_t *sorted_ids,
                                 const int32_t *tile_ranges, const gs_camera *cam,
                                 int32_t n_views, const float *T_final, const int32_t *last,
                                 void *fwd_state, size_t fwd_state_bytes, const float *dL_drgb,
                                 float *dL_dsplat, int32_t *device_status,
                                 const float *background, const float *dL_dT, void *stream) {
  CamK k;
  if (!prep_views(cam, n_views, &k)) return GS_ERR_INVALID_ARGUMENT;
  return bwd_impl(n, splats, sorted_ids, tile_ranges, k, T_final, last, fwd_state,
                  fwd_state_bytes, dL_drgb, dL_dsplat, device_status, background, dL_dT, true,
                  stream);
}

// ---------------------------------------------------------------- allocation-free sort

}  // extern "C"

// The allocation-free sort's workspace: one array per GPU, held until the
// process ends. Host code never passes `scratch` itself to a kernel (on the
// host it names a stand-in, not device memory): each device's address comes
// from hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[GS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[SCRATCH_DEVICES] = {};

// The current device's scratch address (nullptr on a HIP error).
void *scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int32_t gs_sort_keys_noalloc(int32_t n, const float *splats, const gs_camera *cam,
                             int64_t pair_capacity, int32_t *offsets, uint64_t *sorted_keys,
                             int32_t *sorted_ids, int32_t *tile_ranges, int32_t *device_status,
                             void *stream) {
  CamK k;
  if (!prep_camera(cam, &k)) return GS_ERR_INVALID_ARGUMENT;
  if (n < 0 || pair_capacity < 0) return GS_ERR_INVALID_ARGUMENT;
  if (batch_tiles(k) > GS_MAX_TILES || n >= GS_COUNT_LIMIT || pair_capacity >= GS_COUNT_LIMIT)
    return GS_ERR_UNSUPPORTED;
  if (!offsets || !tile_ranges || !device_status || (n > 0 && !splats) ||
      (pair_capacity > 0 && !sorted_ids))
    return GS_ERR_INVALID_ARGUMENT;
  if ((splats && !aligned(splats, 16)) || (sorted_keys && !aligned(sorted_keys, 8)) ||
      !aligned(tile_ranges, 8))
    return GS_ERR_INVALID_ARGUMENT;
  // the frame must fit the static workspace: checked before any HIP call
  if (gs_sort_ws_bytes(n, pair_capacity, k.tiles_x, k.tiles_y) > GS_NOALLOC_SCRATCH_BYTES)
    return GS_ERR_WORKSPACE;
  void *ws = scratch_on_current_device();
  if (!ws) return GS_ERR_HIP;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = gs_launch_bin(n, splats, k, pair_capacity, offsets, nullptr, nullptr, nullptr,
                               device_status, ws, st);
  if (e != hipSuccess) return GS_ERR_HIP;
  return hip_status(gs_launch_sort(n, splats, offsets, pair_capacity, k, sorted_keys, sorted_ids,
                                   tile_ranges, device_status, ws, nullptr, st));
}

int32_t gs_set_wait_limit(int32_t probes) {
  return g_wait_limit.exchange(probes < 0 ? -1 : probes, std::memory_order_relaxed);
}

int32_t gs_timing_start(void) {
  if (!g_timing.made) {
    for (int w = 0; w < 2; w++)
      for (int i = 0; i < TIMING_SLOTS; i++)
        for (int j = 0; j < 2; j++)
          if (hipEventCreate(&g_timing.ev[w][i][j]) != hipSuccess) return GS_ERR_HIP;
    g_timing.made = true;
  }
  g_timing.used[0] = g_timing.used[1] = 0;
  g_timing.on = true;
  return GS_OK;
}

int32_t gs_timing_read(int32_t which, float *ms, int32_t cap) {
  if (which < 0 || which > 1 || cap < 0 || (cap > 0 && !ms)) return GS_ERR_INVALID_ARGUMENT;
  g_timing.on = false;
  if (!g_timing.made) return 0;
  const int n = g_timing.used[which] < cap ? g_timing.used[which] : cap;
  for (int i = 0; i < n; i++) {
    if (hipEventSynchronize(g_timing.ev[which][i][1]) != hipSuccess) return GS_ERR_HIP;
    if (hipEventElapsedTime(&ms[i], g_timing.ev[which][i][0], g_timing.ev[which][i][1]) !=
        hipSuccess)
      return GS_ERR_HIP;
  }
  return n;
}

}  // extern "C"
