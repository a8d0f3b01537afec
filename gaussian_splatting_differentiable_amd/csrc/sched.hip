// gs_plan_tiles and the schedule launch of gs_render_fwd: one workgroup runs
// the per-frame schedule (sched_body.h).
#include "sched_body.h"

namespace {

using namespace sched_impl;

template <bool LDS>
__global__ void __launch_bounds__(NT) k_schedule(const int2 *__restrict__ ranges,
                                                 const int32_t *__restrict__ counts_in, int T,
                                                 int tiles_x, int chunk_mode, int force_k,
                                                 int force_h, double lambda_, double beta,
                                                 double eps, int nblocks,
                                                 char *__restrict__ fwd_state,
                                                 unsigned long long *__restrict__ stats,
                                                 int32_t *__restrict__ status, int64_t cap_pairs) {
  extern __shared__ __align__(16) uint32_t dyn[];
  schedule_frame<LDS>(ranges, counts_in, T, tiles_x, chunk_mode, force_k, force_h, lambda_, beta,
                      eps, nblocks, fwd_state, stats, status, cap_pairs, dyn);
}

}  // namespace

// ranges: the frame's tile ranges (the forward call), or null with counts: the
// per-tile pair counts of the binning pass (the plan built ahead).
hipError_t gs_launch_schedule(const int32_t *ranges, const int32_t *counts, const CamK &cam,
                              int chunk_mode, int force_k, int force_h, double lambda_,
                              double beta, double eps, int nblocks, void *fwd_state,
                              int64_t *stats, int32_t *status, int64_t cap_pairs,
                              hipStream_t st) {
  const int T = cam.tiles_x * cam.tiles_y;
  const size_t lds = T <= TL ? LDS_BYTES : POLICY_BYTES;
  static_assert(POLICY_BYTES <= 4 * (size_t)TL, "the policy arrays fit in the first LDS array");
  auto kern = T <= TL ? k_schedule<true> : k_schedule<false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(1), dim3(NT), lds, st, reinterpret_cast<const int2 *>(ranges),
                     counts, T, cam.tiles_x, chunk_mode, force_k, force_h, lambda_, beta, eps, nblocks,
                     reinterpret_cast<char *>(fwd_state),
                     reinterpret_cast<unsigned long long *>(stats), status, cap_pairs);
  return hipGetLastError();
}
