// Device-wide exclusive prefix sums over int32 (reduce, scan of block sums, apply).
// Used for the per-splat pair offsets of the binning pass, the visible-splat
// compaction, the depth-ordered pair offsets and the radix-sort digit tables.
// The element count may live on the device (a count produced by an earlier
// kernel of the same frame), so no host synchronisation is needed.
#include "gs_common.h"

namespace {

constexpr int SCAN_THREADS = 256;
constexpr int SCAN_ITEMS = 8;
constexpr int SCAN_TILE = SCAN_THREADS * SCAN_ITEMS;  // 2048 elements per block

__device__ __forceinline__ int resolve_n(const int32_t *n_dev, int n_max) {
  if (!n_dev) return n_max;
  const int v = *n_dev;
  return v < 0 ? 0 : (v < n_max ? v : n_max);
}

// Inclusive scan across the 256 threads of a block; returns the block total too.
__device__ __forceinline__ int block_incl_scan(int v, int &total) {
  __shared__ int wsum[SCAN_THREADS / GS_WAVE];
  const int lane = threadIdx.x & (GS_WAVE - 1), wid = threadIdx.x / GS_WAVE;
#pragma unroll
  for (int d = 1; d < GS_WAVE; d <<= 1) {
    const int t = __shfl_up(v, d, GS_WAVE);
    if (lane >= d) v += t;
  }
  if (lane == GS_WAVE - 1) wsum[wid] = v;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SCAN_THREADS / GS_WAVE; w++) {
    const int s = wsum[w];
    base += (w < wid) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return v + base;
}

__global__ void __launch_bounds__(SCAN_THREADS) k_scan_reduce(const int32_t *__restrict__ in,
                                                              const int32_t *n_dev, int n_max,
                                                              int32_t *__restrict__ bsum) {
  const int n = resolve_n(n_dev, n_max);
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE;
  int v = 0;
  if (base < n) {
#pragma unroll
    for (int j = 0; j < SCAN_ITEMS; j++) {
      const int64_t idx = base + (int64_t)j * SCAN_THREADS + threadIdx.x;
      v += idx < n ? in[idx] : 0;
    }
  }
  int total;
  block_incl_scan(v, total);
  if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

// One block scans the block sums (exclusive) in place; bsum[nb] <- grand total.
__global__ void __launch_bounds__(1024) k_scan_top(int32_t *__restrict__ bsum, const int32_t *n_dev,
                                                   int n_max) {
  const int n = resolve_n(n_dev, n_max);
  const int nb = (n + SCAN_TILE - 1) / SCAN_TILE;
  __shared__ int wsum[16];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  const int lane = threadIdx.x & (GS_WAVE - 1), wid = threadIdx.x / GS_WAVE;
  for (int c0 = 0; c0 < nb; c0 += 1024) {
    const int idx = c0 + threadIdx.x;
    int x = idx < nb ? bsum[idx] : 0, v = x;
#pragma unroll
    for (int d = 1; d < GS_WAVE; d <<= 1) {
      const int t = __shfl_up(v, d, GS_WAVE);
      if (lane >= d) v += t;
    }
    if (lane == GS_WAVE - 1) wsum[wid] = v;
    __syncthreads();
    int base = carry, tot = 0;
    for (int w = 0; w < 16; w++) {
      base += (w < wid) ? wsum[w] : 0;
      tot += wsum[w];
    }
    if (idx < nb) bsum[idx] = base + v - x;
    __syncthreads();
    if (threadIdx.x == 0) carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) bsum[nb] = carry;
}

__global__ void __launch_bounds__(SCAN_THREADS) k_scan_apply(const int32_t *in, int32_t *out,
                                                             const int32_t *n_dev, int n_max,
                                                             const int32_t *__restrict__ bsum) {
  const int n = resolve_n(n_dev, n_max);
  const int nb = (n + SCAN_TILE - 1) / SCAN_TILE;
  if (blockIdx.x == 0 && threadIdx.x == 0) out[n] = bsum[nb];
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE;
  if (base >= n) return;
  // blocked layout: thread t owns elements base + t*8 .. +7
  int x[SCAN_ITEMS];
  int v = 0;
#pragma unroll
  for (int j = 0; j < SCAN_ITEMS; j++) {
    const int64_t idx = base + (int64_t)threadIdx.x * SCAN_ITEMS + j;
    x[j] = idx < n ? in[idx] : 0;
    v += x[j];
  }
  int total;
  const int incl = block_incl_scan(v, total);
  int run = bsum[blockIdx.x] + incl - v;
#pragma unroll
  for (int j = 0; j < SCAN_ITEMS; j++) {
    const int64_t idx = base + (int64_t)threadIdx.x * SCAN_ITEMS + j;
    if (idx < n) out[idx] = run;
    run += x[j];
  }
}

}  // namespace

// Exclusive scan of in[0..n) into out[0..n), out[n] = total. n = min(*n_dev, n_max)
// when n_dev is given. in may equal out. block_buf needs scan_buf_elems(n_max) ints.
int gs_scan_buf_elems(int n_max) { return (n_max + SCAN_TILE - 1) / SCAN_TILE + 2; }

hipError_t gs_launch_scan_i32_dev(const int32_t *in, int32_t *out, const int32_t *n_dev, int n_max,
                                  int32_t *block_buf, hipStream_t st) {
  const int nb = (n_max + SCAN_TILE - 1) / SCAN_TILE;
  const int grid = nb > 0 ? nb : 1;
  hipLaunchKernelGGL(k_scan_reduce, dim3(grid), dim3(SCAN_THREADS), 0, st, in, n_dev, n_max,
                     block_buf);
  hipLaunchKernelGGL(k_scan_top, dim3(1), dim3(1024), 0, st, block_buf, n_dev, n_max);
  hipLaunchKernelGGL(k_scan_apply, dim3(grid), dim3(SCAN_THREADS), 0, st, in, out, n_dev, n_max,
                     block_buf);
  return hipGetLastError();
}

hipError_t gs_launch_scan_i32(const int32_t *in, int32_t *out, int n, int32_t *block_buf,
                              hipStream_t st) {
  return gs_launch_scan_i32_dev(in, out, nullptr, n, block_buf, st);
}
