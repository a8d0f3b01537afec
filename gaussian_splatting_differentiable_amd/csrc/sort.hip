// gs_sort_keys: order the (tile, depth) pairs and cut the tile ranges.
//
// "What the 3DGS Literature Left on the Table", Step 1 (d), Figure 5: instead of
// one wide (tile | depth) key sort over all pairs, sort the visible splats once by
// their 32-bit depth, lay their pairs out in that order, then run a narrow stable
// sort over the tile ids. The result is ordered by (tile, depth, splat id): the
// depth sort is stable over an id-ordered input, and the tile sort is stable.
//
// Radix passes are LSD, one wavefront per block (no barriers): a histogram pass
// (LDS atomics), a device-wide scan of the digit-major table, and a scatter pass
// whose stable rank comes from per-bit ballots (a 64-lane match) plus running
// per-digit offsets kept in LDS.
#include "gs_common.h"

hipError_t gs_launch_scan_i32_dev(const int32_t *in, int32_t *out, const int32_t *n_dev, int n_max,
                                  int32_t *block_buf, hipStream_t st);
int gs_scan_buf_elems(int n_max);

namespace {

constexpr int RADIX_RPT = 32;                            // rounds of 64 items per block
constexpr int RADIX_ITEMS = GS_WAVE * RADIX_RPT;         // 2048 items per block

__device__ __forceinline__ int resolve_n(const int32_t *n_dev, int n_max) {
  const int v = *n_dev;
  return v < 0 ? 0 : (v < n_max ? v : n_max);
}

// flags[i] = splat i emits at least one pair
__global__ void __launch_bounds__(256) k_flag_visible(int n, const int32_t *__restrict__ offsets,
                                                      int64_t capacity, int32_t *__restrict__ flags) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const bool overflow = (int64_t)offsets[n] > capacity;
  flags[i] = (!overflow && offsets[i + 1] > offsets[i]) ? 1 : 0;
}

__global__ void __launch_bounds__(256) k_compact_visible(int n, const int32_t *__restrict__ offsets,
                                                         const int32_t *__restrict__ cidx,
                                                         const Splat *__restrict__ splats,
                                                         int64_t capacity,
                                                         uint32_t *__restrict__ dkey,
                                                         int32_t *__restrict__ dval) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if ((int64_t)offsets[n] > capacity) return;
  if (offsets[i + 1] > offsets[i]) {
    const int c = cidx[i];
    dkey[c] = __float_as_uint(splats[i].p2.z);
    dval[c] = i;
  }
}

template <int BITS>
__global__ void __launch_bounds__(GS_WAVE) k_radix_hist(const uint32_t *__restrict__ keys,
                                                        const int32_t *n_dev, int n_max, int shift,
                                                        int nblk, int32_t *__restrict__ hist) {
  constexpr int B = 1 << BITS;
  __shared__ int cnt[B];
  const int n = resolve_n(n_dev, n_max);
  for (int d = threadIdx.x; d < B; d += GS_WAVE) cnt[d] = 0;
  __builtin_amdgcn_wave_barrier();
  const int64_t base = (int64_t)blockIdx.x * RADIX_ITEMS;
  for (int r = 0; r < RADIX_RPT; r++) {
    const int64_t idx = base + r * GS_WAVE + threadIdx.x;
    if (idx < n) atomicAdd(&cnt[(keys[idx] >> shift) & (B - 1)], 1);
  }
  __builtin_amdgcn_wave_barrier();
  __syncthreads();
  for (int d = threadIdx.x; d < B; d += GS_WAVE) hist[d * nblk + blockIdx.x] = cnt[d];
}

template <int BITS>
__global__ void __launch_bounds__(GS_WAVE) k_radix_scatter(
    const uint32_t *__restrict__ kin, const int32_t *__restrict__ vin, uint32_t *__restrict__ kout,
    int32_t *__restrict__ vout, const int32_t *n_dev, int n_max, int shift, int nblk,
    const int32_t *__restrict__ hist_scan) {
  constexpr int B = 1 << BITS;
  __shared__ int run[B];
  const int n = resolve_n(n_dev, n_max);
  const int64_t base = (int64_t)blockIdx.x * RADIX_ITEMS;
  if (base >= n) return;
  for (int d = threadIdx.x; d < B; d += GS_WAVE) run[d] = hist_scan[d * nblk + blockIdx.x];
  __syncthreads();
  const uint64_t lt = (1ull << threadIdx.x) - 1ull;
  for (int r = 0; r < RADIX_RPT; r++) {
    const int64_t idx = base + r * GS_WAVE + threadIdx.x;
    const bool valid = idx < n;
    uint32_t k = 0;
    int32_t v = 0;
    if (valid) {
      k = kin[idx];
      v = vin[idx];
    }
    const uint32_t d = (k >> shift) & (B - 1);
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < BITS; b++) {
      const uint64_t bal = __ballot((d >> b) & 1u);
      peers &= ((d >> b) & 1u) ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt);
    const int cnt = __popcll(peers);
    int dst = 0;
    if (valid) dst = run[d] + rank;
    __builtin_amdgcn_wave_barrier();
    __syncthreads();
    if (valid && rank == cnt - 1) run[d] = dst + 1;
    __syncthreads();
    if (valid) {
      kout[dst] = k;
      vout[dst] = v;
    }
  }
}

// pairs of the r-th splat in depth order
__global__ void __launch_bounds__(256) k_depth_counts(const int32_t *__restrict__ m_dev, int n,
                                                      const int32_t *__restrict__ dval,
                                                      const int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ dcnt) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= resolve_n(m_dev, n)) return;
  const int g = dval[r];
  dcnt[r] = offsets[g + 1] - offsets[g];
}

// Lay the pairs out in (depth, id) order: tile ids and splat ids.
__global__ void __launch_bounds__(256) k_gather_pairs(const int32_t *__restrict__ m_dev, int n,
                                                      const int32_t *__restrict__ dval,
                                                      const int32_t *__restrict__ doff,
                                                      const int32_t *__restrict__ offsets,
                                                      const uint64_t *__restrict__ keys,
                                                      uint32_t *__restrict__ tile_out,
                                                      int32_t *__restrict__ id_out) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= resolve_n(m_dev, n)) return;
  const int g = dval[r];
  const int src = offsets[g], cnt = offsets[g + 1] - src, dst = doff[r];
  const uint32_t *k32 = reinterpret_cast<const uint32_t *>(keys);
  for (int j = 0; j < cnt; j++) {
    tile_out[dst + j] = k32[2 * (int64_t)(src + j) + 1];
    id_out[dst + j] = g;
  }
}

// Pairs to sort this frame: I, or 0 when the pair buffer overflowed.
__global__ void k_effective_count(int n, const int32_t *__restrict__ offsets, int64_t capacity,
                                  int32_t *__restrict__ out) {
  const int32_t I = offsets[n];
  *out = ((int64_t)I <= capacity) ? I : 0;
}

__global__ void __launch_bounds__(256) k_ranges_init(int ntiles, int32_t *__restrict__ ranges) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < ntiles) {
    ranges[2 * t] = -1;
    ranges[2 * t + 1] = -1;
  }
}

__global__ void __launch_bounds__(256) k_ranges_bounds(const int32_t *__restrict__ i_dev, int cap,
                                                       const uint32_t *__restrict__ tiles,
                                                       int32_t *__restrict__ ranges) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  const int I = resolve_n(i_dev, cap);
  if (k >= I) return;
  const uint32_t t = tiles[k];
  if (k == 0 || tiles[k - 1] != t) ranges[2 * t] = k;
  if (k == I - 1 || tiles[k + 1] != t) ranges[2 * t + 1] = k + 1;
}

// Empty tiles get start = end = number of pairs of lower tiles: a prefix max of
// the ends of the non-empty tiles (one block).
__global__ void __launch_bounds__(1024) k_ranges_fill(int ntiles, int32_t *__restrict__ ranges) {
  __shared__ int wmax[16];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  const int lane = threadIdx.x & (GS_WAVE - 1), wid = threadIdx.x / GS_WAVE;
  for (int c0 = 0; c0 < ntiles; c0 += 1024) {
    const int t = c0 + threadIdx.x;
    const int e = t < ntiles ? ranges[2 * t + 1] : -1;
    int v = e;
#pragma unroll
    for (int d = 1; d < GS_WAVE; d <<= 1) {
      const int o = __shfl_up(v, d, GS_WAVE);
      if (lane >= d) v = max(v, o);
    }
    if (lane == GS_WAVE - 1) wmax[wid] = v;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wid; w++) before = max(before, wmax[w]);
    // exclusive prefix max within the wave
    int excl = __shfl_up(v, 1, GS_WAVE);
    if (lane == 0) excl = -1;
    before = max(before, excl);
    if (t < ntiles && e < 0) {
      const int s = max(before, 0);
      ranges[2 * t] = s;
      ranges[2 * t + 1] = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int m = carry;
      for (int w = 0; w < 16; w++) m = max(m, wmax[w]);
      carry = m;
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(256) k_sorted_keys(const int32_t *__restrict__ i_dev, int cap,
                                                     const uint32_t *__restrict__ tiles,
                                                     const int32_t *__restrict__ ids,
                                                     const Splat *__restrict__ splats,
                                                     uint64_t *__restrict__ out) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= resolve_n(i_dev, cap)) return;
  out[k] = ((uint64_t)tiles[k] << 32) | (uint64_t)__float_as_uint(splats[ids[k]].p2.z);
}

template <int BITS>
hipError_t radix_pass(const uint32_t *kin, const int32_t *vin, uint32_t *kout, int32_t *vout,
                      const int32_t *n_dev, int n_max, int shift, int32_t *hist, int32_t *scan_buf,
                      hipStream_t st) {
  const int nblk = gs_div_up(n_max > 0 ? n_max : 1, RADIX_ITEMS);
  constexpr int B = 1 << BITS;
  hipLaunchKernelGGL(k_radix_hist<BITS>, dim3(nblk), dim3(GS_WAVE), 0, st, kin, n_dev, n_max, shift,
                     nblk, hist);
  hipError_t e = gs_launch_scan_i32_dev(hist, hist, nullptr, B * nblk, scan_buf, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_radix_scatter<BITS>, dim3(nblk), dim3(GS_WAVE), 0, st, kin, vin, kout, vout,
                     n_dev, n_max, shift, nblk, hist);
  return hipGetLastError();
}

}  // namespace

// Workspace layout of the sort stage (int32 elements).
struct SortWs {
  int32_t *flags, *cidx, *dcnt;            // n+1 each
  uint32_t *dk[2];                         // n each
  int32_t *dv[2];
  uint32_t *tk[2];                         // capacity each
  int32_t *tv[2];
  int32_t *hist;                           // 256 * blocks(capacity) + 1
  int32_t *scan_buf;
  int32_t *npairs;                         // [1]: pairs to sort
};

size_t gs_sort_ws_bytes(int n, int64_t cap) {
  const int64_t nn = (int64_t)n + 2;
  const int64_t items = cap > (int64_t)n ? cap : (int64_t)n;  // both sorts share the table
  const int64_t nblk = (items + RADIX_ITEMS - 1) / RADIX_ITEMS + 1;
  const int64_t hist = 256 * nblk + 2;
  const int64_t maxscan = hist > nn ? hist : nn;
  int64_t elems = 3 * nn + 4 * nn + 4 * (cap + 2) + hist + gs_scan_buf_elems((int)maxscan) + 64;
  return (size_t)elems * 4 + 16 * 256;
}

static SortWs carve(void *ws, int n, int64_t cap) {
  char *p = reinterpret_cast<char *>(ws);
  auto take = [&](int64_t elems) {
    char *r = p;
    p += ((elems * 4 + 255) / 256) * 256;
    return r;
  };
  const int64_t nn = (int64_t)n + 2;
  const int64_t items = cap > (int64_t)n ? cap : (int64_t)n;
  const int64_t nblk = (items + RADIX_ITEMS - 1) / RADIX_ITEMS + 1;
  const int64_t hist = 256 * nblk + 2;
  const int64_t maxscan = hist > nn ? hist : nn;
  SortWs w;
  w.flags = (int32_t *)take(nn);
  w.cidx = (int32_t *)take(nn);
  w.dcnt = (int32_t *)take(nn);
  w.dk[0] = (uint32_t *)take(nn);
  w.dk[1] = (uint32_t *)take(nn);
  w.dv[0] = (int32_t *)take(nn);
  w.dv[1] = (int32_t *)take(nn);
  w.tk[0] = (uint32_t *)take(cap + 2);
  w.tk[1] = (uint32_t *)take(cap + 2);
  w.tv[0] = (int32_t *)take(cap + 2);
  w.tv[1] = (int32_t *)take(cap + 2);
  w.hist = (int32_t *)take(hist);
  w.scan_buf = (int32_t *)take(gs_scan_buf_elems((int)maxscan));
  w.npairs = (int32_t *)take(1);
  return w;
}

hipError_t gs_launch_sort(int n, const float *splats, const int32_t *offsets, const uint64_t *keys,
                          int64_t cap, const CamK &cam, uint64_t *sorted_keys, int32_t *sorted_ids,
                          int32_t *ranges, void *ws, hipStream_t st) {
  const Splat *sp = reinterpret_cast<const Splat *>(splats);
  SortWs w = carve(ws, n, cap);
  const int ntiles = cam.tiles_x * cam.tiles_y;
  const int capi = (int)cap;
  hipError_t e;
  const dim3 b256(256);
  const dim3 gn(gs_div_up(n > 0 ? n : 1, 256));
  // 1. compact the splats that emit pairs, in id order
  hipLaunchKernelGGL(k_flag_visible, gn, b256, 0, st, n, offsets, cap, w.flags);
  if ((e = gs_launch_scan_i32_dev(w.flags, w.cidx, nullptr, n, w.scan_buf, st)) != hipSuccess) return e;
  const int32_t *m_dev = w.cidx + n;  // number of visible splats
  hipLaunchKernelGGL(k_compact_visible, gn, b256, 0, st, n, offsets, w.cidx, sp, cap, w.dk[0], w.dv[0]);
  // 2. stable depth sort of the visible splats (4 passes of 8 bits)
  int cur = 0;
  for (int pass = 0; pass < 4; pass++) {
    if ((e = radix_pass<8>(w.dk[cur], w.dv[cur], w.dk[cur ^ 1], w.dv[cur ^ 1], m_dev, n, 8 * pass,
                           w.hist, w.scan_buf, st)) != hipSuccess)
      return e;
    cur ^= 1;
  }
  const int32_t *dval = w.dv[cur];
  // 3. depth-ordered pair offsets, then the pairs in (depth, id) order
  hipLaunchKernelGGL(k_depth_counts, gn, b256, 0, st, m_dev, n, dval, offsets, w.dcnt);
  if ((e = gs_launch_scan_i32_dev(w.dcnt, w.dcnt, m_dev, n, w.scan_buf, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_gather_pairs, gn, b256, 0, st, m_dev, n, dval, w.dcnt, offsets, keys,
                     w.tk[0], w.tv[0]);
  // 4. stable sort by tile id; the last pass writes sorted_ids directly
  hipLaunchKernelGGL(k_effective_count, dim3(1), dim3(1), 0, st, n, offsets, cap, w.npairs);
  const int32_t *i_dev = w.npairs;
  int tbits = 1;
  while ((1 << tbits) < ntiles) tbits++;
  const uint32_t *tiles_sorted;
  if (tbits <= 8) {
    if ((e = radix_pass<8>(w.tk[0], w.tv[0], w.tk[1], sorted_ids, i_dev, capi, 0, w.hist, w.scan_buf, st)) != hipSuccess) return e;
    tiles_sorted = w.tk[1];
  } else if (tbits <= 14) {
    if ((e = radix_pass<7>(w.tk[0], w.tv[0], w.tk[1], w.tv[1], i_dev, capi, 0, w.hist, w.scan_buf, st)) != hipSuccess) return e;
    if ((e = radix_pass<7>(w.tk[1], w.tv[1], w.tk[0], sorted_ids, i_dev, capi, 7, w.hist, w.scan_buf, st)) != hipSuccess) return e;
    tiles_sorted = w.tk[0];
  } else {
    if ((e = radix_pass<8>(w.tk[0], w.tv[0], w.tk[1], w.tv[1], i_dev, capi, 0, w.hist, w.scan_buf, st)) != hipSuccess) return e;
    if ((e = radix_pass<8>(w.tk[1], w.tv[1], w.tk[0], sorted_ids, i_dev, capi, 8, w.hist, w.scan_buf, st)) != hipSuccess) return e;
    tiles_sorted = w.tk[0];
  }
  // 5. optional keys and the tile ranges
  const int gc = gs_div_up(cap > 0 ? cap : 1, 256);
  if (sorted_keys)
    hipLaunchKernelGGL(k_sorted_keys, dim3(gc), b256, 0, st, i_dev, capi, tiles_sorted, sorted_ids, sp, sorted_keys);
  hipLaunchKernelGGL(k_ranges_init, dim3(gs_div_up(ntiles, 256)), b256, 0, st, ntiles, ranges);
  hipLaunchKernelGGL(k_ranges_bounds, dim3(gc), b256, 0, st, i_dev, capi, tiles_sorted, ranges);
  hipLaunchKernelGGL(k_ranges_fill, dim3(1), dim3(1024), 0, st, ntiles, ranges);
  return hipGetLastError();
}
