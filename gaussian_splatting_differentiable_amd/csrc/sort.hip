// gs_sort_keys: order the (tile, depth) pairs and cut the tile ranges.
//
// "What the 3DGS Literature Left on the Table", Step 1 (d), Figure 5: filter the
// visible splats, sort them once front to back by their 32-bit depth, emit the
// tile keys in that depth order, then run a narrow stable sort over the tile ids.
// The result is ordered by (tile, depth, splat id): the depth sort is stable over
// an id-ordered input and the tile sort is stable.
//
// Radix passes are onesweep-style LSD passes, one kernel per digit. A block takes
// a partition by atomic ticket, ranks its 4096 keys stably (per-wave ballot match
// on the digit bits), publishes its digit counts and looks back over earlier
// partitions for its global offsets (decoupled look-back: a partition only waits
// for partitions with a lower ticket, which are already running, and the wait is
// bounded). Keys are reordered in LDS so that global writes are contiguous runs
// per digit. Per-tile counts come from an LDS histogram in the emission kernel;
// the tile ranges are their exclusive prefix sum.
//
// This TU includes the canonical binning code: compile with -ffp-contract=off.
#include <stddef.h>

#include "bin_spans.h"

namespace {

constexpr int OS_THREADS = 1024;
constexpr int OS_WAVES = OS_THREADS / 64;
constexpr int OS_ITEMS = 16;
constexpr int OS_PART = OS_THREADS * OS_ITEMS;  // keys per partition
constexpr uint32_t ST_AGG = 1u << 30, ST_INC = 2u << 30, ST_CNT = (1u << 30) - 1;
constexpr int SPIN_LIMIT = 1 << 22;
constexpr int HIST_TILES_LDS = 16384;  // tile histogram kept in LDS up to this many tiles
constexpr int SCAN_T = 256, SCAN_I = 8, SCAN_TILE = SCAN_T * SCAN_I;

// Per-call control block at the start of the sort workspace.
struct SortCtl {
  int32_t m;               // visible splats (with at least one pair)
  int32_t npairs;          // pairs of this frame (0 after an overflow)
  int32_t err;             // a look-back wait hit its bound (never expected)
  int32_t tickets[8];      // partition tickets, one per radix pass
  uint32_t dhist[4][256];  // depth digit histograms
  uint32_t dbase[4][256];  // depth digit exclusive offsets
  uint32_t tbase[2][256];  // tile digit exclusive offsets
};

__device__ __forceinline__ int clamp_n(int v, int hi) { return v < 0 ? 0 : (v < hi ? v : hi); }

__device__ __forceinline__ uint32_t ld_status(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_status(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive scan over a 256-thread block; total of the block in `total`.
__device__ __forceinline__ int block_scan256(int v, int &total) {
  __shared__ int wsum[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; w++) {
    base += (w < wid) ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();
  total = tot;
  return v + base;
}

__device__ __forceinline__ bool splat_visible(const int32_t *offsets, int i, bool overflow) {
  return !overflow && offsets[i + 1] > offsets[i];
}

// Inclusive scan over a block of OS_THREADS threads; total in `total`.
__device__ __forceinline__ int block_scan_os(int v, int &total) {
  __shared__ int wsum[OS_WAVES];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < OS_WAVES; w++) {
    base += (w < wid) ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();
  total = tot;
  return v + base;
}

// ---------------------------------------------------------------- setup

__global__ void __launch_bounds__(1024) k_sort_init(SortCtl *__restrict__ ctl,
                                                    int32_t *__restrict__ tile_counts, int ntiles) {
  int32_t *w = reinterpret_cast<int32_t *>(ctl);
  const int nw = (int)(sizeof(SortCtl) / 4);
  for (int i = threadIdx.x; i < nw; i += blockDim.x) w[i] = 0;
  for (int i = threadIdx.x; i < ntiles; i += blockDim.x) tile_counts[i] = 0;
}

// Depth digit histograms of the visible splats (all four passes at once); also
// clears the look-back status words of every pass.
__global__ void __launch_bounds__(256) k_depth_hist(int n, const Splat *__restrict__ splats,
                                                   const int32_t *__restrict__ offsets,
                                                   int64_t cap, SortCtl *__restrict__ ctl,
                                                   uint32_t *__restrict__ status, int64_t nstatus) {
  __shared__ uint32_t h[4][256];
  for (int i = threadIdx.x; i < 1024; i += 256) (&h[0][0])[i] = 0;
  __syncthreads();
  const bool overflow = (int64_t)offsets[n] > cap;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nstatus;
       i += (int64_t)gridDim.x * 256)
    status[i] = 0;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    if (!splat_visible(offsets, i, overflow)) continue;
    const uint32_t k = __float_as_uint(splats[i].p2.z);
#pragma unroll
    for (int p = 0; p < 4; p++) atomicAdd(&h[p][(k >> (8 * p)) & 255], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 1024; i += 256) {
    const uint32_t v = (&h[0][0])[i];
    if (v) atomicAdd(&ctl->dhist[0][0] + i, v);
  }
}

__global__ void __launch_bounds__(256) k_depth_bases(SortCtl *__restrict__ ctl) {
  for (int p = 0; p < 4; p++) {
    int tot;
    const int v = (int)ctl->dhist[p][threadIdx.x];
    const int incl = block_scan256(v, tot);
    ctl->dbase[p][threadIdx.x] = (uint32_t)(incl - v);
    if (p == 0 && threadIdx.x == 0) ctl->m = tot;
  }
}

// ---------------------------------------------------------------- onesweep pass

// FIRST: the keys are the depths of the visible splats read in id order (the
// compaction is fused into the first pass); otherwise keys/values come from kin/vin.
template <int BITS, bool FIRST>
__global__ void __launch_bounds__(OS_THREADS) k_onesweep(
    const uint32_t *__restrict__ kin, const uint32_t *__restrict__ vin, uint32_t *__restrict__ kout,
    uint32_t *__restrict__ vout, const int32_t *__restrict__ n_dev, int n_max,
    const Splat *__restrict__ splats, const int32_t *__restrict__ offsets, int64_t cap, int shift,
    const uint32_t *__restrict__ digit_base, uint32_t *__restrict__ status,
    int32_t *__restrict__ ticket, int32_t *__restrict__ err) {
  constexpr int B = 1 << BITS;
  __shared__ uint32_t s_key[OS_PART];
  __shared__ uint32_t s_val[OS_PART];
  __shared__ int s_wcnt[OS_WAVES][B];
  __shared__ int s_lbase[B];
  __shared__ uint32_t s_gbase[B];
  __shared__ int s_part, s_nvalid;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) s_part = atomicAdd(ticket, 1);
  for (int i = tid; i < OS_WAVES * B; i += OS_THREADS) (&s_wcnt[0][0])[i] = 0;
  __syncthreads();
  const int part = s_part;
  const int n = FIRST ? n_max : clamp_n(*n_dev, n_max);
  const bool overflow = FIRST ? ((int64_t)offsets[n_max] > cap) : false;
  const int64_t base = (int64_t)part * OS_PART + (int64_t)w * (OS_ITEMS * 64);
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t key[OS_ITEMS], val[OS_ITEMS];
  int rnk[OS_ITEMS];
#pragma unroll
  for (int r = 0; r < OS_ITEMS; r++) {
    const int64_t e = base + r * 64 + lane;
    bool valid = e < n;
    uint32_t k = 0, v = 0;
    if (valid) {
      if constexpr (FIRST) {
        valid = splat_visible(offsets, (int)e, overflow);
        if (valid) {
          k = __float_as_uint(splats[e].p2.z);
          v = (uint32_t)e;
        }
      } else {
        k = kin[e];
        v = vin[e];
      }
    }
    const uint32_t d = (k >> shift) & (B - 1);
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < BITS; b++) {
      const uint64_t bal = __ballot((d >> b) & 1u);
      peers &= ((d >> b) & 1u) ? bal : ~bal;
    }
    int wr = -1;
    if (valid) {
      const int below = __popcll(peers & lt);
      wr = s_wcnt[w][d] + below;
      if (below == __popcll(peers) - 1) s_wcnt[w][d] = wr + 1;
    }
    key[r] = k;
    val[r] = v;
    rnk[r] = wr;
  }
  __syncthreads();
  // per digit: exclusive prefix over the 4 waves and the block total
  int total = 0;
  if (tid < B) {
#pragma unroll
    for (int q = 0; q < OS_WAVES; q++) {
      const int c = s_wcnt[q][tid];
      s_wcnt[q][tid] = total;
      total += c;
    }
  }
  int ntot;
  const int incl = block_scan_os(tid < B ? total : 0, ntot);
  if (tid < B) {
    s_lbase[tid] = incl - total;
    // publish this partition's count, then look back for the exclusive prefix
    const int64_t me = (int64_t)part * B + tid;
    uint32_t excl = 0;
    if (part == 0) {
      st_status(&status[me], ST_INC | (uint32_t)total);
    } else {
      st_status(&status[me], ST_AGG | (uint32_t)total);
      int p = part - 1;
      int spins = 0;
      while (p >= 0) {
        const uint32_t s = ld_status(&status[(int64_t)p * B + tid]);
        const uint32_t f = s & ~ST_CNT;
        if (f == 0) {
          if (++spins > SPIN_LIMIT) {
            atomicOr(err, 1);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          continue;
        }
        excl += s & ST_CNT;
        if (f == ST_INC) break;
        p--;
      }
      st_status(&status[me], ST_INC | (excl + (uint32_t)total));
    }
    s_gbase[tid] = digit_base[tid] + excl;
  }
  if (tid == 0) s_nvalid = ntot;
  __syncthreads();
  // reorder in LDS by digit (stable)
#pragma unroll
  for (int r = 0; r < OS_ITEMS; r++) {
    if (rnk[r] >= 0) {
      const uint32_t d = (key[r] >> shift) & (B - 1);
      const int pos = s_lbase[d] + s_wcnt[w][d] + rnk[r];
      s_key[pos] = key[r];
      s_val[pos] = val[r];
    }
  }
  __syncthreads();
  const int nv = s_nvalid;
  for (int i = tid; i < nv; i += OS_THREADS) {
    const uint32_t k = s_key[i];
    const uint32_t d = (k >> shift) & (B - 1);
    const uint32_t dst = s_gbase[d] + (uint32_t)(i - s_lbase[d]);
    if (dst >= (uint32_t)n) continue;  // only after a look-back bound was hit (err is set)
    if (kout) kout[dst] = k;
    vout[dst] = s_val[i];
  }
}

// ---------------------------------------------------------------- depth-ordered pair offsets

__global__ void __launch_bounds__(SCAN_T) k_dcount_reduce(const SortCtl *__restrict__ ctl,
                                                          int n_max,
                                                          const uint32_t *__restrict__ dval,
                                                          const int32_t *__restrict__ offsets,
                                                          int32_t *__restrict__ bsum) {
  const int m = clamp_n(ctl->m, n_max);
  const int base = blockIdx.x * SCAN_TILE;
  int v = 0;
  for (int j = 0; j < SCAN_I; j++) {
    const int r = base + j * SCAN_T + threadIdx.x;
    if (r < m) {
      const int g = (int)dval[r];
      v += offsets[g + 1] - offsets[g];
    }
  }
  int tot;
  block_scan256(v, tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

// doff[r] = pairs of the splats ranked before r. Each block sums the (few) block
// sums before it itself, so the scan needs no third kernel; the block after the
// last writes the grand total.
__global__ void __launch_bounds__(SCAN_T) k_dcount_apply(SortCtl *__restrict__ ctl, int n_max,
                                                         const uint32_t *__restrict__ dval,
                                                         const int32_t *__restrict__ offsets,
                                                         const int32_t *__restrict__ bsum,
                                                         int32_t *__restrict__ doff) {
  const int m = clamp_n(ctl->m, n_max);
  const int nb = (m + SCAN_TILE - 1) / SCAN_TILE;
  if ((int)blockIdx.x > nb) return;
  int pre = 0;
  for (int b = threadIdx.x; b < (int)blockIdx.x; b += SCAN_T) pre += bsum[b];
  int block_base;
  block_scan256(pre, block_base);
  if ((int)blockIdx.x == nb) {
    if (threadIdx.x == 0) {
      doff[m] = block_base;
      ctl->npairs = block_base;
    }
    return;
  }
  const int base = blockIdx.x * SCAN_TILE;
  int x[SCAN_I];
  int v = 0;
#pragma unroll
  for (int j = 0; j < SCAN_I; j++) {
    const int r = base + threadIdx.x * SCAN_I + j;
    x[j] = 0;
    if (r < m) {
      const int g = (int)dval[r];
      x[j] = offsets[g + 1] - offsets[g];
    }
    v += x[j];
  }
  int t2;
  const int incl = block_scan256(v, t2);
  int run = block_base + incl - v;
#pragma unroll
  for (int j = 0; j < SCAN_I; j++) {
    const int r = base + threadIdx.x * SCAN_I + j;
    if (r < m) doff[r] = run;
    run += x[j];
  }
}

// ---------------------------------------------------------------- emission in depth order

__global__ void __launch_bounds__(256) k_emit_depth_order(
    const SortCtl *__restrict__ ctl, int n_max, const uint32_t *__restrict__ dval,
    const int32_t *__restrict__ doff, const Splat *__restrict__ splats, int W, int H, int tiles_x,
    int tiles_y, uint32_t *__restrict__ tile_out, uint32_t *__restrict__ id_out,
    int32_t *__restrict__ tile_counts) {
  __shared__ int hist[HIST_TILES_LDS];
  const int ntiles = tiles_x * tiles_y;
  const bool lds_hist = ntiles <= HIST_TILES_LDS;
  if (lds_hist)
    for (int i = threadIdx.x; i < ntiles; i += 256) hist[i] = 0;
  __syncthreads();
  const int m = clamp_n(ctl->m, n_max);
  for (int r = blockIdx.x * 256 + threadIdx.x; r < m; r += gridDim.x * 256) {
    const int g = (int)dval[r];
    const RowSpans rs = spans_setup(splats[g], tiles_y);
    if (!rs.ok) continue;
    int pos = doff[r];
    for (int ty = rs.ty_a; ty < rs.ty_b; ty++) {
      int a, b;
      row_span(rs, ty, W, H, tiles_x, a, b);
      for (int tx = a; tx < b; tx++) {
        const int t = ty * tiles_x + tx;
        tile_out[pos] = (uint32_t)t;
        id_out[pos] = (uint32_t)g;
        pos++;
        if (lds_hist)
          atomicAdd(&hist[t], 1);
        else
          atomicAdd(&tile_counts[t], 1);
      }
    }
  }
  __syncthreads();
  if (lds_hist)
    for (int i = threadIdx.x; i < ntiles; i += 256)
      if (hist[i]) atomicAdd(&tile_counts[i], hist[i]);
}

// Tile ranges (exclusive prefix of the per-tile counts) and the digit offsets of
// the two tile passes: the low digit groups tiles by t mod 2^b0, the high digit
// by t >> b0, whose offset is the start of tile d << b0.
__global__ void __launch_bounds__(1024) k_tile_bases(SortCtl *__restrict__ ctl,
                                                     const int32_t *__restrict__ tile_counts,
                                                     int ntiles, int b0,
                                                     int32_t *__restrict__ ranges) {
  __shared__ int wsum[16];
  __shared__ int carry;
  __shared__ uint32_t lo_hist[256];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry = 0;
  if (threadIdx.x < 256) lo_hist[threadIdx.x] = 0;
  __syncthreads();
  const uint32_t mask0 = (1u << b0) - 1u;
  for (int c0 = 0; c0 < ntiles; c0 += 1024) {
    const int t = c0 + threadIdx.x;
    const int x = t < ntiles ? tile_counts[t] : 0;
    if (x) atomicAdd(&lo_hist[t & mask0], (uint32_t)x);
    int v = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(v, d, 64);
      if (lane >= d) v += o;
    }
    if (lane == 63) wsum[wid] = v;
    __syncthreads();
    int base = carry, tot = 0;
    for (int q = 0; q < 16; q++) {
      base += (q < wid) ? wsum[q] : 0;
      tot += wsum[q];
    }
    if (t < ntiles) {
      ranges[2 * t] = base + v - x;
      ranges[2 * t + 1] = base + v;
      if ((t & mask0) == 0) ctl->tbase[1][t >> b0] = (uint32_t)(base + v - x);
    }
    __syncthreads();
    if (threadIdx.x == 0) carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (uint32_t d = 0; d <= mask0; d++) {
      ctl->tbase[0][d] = run;
      run += lo_hist[d];
    }
  }
}

__global__ void __launch_bounds__(256) k_sorted_keys(const SortCtl *__restrict__ ctl, int cap,
                                                     const uint32_t *__restrict__ tiles,
                                                     const uint32_t *__restrict__ ids,
                                                     const Splat *__restrict__ splats,
                                                     uint64_t *__restrict__ out) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= clamp_n(ctl->npairs, cap)) return;
  out[k] = ((uint64_t)tiles[k] << 32) | (uint64_t)__float_as_uint(splats[ids[k]].p2.z);
}

// ---------------------------------------------------------------- workspace layout

int64_t parts_of(int64_t n) { return (n + OS_PART - 1) / OS_PART; }

struct SortWs {
  SortCtl *ctl;
  int32_t *tile_counts;
  uint32_t *dk[2], *dv[2];  // n each
  int32_t *doff;            // n + 1
  int32_t *bsum;            // block sums of the depth-order scan
  uint32_t *tk[2], *tv[2];  // capacity each
  uint32_t *status;         // look-back words: 4 depth passes, then 2 tile passes
  int64_t pd, pt;           // status words per depth pass / per tile pass
  size_t bytes;
};

SortWs carve(char *base, int n, int64_t cap, int ntiles) {
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    char *r = base + off;
    off += (size_t)((bytes + 255) / 256) * 256;
    return r;
  };
  SortWs w;
  w.ctl = (SortCtl *)take(sizeof(SortCtl));
  w.tile_counts = (int32_t *)take(4 * (int64_t)(ntiles + 1));
  for (int i = 0; i < 2; i++) w.dk[i] = (uint32_t *)take(4 * ((int64_t)n + 2));
  for (int i = 0; i < 2; i++) w.dv[i] = (uint32_t *)take(4 * ((int64_t)n + 2));
  w.doff = (int32_t *)take(4 * ((int64_t)n + 2));
  w.bsum = (int32_t *)take(4 * ((int64_t)n / SCAN_TILE + 4));
  for (int i = 0; i < 2; i++) w.tk[i] = (uint32_t *)take(4 * (cap + 2));
  for (int i = 0; i < 2; i++) w.tv[i] = (uint32_t *)take(4 * (cap + 2));
  w.pd = (parts_of(n) + 1) * 256;
  w.pt = (parts_of(cap) + 1) * 256;
  w.status = (uint32_t *)take(4 * (4 * w.pd + 2 * w.pt));
  w.bytes = off;
  return w;
}

}  // namespace

size_t gs_sort_ws_bytes(int n, int64_t cap, int ntiles) {
  return carve(nullptr, n, cap, ntiles).bytes + 256;
}

hipError_t gs_launch_sort(int n, const float *splats, const int32_t *offsets, int64_t cap,
                          const CamK &cam, uint64_t *sorted_keys, int32_t *sorted_ids,
                          int32_t *ranges, void *ws, hipStream_t st) {
  const Splat *sp = reinterpret_cast<const Splat *>(splats);
  const int ntiles = cam.tiles_x * cam.tiles_y;
  SortWs w = carve(reinterpret_cast<char *>(ws), n, cap, ntiles);
  SortCtl *ctl = w.ctl;
  char *cb = reinterpret_cast<char *>(ctl);
  auto dbase = [&](int p) { return reinterpret_cast<uint32_t *>(cb + offsetof(SortCtl, dbase)) + 256 * p; };
  auto tbase = [&](int p) { return reinterpret_cast<uint32_t *>(cb + offsetof(SortCtl, tbase)) + 256 * p; };
  auto ticket = [&](int p) { return reinterpret_cast<int32_t *>(cb + offsetof(SortCtl, tickets)) + p; };
  int32_t *err = reinterpret_cast<int32_t *>(cb + offsetof(SortCtl, err));
  const int32_t *m_dev = reinterpret_cast<const int32_t *>(cb + offsetof(SortCtl, m));
  const int32_t *i_dev = reinterpret_cast<const int32_t *>(cb + offsetof(SortCtl, npairs));
  const int capi = (int)cap;
  const int64_t nstatus = 4 * w.pd + 2 * w.pt;

  hipLaunchKernelGGL(k_sort_init, dim3(1), dim3(1024), 0, st, ctl, w.tile_counts, ntiles);
  const int hist_blocks = max(1, min(1024, gs_div_up(n > 0 ? n : 1, 256)));
  hipLaunchKernelGGL(k_depth_hist, dim3(hist_blocks), dim3(256), 0, st, n, sp, offsets, cap, ctl,
                     w.status, nstatus);
  hipLaunchKernelGGL(k_depth_bases, dim3(1), dim3(256), 0, st, ctl);
  // depth sort of the visible splats: 4 passes of 8 bits
  const int npd = (int)(parts_of(n) > 1 ? parts_of(n) : 1);
  hipLaunchKernelGGL((k_onesweep<8, true>), dim3(npd), dim3(OS_THREADS), 0, st, nullptr, nullptr,
                     w.dk[1], w.dv[1], nullptr, n, sp, offsets, cap, 0, dbase(0), w.status,
                     ticket(0), err);
  int cur = 1;
  for (int pass = 1; pass < 4; pass++) {
    hipLaunchKernelGGL((k_onesweep<8, false>), dim3(npd), dim3(OS_THREADS), 0, st, w.dk[cur],
                       w.dv[cur], w.dk[cur ^ 1], w.dv[cur ^ 1], m_dev, n, nullptr, nullptr, cap,
                       8 * pass, dbase(pass), w.status + pass * w.pd, ticket(pass), err);
    cur ^= 1;
  }
  const uint32_t *dval = w.dv[cur];
  // pair offsets in depth order
  const int nb = gs_div_up(n > 0 ? n : 1, SCAN_TILE);
  hipLaunchKernelGGL(k_dcount_reduce, dim3(nb), dim3(SCAN_T), 0, st, ctl, n, dval, offsets, w.bsum);
  hipLaunchKernelGGL(k_dcount_apply, dim3(nb + 1), dim3(SCAN_T), 0, st, ctl, n, dval, offsets,
                     w.bsum, w.doff);
  // emit the pairs in depth order, with the per-tile histogram
  const int eblocks = max(1, min(2048, gs_div_up(n > 0 ? n : 1, 256)));
  hipLaunchKernelGGL(k_emit_depth_order, dim3(eblocks), dim3(256), 0, st, ctl, n, dval, w.doff, sp,
                     cam.width, cam.height, cam.tiles_x, cam.tiles_y, w.tk[0], w.tv[0],
                     w.tile_counts);
  // stable sort by tile id: the low 8 bits, then (for more than 256 tiles) the rest
  int tbits = 1;
  while ((1 << tbits) < ntiles) tbits++;
  const int b0 = 8;
  hipLaunchKernelGGL(k_tile_bases, dim3(1), dim3(1024), 0, st, ctl, w.tile_counts, ntiles, b0,
                     ranges);
  const int npt = (int)(parts_of(cap) > 1 ? parts_of(cap) : 1);
  uint32_t *status_t0 = w.status + 4 * w.pd, *status_t1 = status_t0 + w.pt;
  uint32_t *final_tiles = sorted_keys ? w.tk[0] : nullptr;
  uint32_t *ids_out = reinterpret_cast<uint32_t *>(sorted_ids);
  if (tbits <= 8) {
    hipLaunchKernelGGL((k_onesweep<8, false>), dim3(npt), dim3(OS_THREADS), 0, st, w.tk[0],
                       w.tv[0], final_tiles ? w.tk[1] : nullptr, ids_out, i_dev, capi, nullptr,
                       nullptr, cap, 0, tbase(0), status_t0, ticket(4), err);
    final_tiles = w.tk[1];
  } else {
    hipLaunchKernelGGL((k_onesweep<8, false>), dim3(npt), dim3(OS_THREADS), 0, st, w.tk[0],
                       w.tv[0], w.tk[1], w.tv[1], i_dev, capi, nullptr, nullptr, cap, 0, tbase(0),
                       status_t0, ticket(4), err);
    hipLaunchKernelGGL((k_onesweep<8, false>), dim3(npt), dim3(OS_THREADS), 0, st, w.tk[1],
                       w.tv[1], final_tiles, ids_out, i_dev, capi, nullptr, nullptr, cap, b0,
                       tbase(1), status_t1, ticket(5), err);
  }
  if (sorted_keys)
    hipLaunchKernelGGL(k_sorted_keys, dim3(gs_div_up(cap > 0 ? cap : 1, 256)), dim3(256), 0, st,
                       ctl, capi, final_tiles, reinterpret_cast<const uint32_t *>(sorted_ids), sp,
                       sorted_keys);
  return hipGetLastError();
}
