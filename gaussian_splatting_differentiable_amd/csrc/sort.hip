// Pair ordering for the tile rasterizer: the counting half of gs_bin_tiles and
// all of gs_sort_keys.
//
// "What the 3DGS Literature Left on the Table", Step 1 (d), Figure 5: filter the
// visible splats, sort them once front to back by their 32-bit depth, emit the
// tile keys in that depth order, then run a narrow stable sort over the tile ids.
// The result is ordered by (tile, depth, splat id): the depth sort is stable over
// an id-ordered input and the tile sort is stable.
//
// gs_bin_tiles counts every splat's pairs with the canonical row spans and, in
// the same pass over the splat records, leaves in the workspace what the sort
// needs: each splat's 32-bit depth key (or "no pairs"), the histograms of the
// two low 9-bit depth digits, the range of the keys' exponent field and the
// per-tile pair counts (LDS histograms per workgroup). It also clears the
// look-back words of every radix pass of the frame.
//
// gs_sort_keys then runs:
//   - three onesweep LSD passes of 9 bits over the visible splats' depth keys
//     less the smallest exponent (key - (emin << 23): the depths are positive,
//     so the order is kept, and 27 bits hold every key when the exponents span
//     fewer than 16 values), and a fourth over bits 27-31 that runs only when
//     they span more (6144-key partitions). Their values are 64-bit: the splat
//     id, and above it the splat's pair count, read by the first pass in id
//     order, so the last pass writes the counts in depth order from its own
//     values;
//   - an exclusive scan of those counts: the pair offsets in depth order, and
//     for every 16384-pair partition the splat its first pair belongs to;
//   - the first tile pass (low 8 bits of the tile id) with the emission fused
//     in: a partition generates its own pairs into LDS from the splats that
//     cover it, one record per tile row, so the depth-ordered pair list is
//     never written to memory;
//   - the second tile pass (the high bits), writing the sorted ids.
//
// A onesweep pass: a workgroup takes a partition by atomic ticket, ranks its
// keys stably (per-wave ballot match on the digit bits), publishes its digit
// counts and looks back over earlier partitions for its global offsets
// (decoupled look-back: a partition only waits for partitions with a lower
// ticket, which are already running, and the wait is bounded). Keys are
// reordered in LDS so that global writes are contiguous runs per digit.
//
// This TU includes the canonical binning code: compile with -ffp-contract=off.
#include <stddef.h>

#include <type_traits>

#include "bin_spans.h"
#include "sched_body.h"

namespace {

constexpr uint32_t ST_AGG = 1u << 30, ST_INC = 2u << 30, ST_CNT = (1u << 30) - 1;
constexpr int SPIN_LIMIT = 1 << 22;
// The counting kernel keeps its workgroup's tile-count difference array in LDS
// up to this many words (144 KB: a batch of views has several images' tiles);
// beyond it, or if the device refuses that much LDS, it adds to the global
// array directly, which costs far more in atomics.
constexpr int HIST_TILES_LDS = 36864;
constexpr int SCAN_T = 256, SCAN_I = 4, SCAN_TILE = SCAN_T * SCAN_I;
constexpr uint32_t NO_DEPTH = 0xFFFFFFFFu;  // depth key of a splat without pairs (a NaN pattern)
constexpr int BIN_T = 512, BIN_BLOCKS_MAX = 1024, BIN_TILE = 2048;
constexpr uint32_t WS_MAGIC = 0x47534254u;  // a binning pass's state is present

// partitions: depth passes and tile passes
constexpr int DS_THREADS = 1024, DS_ITEMS = 6, DS_PART = DS_THREADS * DS_ITEMS;
constexpr int TS_THREADS = 1024, TS_ITEMS = 16, TS_PART = TS_THREADS * TS_ITEMS;

// Per-frame control block at the start of the workspace.
struct SortCtl {
  int32_t m;               // visible splats (with at least one pair)
  int32_t npairs;          // pairs of this frame (0 after an overflow)
  int32_t err;             // a look-back wait hit its bound (never expected)
  int32_t overflow;        // the frame's pairs exceed the capacity, or the frame failed
  // Tag of the binning pass that filled this workspace: gs_sort_keys checks it
  // against its own arguments and clears it, so a sort without a matching
  // binning pass of its own is reported instead of reading stale state.
  uint32_t magic;
  int32_t tag_n, tag_tiles_x, tag_tiles_y;
  int64_t tag_cap;
  int32_t tickets[8];      // partition tickets, one per radix pass
  // Depth keys are sorted as key - (emin << 23), which keeps their order (the
  // depths are positive): 9-bit digits at bits 0, 9 and 18, and bits 27-31 in
  // a fourth pass only when the keys' exponent field spans 16 values or more.
  uint32_t dhist[2][512];  // digit histograms 0 and 1 (binning pass)
  // digit 2, by the first depth pass: eight copies (workgroup index mod 8), so
  // that its workgroups' additions spread over eight times as many addresses
  uint32_t dhist2[8][512];
  uint32_t dhist3[32];     // bits 27-31 (first depth pass, wide frames only)
  int32_t emin, emax;      // the visible keys' exponent field range
  int32_t wide;            // the fourth depth pass runs
  uint32_t tbase[2][256];  // tile digit exclusive offsets
};

__device__ __forceinline__ int clamp_n(int v, int hi) { return v < 0 ? 0 : (v < hi ? v : hi); }

__device__ __forceinline__ uint32_t ld_status(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_status(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive scan over a block of NT threads; total of the block in `total`.
template <int NT, typename T = int>
__device__ __forceinline__ T block_scan(T v, T &total) {
  constexpr int NWV = NT / 64;
  __shared__ T wsum[NWV];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  if (lane == 63) wsum[wid] = v;
  __syncthreads();
  T base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NWV; w++) {
    base += (w < wid) ? wsum[w] : 0;
    tot += wsum[w];
  }
  __syncthreads();
  total = tot;
  return v + base;
}

// ---------------------------------------------------------------- workspace layout

__host__ __device__ inline int64_t parts_of(int64_t n, int part) { return (n + part - 1) / part; }

// Splats per counting block: a multiple of the block size, at most
// BIN_BLOCKS_MAX blocks.
__host__ __device__ inline int bin_chunk(int n) {
  const int per = (int)parts_of(n > 0 ? n : 1, BIN_BLOCKS_MAX);
  return (int)parts_of(per, BIN_T) * BIN_T;
}
__host__ __device__ inline int bin_blocks(int n) { return (int)parts_of(n > 0 ? n : 1, bin_chunk(n)); }

struct SortWs {
  SortCtl *ctl;
  int32_t *tile_counts;     // T
  int32_t *tile_diff;       // tiles_y x (tiles_x + 1): per-row difference array of pair counts
  uint32_t *dkey;           // n: depth key per splat (NO_DEPTH without pairs)
  uint32_t *dk[2];          // n each: depth passes, keys
  uint32_t *dv[2];          // n 64-bit values each: splat id, its pair count above it
  uint32_t *dfinal;         // n: splat ids in depth order (the last depth pass's output)
  int32_t *dcnt;            // n: pair counts in depth order
  int32_t *doff;            // n + 1: pair offsets in depth order
  int32_t *part_first;      // tile partitions: the splat (depth rank) of the first pair
  int32_t *bsum;            // block sums of the depth-order scan
  uint32_t *tk[2], *tv[2];  // capacity each: tile passes
  uint32_t *status;         // look-back words: 4 depth passes, then 2 tile passes
  int32_t *bin_sum;         // pair count of every counting block's chunk
  int64_t pd, pt;           // status words per depth pass / per tile pass
  int64_t nstatus;
  size_t bytes;
};

SortWs carve(char *base, int n, int64_t cap, int tiles_x, int tiles_y) {
  const int ntiles = tiles_x * tiles_y;
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    char *r = base + off;
    off += (size_t)((bytes + 255) / 256) * 256;
    return r;
  };
  SortWs w;
  const int64_t n2 = (int64_t)n + 2;
  w.ctl = (SortCtl *)take(sizeof(SortCtl));
  w.tile_counts = (int32_t *)take(4 * (int64_t)(ntiles + 1));
  w.tile_diff = (int32_t *)take(4 * (int64_t)tiles_y * (tiles_x + 1));
  w.dkey = (uint32_t *)take(4 * n2);
  for (int i = 0; i < 2; i++) w.dk[i] = (uint32_t *)take(4 * n2);
  for (int i = 0; i < 2; i++) w.dv[i] = (uint32_t *)take(8 * n2);  // id | pair count << 32
  w.dfinal = (uint32_t *)take(4 * n2);
  w.dcnt = (int32_t *)take(4 * n2);
  w.doff = (int32_t *)take(4 * n2);
  w.part_first = (int32_t *)take(4 * (parts_of(cap, TS_PART) + 2));
  w.bsum = (int32_t *)take(4 * ((int64_t)n / SCAN_TILE + 4));
  for (int i = 0; i < 2; i++) w.tk[i] = (uint32_t *)take(4 * (cap + 2));
  for (int i = 0; i < 2; i++) w.tv[i] = (uint32_t *)take(4 * (cap + 2));
  w.pd = (parts_of(n, DS_PART) + 1) * 512;
  w.pt = (parts_of(cap, TS_PART) + 1) * 256;
  w.nstatus = 4 * w.pd + 2 * w.pt;
  w.status = (uint32_t *)take(4 * w.nstatus);
  w.bin_sum = (int32_t *)take(4 * ((int64_t)bin_blocks(n) + 1));
  w.bytes = off;
  return w;
}

// ---------------------------------------------------------------- binning side

__global__ void __launch_bounds__(1024) k_bin_init(SortCtl *__restrict__ ctl,
                                                   int32_t *__restrict__ tile_diff, int ndiff,
                                                   int n, int64_t cap, int tiles_x,
                                                   int tiles_y) {
  int32_t *w = reinterpret_cast<int32_t *>(ctl);
  const int nw = (int)(sizeof(SortCtl) / 4);
  for (int i = threadIdx.x; i < nw; i += blockDim.x) w[i] = 0;
  for (int i = threadIdx.x; i < ndiff; i += blockDim.x) tile_diff[i] = 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    ctl->emin = 255;
    ctl->tag_n = n;
    ctl->tag_cap = cap;
    ctl->tag_tiles_x = tiles_x;
    ctl->tag_tiles_y = tiles_y;
    ctl->magic = WS_MAGIC;
  }
}

// Per-splat pair counts (exact spans) and every block's chunk sum, plus the
// depth keys, the depth-digit histograms and the per-row difference array of
// the tile counts (+1 where a row span starts, -1 where it ends: two updates
// per row, however long the span) for the sort; clears the sort's look-back
// words. Block b counts the splats [b chunk, (b + 1) chunk).
__global__ void __launch_bounds__(BIN_T) k_bin_count(
    int n, const Splat *__restrict__ splats, int W, int H, int tiles_x, int tiles_y, int vty,
    int views, int32_t *__restrict__ counts, int chunk, int32_t *__restrict__ bin_sum,
    uint32_t *__restrict__ dkey, SortCtl *__restrict__ ctl, int32_t *__restrict__ tile_diff,
    uint32_t *__restrict__ status, int64_t nstatus, bool lds_hist) {
  __shared__ uint32_t dh[2][512];
  __shared__ int s_emin, s_emax;
  extern __shared__ int th[];  // the difference array, when lds_hist (sized at launch)
  const int stride = tiles_x + 1;
  const int ndiff = tiles_y * stride;
  for (int i = threadIdx.x; i < 1024; i += BIN_T) (&dh[0][0])[i] = 0;
  if (threadIdx.x == 0) {
    s_emin = 255;
    s_emax = 0;
  }
  int emin = 255, emax = 0;
  if (lds_hist)
    for (int i = threadIdx.x; i < ndiff; i += BIN_T) th[i] = 0;
  for (int64_t i = (int64_t)blockIdx.x * BIN_T + threadIdx.x; i < nstatus;
       i += (int64_t)gridDim.x * BIN_T)
    status[i] = 0;
  __syncthreads();
  const int i0 = blockIdx.x * chunk;
  const int i1 = (int)min((int64_t)n, (int64_t)i0 + chunk);
  int csum = 0;
  for (int i = i0 + threadIdx.x; i < i1; i += BIN_T) {
    const Splat s = splats[i];
    const RowSpans r = spans_setup(s, vty, views);
    int cnt = 0;
    if (r.ok) {
      for (int ty = r.ty_a; ty < r.ty_b; ty++) {
        int a, b;
        row_span(r, ty, W, H, tiles_x, a, b);
        if (b > a) {
          int32_t *h = lds_hist ? th : tile_diff;
          atomicAdd(&h[(r.row0 + ty) * stride + a], 1);
          atomicAdd(&h[(r.row0 + ty) * stride + b], -1);
          cnt += b - a;
        }
      }
    }
    counts[i] = cnt;
    csum += cnt;
    uint32_t k = NO_DEPTH;
    if (cnt > 0) {
      k = __float_as_uint(s.p2.z);
      atomicAdd(&dh[0][k & 511u], 1u);
      atomicAdd(&dh[1][(k >> 9) & 511u], 1u);
      const int e = (int)((k >> 23) & 255u);
      emin = min(emin, e);
      emax = max(emax, e);
    }
    dkey[i] = k;
  }
  // the block's exponent range: a wave reduction, then one LDS atomic per wave
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    emin = min(emin, __shfl_xor(emin, o, 64));
    emax = max(emax, __shfl_xor(emax, o, 64));
  }
  if ((threadIdx.x & 63) == 0 && emin <= emax) {
    atomicMin(&s_emin, emin);
    atomicMax(&s_emax, emax);
  }
  int ctot;
  block_scan<BIN_T>(csum, ctot);  // ends with a barrier: the LDS histograms are complete
  if (threadIdx.x == 0) {
    bin_sum[blockIdx.x] = ctot;
    if (s_emin <= s_emax) {
      atomicMin(&ctl->emin, s_emin);
      atomicMax(&ctl->emax, s_emax);
    }
  }
  for (int i = threadIdx.x; i < 1024; i += BIN_T) {
    const uint32_t v = (&dh[0][0])[i];
    if (v) atomicAdd(&ctl->dhist[0][0] + i, v);
  }
  if (lds_hist)
    for (int i = threadIdx.x; i < ndiff; i += BIN_T)
      if (th[i]) atomicAdd(&tile_diff[i], th[i]);
}

// Per-tile pair counts from the binning pass's row difference array: each row
// of it sums to zero (a span adds +1 where it starts and -1 where it ends), so
// the inclusive prefix along a row is the count of each of its tiles. One wave
// per row (row = wave index over the extra blocks); the row's entries are
// loaded before any is scanned, 64 per register.
constexpr int TC_ROW_REGS = 4;  // rows of up to 256 tiles in one load round
__device__ void tile_counts_rows(const int32_t *__restrict__ tile_diff, int tiles_x, int tiles_y,
                                 int32_t *__restrict__ tile_counts, int row0) {
  const int lane = threadIdx.x & 63, ty = row0 + (threadIdx.x >> 6);
  if (ty >= tiles_y) return;
  const int32_t *row = tile_diff + (int64_t)ty * (tiles_x + 1);
  int32_t *out = tile_counts + (int64_t)ty * tiles_x;
  int carry = 0;
  for (int x0 = 0; x0 < tiles_x; x0 += 64 * TC_ROW_REGS) {
    int v[TC_ROW_REGS];
#pragma unroll
    for (int r = 0; r < TC_ROW_REGS; r++) {
      const int x = x0 + 64 * r + lane;
      v[r] = x < tiles_x ? row[x] : 0;
    }
#pragma unroll
    for (int r = 0; r < TC_ROW_REGS; r++) {
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v[r], d, 64);
        if (lane >= d) v[r] += o;
      }
      const int x = x0 + 64 * r + lane;
      if (x < tiles_x) out[x] = carry + v[r];
      carry += __shfl(v[r], 63, 64);
    }
  }
}

// Exclusive prefix of the counts in place (offsets[0, n)), offsets[n] = I and
// the status: block b scans its own chunk, starting from the sum of the chunk
// sums before it. With tile_counts, extra blocks after those write the per-tile
// counts (a wave per tile row).
__global__ void __launch_bounds__(BIN_T) k_bin_offsets(int n, int chunk,
                                                       const int32_t *__restrict__ bin_sum,
                                                       int32_t *__restrict__ offsets,
                                                       int64_t capacity,
                                                       int32_t *__restrict__ status,
                                                       const int32_t *__restrict__ tile_diff,
                                                       int tiles_x, int tiles_y,
                                                       int32_t *__restrict__ tile_counts) {
  const int nrb = tile_counts ? (tiles_y + BIN_T / 64 - 1) / (BIN_T / 64) : 0;
  if ((int)blockIdx.x >= (int)gridDim.x - nrb) {
    tile_counts_rows(tile_diff, tiles_x, tiles_y, tile_counts,
                     ((int)blockIdx.x - ((int)gridDim.x - nrb)) * (BIN_T / 64));
    return;
  }
  int64_t pre = 0;
  for (int b = threadIdx.x; b < (int)blockIdx.x; b += BIN_T) pre += bin_sum[b];
  int64_t base;
  block_scan<BIN_T, int64_t>(pre, base);
  const int i0 = blockIdx.x * chunk;
  const int i1 = (int)min((int64_t)n, (int64_t)i0 + chunk);
  int64_t carry = base;
  for (int t0 = i0; t0 < i1; t0 += BIN_TILE) {
    constexpr int IT = BIN_TILE / BIN_T;
    int x[IT];
    int v = 0;
#pragma unroll
    for (int j = 0; j < IT; j++) {
      const int idx = t0 + threadIdx.x * IT + j;
      x[j] = idx < i1 ? offsets[idx] : 0;
      v += x[j];
    }
    int tot;
    const int incl = block_scan<BIN_T>(v, tot);
    int run = (int)carry + incl - v;
#pragma unroll
    for (int j = 0; j < IT; j++) {
      const int idx = t0 + threadIdx.x * IT + j;
      if (idx < i1) offsets[idx] = run;
      run += x[j];
    }
    carry += tot;
  }
  if ((int)blockIdx.x == (int)gridDim.x - 1 - nrb && threadIdx.x == 0) {
    offsets[n] = (int32_t)min(carry, (int64_t)INT32_MAX);
    *status = carry > capacity ? GS_ERR_CAPACITY : GS_OK;
  }
}

// ---------------------------------------------------------------- sort setup

// ---------------------------------------------------------------- onesweep pass

// Tile counts, ranges and the tile-digit offsets, by one workgroup of 1024
// threads (it runs as an extra workgroup of the first depth pass, which does
// not depend on it).
__device__ void tile_bases_block(SortCtl *__restrict__ ctl, const int32_t *__restrict__ tile_diff,
                                 int32_t *__restrict__ tile_counts, int tiles_x, int tiles_y,
                                 int b0, int32_t *__restrict__ ranges, bool overflow) {
  __shared__ int wsum[16];
  __shared__ int carry;
  __shared__ uint32_t lo_hist[256];
  const int ntiles = tiles_x * tiles_y;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // the frame's sort state for the later passes: visible splats, the overflow
  // flag and whether the depth keys need the fourth pass (an overflowing frame
  // sorts nothing)
  {
    const int v = (threadIdx.x < 512 && !overflow) ? (int)ctl->dhist[0][threadIdx.x] : 0;
    int tot;
    block_scan<1024>(v, tot);
    if (threadIdx.x == 0) {
      ctl->m = tot;
      ctl->overflow = overflow ? 1 : 0;
      ctl->wide = !overflow && tot > 0 && ctl->emax - ctl->emin > 15;
    }
  }
  // per-tile counts: every row of the difference array sums to zero (each span
  // adds +1 and -1 in its own row), so the inclusive prefix of the whole array,
  // taken row-major, is the count of each tile
  const int stride = tiles_x + 1, ndiff = tiles_y * stride;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int c0 = 0; c0 < ndiff; c0 += 1024) {
    const int i = c0 + threadIdx.x;
    const int x = i < ndiff ? tile_diff[i] : 0;
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
    if (i < ndiff) {
      const int ty = i / stride, tx = i - ty * stride;
      if (tx < tiles_x) tile_counts[ty * tiles_x + tx] = base + v;
    }
    __syncthreads();
    if (threadIdx.x == 0) carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) carry = 0;
  if (threadIdx.x < 256) lo_hist[threadIdx.x] = 0;
  __syncthreads();
  const uint32_t mask0 = (1u << b0) - 1u;
  for (int c0 = 0; c0 < ntiles; c0 += 1024) {
    const int t = c0 + threadIdx.x;
    const int x = (t < ntiles && !overflow) ? tile_counts[t] : 0;
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
  // low-digit offsets: every thread takes part in the scan
  const int v = threadIdx.x <= (int)mask0 ? (int)lo_hist[threadIdx.x] : 0;
  int tot;
  const int incl = block_scan<1024>(v, tot);
  if (threadIdx.x <= (int)mask0) ctl->tbase[0][threadIdx.x] = (uint32_t)(incl - v);
}

// SRC_WIDE: the fourth depth pass, which does nothing unless the frame's
// depth keys need it.
enum Src { SRC_KEYS = 0, SRC_DEPTH0 = 1, SRC_EMIT = 2, SRC_WIDE = 3 };

// Inputs of one pass beyond the (key, value) arrays.
struct PassIn {
  const SortCtl *ctl;
  int64_t cap;                 // SRC_DEPTH0: the pair capacity (offsets[n_max] above it: overflow)
  const uint32_t *dkey;        // SRC_DEPTH0
  const int32_t *offsets;      // SRC_DEPTH0 (the pair total) and the last depth pass (counts)
  int32_t *cout;               // last depth pass: pair counts in depth order (or null)
  const uint32_t *dval;        // SRC_EMIT: splat ids in depth order
  const int32_t *doff;         // SRC_EMIT: pair offsets in depth order
  const int32_t *part_first;   // SRC_EMIT
  const Splat *splats;         // SRC_EMIT
  int W, H, tiles_x, tiles_y;  // SRC_EMIT; SRC_DEPTH0's extra workgroup (tiles)
  int vty, views;              // SRC_EMIT: the batch's views
  const int32_t *tile_diff;    // SRC_DEPTH0's extra workgroup: tile counts and ranges
  int32_t *tile_counts, *ranges;
  int b0;
  int32_t *status;             // the frame's device status (bounded waits report here)
  const uint32_t *dhist_in;    // depth passes: this pass's digit histogram (offsets made in-block)
  int dhist_copies;            // ... as this many copies, B apart, to be summed
  uint32_t *wide_kout, *wide_vout;  // third depth pass: its output when the fourth pass runs
  int spin_limit;              // probes before a look-back wait gives up
  // the 5-bit tile pass: the frame's tile schedule, built by its first workgroup
  // from the tile counts (plan_state null: none)
  char *plan_state;
  const int32_t *plan_counts;
  int plan_mode, plan_force_k, plan_force_h, plan_nblocks;
  double plan_lambda, plan_beta, plan_eps;
  int64_t plan_cap;
};

template <int NT, int ITEMS, int BITS, int SRC>
__global__ void __launch_bounds__(NT) k_onesweep(
    const uint32_t *__restrict__ kin, const uint32_t *__restrict__ vin, uint32_t *__restrict__ kout,
    uint32_t *__restrict__ vout, const int32_t *__restrict__ n_dev, int n_max, int shift,
    const uint32_t *__restrict__ digit_base, uint32_t *__restrict__ status,
    int32_t *__restrict__ ticket, int32_t *__restrict__ err, PassIn in) {
  constexpr int B = 1 << BITS;
  constexpr int NWV = NT / 64;
  constexpr int PART = NT * ITEMS;
  // keys and values in one array: the schedule's workgroup (below) takes all of
  // it as its working LDS
  // The depth passes carry 64-bit values: the splat id in the low word and its
  // pair count in the high word (read by the first pass in id order), so that
  // the last one writes the counts in depth order without gathering them.
  constexpr bool DEPTH = NT == DS_THREADS && ITEMS == DS_ITEMS && SRC != SRC_EMIT;
  using VT = typename std::conditional<DEPTH, uint64_t, uint32_t>::type;
  constexpr int VW = sizeof(VT) / 4;
  __shared__ __align__(16) uint32_t s_kv[(1 + VW) * PART];
  uint32_t *const s_key = s_kv;
  VT *const s_val = reinterpret_cast<VT *>(s_kv + PART);
  __shared__ int s_wcnt[NWV][B];
  __shared__ int s_lbase[B];
  __shared__ uint32_t s_gbase[B];
  __shared__ int s_part, s_nvalid;
  __shared__ uint32_t s_mark[SRC == SRC_EMIT ? PART / 32 : 1];
  __shared__ uint32_t s_h2[SRC == SRC_DEPTH0 ? 512 : 1], s_h3[SRC == SRC_DEPTH0 ? 32 : 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // The 5-bit tile pass (frames of 257 to 8192 tiles) builds the frame's tile
  // schedule in its first workgroup, beside the partitions, with the key and
  // value arrays as the schedule's LDS (4 x 8192 words); its partitions are
  // the later workgroups.
  constexpr bool PLANS = SRC == SRC_KEYS && BITS == 5 && NT == 1024 && 2 * PART == 4 * 8192;
  int bid = blockIdx.x;
  if constexpr (PLANS) {
    if (in.plan_state) {
      if (blockIdx.x == 0) {
        const int T = in.tiles_x * in.tiles_y;
        sched_impl::schedule_frame<true>(nullptr, in.plan_counts, T, in.tiles_x, in.plan_mode,
                                         in.plan_force_k, in.plan_force_h, in.plan_lambda,
                                         in.plan_beta, in.plan_eps, in.plan_nblocks,
                                         in.plan_state, nullptr, in.status, in.plan_cap, s_kv);
        return;
      }
      bid -= 1;
    }
  }
  // a depth pass takes its digit offsets (and the first one the number of
  // visible splats) from its digit histogram itself
  uint32_t dbase0 = 0;
  int m0 = 0;
  bool overflow = false;
  if constexpr (SRC == SRC_WIDE) {
    if (!in.ctl->wide) return;  // the frame's keys fit three passes
  }
  if constexpr (SRC == SRC_DEPTH0) {
    static_assert(SRC != SRC_DEPTH0 || NT == 1024, "the tile-bases workgroup has 1024 threads");
    // a frame sorts nothing when its pairs overflowed, an earlier call failed,
    // or the workspace does not hold a binning pass of these sizes
    const SortCtl *c = in.ctl;
    const bool tag_ok = c->magic == WS_MAGIC && c->tag_n == n_max && c->tag_cap == in.cap &&
                        c->tag_tiles_x == in.tiles_x && c->tag_tiles_y == in.tiles_y;
    overflow = !tag_ok || *in.status != GS_OK || (int64_t)in.offsets[n_max] > in.cap;
    if (!tag_ok && blockIdx.x == 0 && tid == 0) report_status(in.status, GS_ERR_WORKSPACE);
    if (in.ranges && blockIdx.x == gridDim.x - 1) {
      tile_bases_block(const_cast<SortCtl *>(in.ctl), in.tile_diff, in.tile_counts, in.tiles_x,
                       in.tiles_y, in.b0, in.ranges, overflow);
      return;
    }
  }
  if (in.dhist_in) {
    int v = 0;
    if (tid < B && !overflow)
      for (int c = 0; c < in.dhist_copies; c++) v += (int)in.dhist_in[c * B + tid];
    const int incl = block_scan<NT>(v, m0);
    dbase0 = (uint32_t)(incl - v);
  }
  {
    // blocks beyond the frame's partitions take no ticket (the launch is sized
    // for the capacity); exactly the first parts_of(n) block indices remain
    const int n_pre = SRC == SRC_DEPTH0 ? n_max : clamp_n(*n_dev, n_max);
    if ((int64_t)bid * PART >= (int64_t)n_pre) return;
  }
  // after the first pass, a frame that has failed (here or in a call beside
  // this one) sorts no further: its earlier passes may have left positions
  // unwritten, and nothing downstream reads them. The status and the ticket
  // are read together; a partition that stops never publishes, and a later one
  // waiting for it stops as soon as it sees the status.
  if (tid == 0) {
    const int st = SRC != SRC_DEPTH0 ? *in.status : GS_OK;
    const int t = atomicAdd(ticket, 1);
    s_part = st != GS_OK ? -1 : t;
  }
  for (int i = tid; i < NWV * B; i += NT) (&s_wcnt[0][0])[i] = 0;
  if constexpr (SRC == SRC_DEPTH0) {
    for (int i = tid; i < 512; i += NT) s_h2[i] = 0;
    if (tid < 32) s_h3[tid] = 0;
  }
  __syncthreads();
  const int part = s_part;
  if (part < 0) return;
  const int n = SRC == SRC_DEPTH0 ? n_max : clamp_n(*n_dev, n_max);
  const int64_t p0 = (int64_t)part * PART;
  if constexpr (SRC == SRC_DEPTH0) {
    if (p0 >= n) return;  // past the last splat
  } else {
    if (p0 >= n) return;  // past the last key: no later partition waits on it
  }
  if constexpr (SRC == SRC_EMIT) {
    // generate this partition's pairs, in depth order: every tile row of a
    // splat that reaches into the partition leaves one record at the position
    // of its first pair here (s_key: that pair's tile, s_val: the splat) and
    // sets that position's bit in s_mark; a pair's key is then its row's first
    // tile plus its distance from the row start. Each thread takes GEN splats
    // at a time with their loads in flight together (one: more splats per
    // thread measured slower, 2 µs per added splat per frame).
    constexpr int GEN = 1;
    for (int i = tid; i < PART / 32; i += NT) s_mark[i] = 0u;
    __syncthreads();
    const int nv = (int)min((int64_t)PART, n - p0);
    const int m = in.ctl->m;
    const int nparts = (int)parts_of(n, PART);
    const int r0 = in.part_first[part];
    const int r1 = part + 1 < nparts ? in.part_first[part + 1] : m - 1;
    for (int rb = r0; rb <= r1; rb += NT * GEN) {
      int gg[GEN];
      int64_t qq[GEN];
      Splat sp[GEN];
#pragma unroll
      for (int u = 0; u < GEN; u++) {
        const int r = rb + u * NT + tid;
        gg[u] = r <= r1 ? (int)in.dval[r] : -1;
        qq[u] = r <= r1 ? in.doff[r] : 0;
      }
#pragma unroll
      for (int u = 0; u < GEN; u++) sp[u] = in.splats[gg[u] >= 0 ? gg[u] : 0];
#pragma unroll
      for (int u = 0; u < GEN; u++) {
        if (gg[u] < 0) continue;
        const int g = gg[u];
        int64_t q = qq[u];
        const RowSpans rs = spans_setup(sp[u], in.vty, in.views);
        if (!rs.ok) continue;
        for (int ty = rs.ty_a; ty < rs.ty_b && q < p0 + nv; ty++) {
          int a, b;
          row_span(rs, ty, in.W, in.H, in.tiles_x, a, b);
          if (b <= a) continue;
          if (q + (b - a) > p0) {
            const int64_t q0 = q > p0 ? q : p0;
            const int sl = (int)(q0 - p0);
            s_key[sl] = (uint32_t)((rs.row0 + ty) * in.tiles_x + a + (int)(q0 - q));
            s_val[sl] = (uint32_t)g;
            atomicOr(&s_mark[sl >> 5], 1u << (sl & 31));
          }
          q += b - a;
        }
      }
    }
    __syncthreads();
  }
  const int emin = SRC == SRC_DEPTH0 ? in.ctl->emin : 0;
  const bool wide = SRC == SRC_DEPTH0 && in.ctl->emax - emin > 15;
  const int64_t base = p0 + (int64_t)w * (ITEMS * 64);
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t key[ITEMS];
  VT val[ITEMS];
  int rnk[ITEMS];
  int hi[SRC == SRC_DEPTH0 ? ITEMS : 1], lo[SRC == SRC_DEPTH0 ? ITEMS : 1];
  // all of this thread's keys are loaded before any is ranked
#pragma unroll
  for (int r = 0; r < ITEMS; r++) {
    const int64_t e = base + r * 64 + lane;
    uint32_t k = NO_DEPTH;
    VT v = 0;
    if constexpr (SRC == SRC_DEPTH0) {
      // the splat's pair count, loaded outside the branch so that every
      // load is in flight at once (a slot past the end reads splat 0's)
      const int64_t ec = e < n ? e : 0;
      hi[r] = in.offsets[ec + 1];
      lo[r] = in.offsets[ec];
    }
    if (e < n) {
      if constexpr (SRC == SRC_DEPTH0) {
        k = in.dkey[e];
        if (k != NO_DEPTH) k -= (uint32_t)emin << 23;  // order kept: positive depths
        v = (VT)e;
      } else if constexpr (SRC == SRC_EMIT) {
        // the nearest row start at or before this pair (position 0 always
        // starts one: the partition's first pair opens a row record)
        const int x = (int)(e - p0);
        int wi = x >> 5;
        uint32_t bits = s_mark[wi] & (0xFFFFFFFFu >> (31 - (x & 31)));
        while (bits == 0u && wi > 0) bits = s_mark[--wi];
        const int st = bits ? wi * 32 + 31 - (int)__clz(bits) : 0;
        k = s_key[st] + (uint32_t)(x - st);
        v = s_val[st];
      } else {
        k = kin[e];
        v = reinterpret_cast<const VT *>(vin)[e];
      }
    }
    key[r] = k;
    val[r] = v;
  }
  if constexpr (SRC == SRC_DEPTH0) {
#pragma unroll
    for (int r = 0; r < ITEMS; r++)
      if (base + r * 64 + lane < n) val[r] |= (VT)(uint32_t)(hi[r] - lo[r]) << 32;
  }
#pragma unroll
  for (int r = 0; r < ITEMS; r++) {
    const int64_t e = base + r * 64 + lane;
    bool valid = e < n;
    if constexpr (SRC == SRC_DEPTH0) valid = valid && key[r] != NO_DEPTH && !overflow;
    const uint32_t k = valid ? key[r] : 0u;
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
    rnk[r] = wr;
    if constexpr (SRC == SRC_DEPTH0) {
      if (valid) {
        atomicAdd(&s_h2[(k >> 18) & 511u], 1u);
        if (wide) atomicAdd(&s_h3[(k >> 27) & 31u], 1u);
      }
    }
  }
  __syncthreads();
  if constexpr (SRC == SRC_DEPTH0) {
    SortCtl *c = const_cast<SortCtl *>(in.ctl);
    uint32_t *h2 = c->dhist2[blockIdx.x & 7];
    for (int i = tid; i < 512; i += NT)
      if (s_h2[i]) atomicAdd(&h2[i], s_h2[i]);
    if (tid < 32 && s_h3[tid]) atomicAdd(&c->dhist3[tid], s_h3[tid]);
  }
  // per digit: exclusive prefix over the waves and the block total
  int total = 0;
  if (tid < B) {
#pragma unroll
    for (int q = 0; q < NWV; q++) {
      const int c = s_wcnt[q][tid];
      s_wcnt[q][tid] = total;
      total += c;
    }
  }
  int ntot;
  const int incl = block_scan<NT>(tid < B ? total : 0, ntot);
  if (tid < B) {
    s_lbase[tid] = incl - total;
    // publish this partition's count, then look back for the exclusive prefix
    const int64_t me = (int64_t)part * B + tid;
    uint32_t excl = 0;
    if (part == 0) {
      st_status(&status[me], ST_INC | (uint32_t)total);
    } else {
      st_status(&status[me], ST_AGG | (uint32_t)total);
      // walk back LBW predecessors per round trip: sum aggregates up to the
      // first inclusive prefix; wait where a predecessor has not published
      constexpr int LBW = 4;
      int p = part - 1;
      int spins = 0;
      while (p >= 0) {
        uint32_t sw[LBW];
#pragma unroll
        for (int j = 0; j < LBW; j++)
          sw[j] = p - j >= 0 ? ld_status(&status[(int64_t)(p - j) * B + tid]) : ST_INC;
        bool done = false;
        int used = 0;
#pragma unroll
        for (int j = 0; j < LBW; j++) {
          if (done || used < j) continue;
          const uint32_t f = sw[j] & ~ST_CNT;
          if (f == 0) continue;
          excl += sw[j] & ST_CNT;
          used = j + 1;
          if (f == ST_INC) done = true;
        }
        if (done) break;
        p -= used;
        if (used < LBW) {  // stopped at an unpublished predecessor
          // a frame that failed meanwhile may leave it unpublished for good
          if (__hip_atomic_load(in.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != GS_OK)
            break;
          if (++spins > in.spin_limit) {
            atomicOr(err, 1);
            report_status(in.status, GS_ERR_TIMEOUT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      st_status(&status[me], ST_INC | (excl + (uint32_t)total));
    }
    s_gbase[tid] = (in.dhist_in ? dbase0 : digit_base[tid]) + excl;
  }
  if (tid == 0) s_nvalid = ntot;
  __syncthreads();
  // reorder in LDS by digit (stable)
#pragma unroll
  for (int r = 0; r < ITEMS; r++) {
    if (rnk[r] >= 0) {
      const uint32_t d = (key[r] >> shift) & (B - 1);
      const int pos = s_lbase[d] + s_wcnt[w][d] + rnk[r];
      s_key[pos] = key[r];
      s_val[pos] = val[r];
    }
  }
  __syncthreads();
  const int nv = s_nvalid;
  const int bound = SRC == SRC_DEPTH0 ? m0 : n;
  // the third depth pass hands its keys to the fourth when that one runs
  const bool handoff = in.wide_vout && in.ctl->wide;
  uint32_t *ko = handoff ? in.wide_kout : kout, *vo = handoff ? in.wide_vout : vout;
  // the last depth pass splits its values: ids to vout, pair counts to cout
  int32_t *co = handoff ? nullptr : in.cout;
  for (int i = tid; i < nv; i += NT) {
    const uint32_t k = s_key[i];
    const uint32_t d = (k >> shift) & (B - 1);
    const uint32_t dst = s_gbase[d] + (uint32_t)(i - s_lbase[d]);
    if (dst >= (uint32_t)bound) continue;  // only after a look-back bound was hit (err is set)
    if (ko) ko[dst] = k;
    const VT v = s_val[i];
    if (co) {
      vo[dst] = (uint32_t)v;
      co[dst] = (int32_t)(v >> 32);
    } else {
      reinterpret_cast<VT *>(vo)[dst] = v;
    }
  }
}

// ---------------------------------------------------------------- depth-ordered pair offsets

// Whether the frame still runs, read once per workgroup (the status word only
// ever leaves GS_OK, so every thread of the block takes the same branch).
__device__ __forceinline__ bool frame_ok(const int32_t *status) {
  __shared__ int ok;
  if (threadIdx.x == 0) ok = *status == GS_OK;
  __syncthreads();
  return ok != 0;
}

__global__ void __launch_bounds__(SCAN_T) k_dscan_reduce(const SortCtl *__restrict__ ctl,
                                                         int n_max,
                                                         const int32_t *__restrict__ dcnt,
                                                         int32_t *__restrict__ bsum,
                                                         const int32_t *__restrict__ status) {
  if (!frame_ok(status)) return;
  const int m = clamp_n(ctl->m, n_max);
  const int base = blockIdx.x * SCAN_TILE;
  int v = 0;
#pragma unroll
  for (int j = 0; j < SCAN_I; j++) {
    const int r = base + j * SCAN_T + threadIdx.x;
    v += r < m ? dcnt[r] : 0;
  }
  int tot;
  block_scan<SCAN_T>(v, tot);
  if (threadIdx.x == 0) bsum[blockIdx.x] = tot;
}

// doff[r] = pairs of the splats ranked before r; for every tile partition k the
// splat whose pairs contain pair k * TS_PART. Each block sums the (few) block
// sums before it itself; the block after the last writes the total.
__global__ void __launch_bounds__(SCAN_T) k_dscan_apply(SortCtl *__restrict__ ctl, int n_max,
                                                        const int32_t *__restrict__ dcnt,
                                                        const int32_t *__restrict__ bsum,
                                                        int32_t *__restrict__ doff,
                                                        int32_t *__restrict__ part_first,
                                                        const int32_t *__restrict__ status) {
  if (!frame_ok(status)) return;
  const int m = clamp_n(ctl->m, n_max);
  const int nb = (m + SCAN_TILE - 1) / SCAN_TILE;
  if ((int)blockIdx.x > nb) return;
  int pre = 0;
  for (int b = threadIdx.x; b < (int)blockIdx.x; b += SCAN_T) pre += bsum[b];
  int block_base;
  block_scan<SCAN_T>(pre, block_base);
  if ((int)blockIdx.x == nb) {
    if (threadIdx.x == 0) {
      doff[m] = block_base;
      ctl->npairs = ctl->overflow ? 0 : block_base;
      ctl->magic = 0u;  // every depth pass has read the tag: this binning pass is used up
    }
    return;
  }
  const int base = blockIdx.x * SCAN_TILE;
  int x[SCAN_I];
  int v = 0;
#pragma unroll
  for (int j = 0; j < SCAN_I; j++) {
    const int r = base + threadIdx.x * SCAN_I + j;
    x[j] = r < m ? dcnt[r] : 0;
    v += x[j];
  }
  int t2;
  const int incl = block_scan<SCAN_T>(v, t2);
  int run = block_base + incl - v;
#pragma unroll
  for (int j = 0; j < SCAN_I; j++) {
    const int r = base + threadIdx.x * SCAN_I + j;
    if (r < m) {
      doff[r] = run;
      // tile partitions whose first pair lies in [run, run + x[j])
      for (int64_t k = ((int64_t)run + TS_PART - 1) / TS_PART; k * TS_PART < (int64_t)run + x[j]; k++)
        part_first[k] = r;
    }
    run += x[j];
  }
}

// Tile ranges (exclusive prefix of the per-tile counts) and the digit offsets of
// the two tile passes: the low digit groups tiles by t mod 2^b0, the high digit
// by t >> b0, whose offset is the start of tile d << b0. An overflowing frame
// gets empty ranges.
__global__ void __launch_bounds__(256) k_sorted_keys(const SortCtl *__restrict__ ctl, int cap,
                                                     const uint32_t *__restrict__ tiles,
                                                     const uint32_t *__restrict__ ids,
                                                     const Splat *__restrict__ splats,
                                                     uint64_t *__restrict__ out,
                                                     const int32_t *__restrict__ status) {
  if (!frame_ok(status)) return;
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= clamp_n(ctl->npairs, cap)) return;
  out[k] = ((uint64_t)tiles[k] << 32) | (uint64_t)__float_as_uint(splats[ids[k]].p2.z);
}

}  // namespace

size_t gs_sort_ws_bytes(int n, int64_t cap, int tiles_x, int tiles_y) {
  return carve(nullptr, n, cap, tiles_x, tiles_y).bytes + 256;
}

// gs_bin_tiles' counting kernels and the prefix sum: offsets[0, n], the
// status (GS_OK, or GS_ERR_CAPACITY when the pairs exceed cap) and, when
// tile_counts is not null, the per-tile pair counts.
hipError_t gs_launch_bin_count(int n, const float *splats, const CamK &cam, int64_t cap,
                               int32_t *offsets, int32_t *tile_counts, int32_t *status, void *ws,
                               hipStream_t st) {
  SortWs w = carve(reinterpret_cast<char *>(ws), n, cap, cam.tiles_x, cam.tiles_y);
  hipLaunchKernelGGL(k_bin_init, dim3(1), dim3(1024), 0, st, w.ctl, w.tile_diff,
                     cam.tiles_y * (cam.tiles_x + 1), n, cap, cam.tiles_x, cam.tiles_y);
  const int chunk = bin_chunk(n), blocks = bin_blocks(n);
  const int ndiff = cam.tiles_y * (cam.tiles_x + 1);
  size_t lds = ndiff <= HIST_TILES_LDS ? 4 * (size_t)ndiff : 0;
  if (lds > 65536 &&
      hipFuncSetAttribute(reinterpret_cast<const void *>(k_bin_count),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    (void)hipGetLastError();
    lds = 0;
  }
  hipLaunchKernelGGL(k_bin_count, dim3(blocks), dim3(BIN_T), lds, st, n,
                     reinterpret_cast<const Splat *>(splats), cam.width, cam.height, cam.tiles_x,
                     cam.tiles_y, cam.vty, cam.views, offsets, chunk, w.bin_sum, w.dkey, w.ctl,
                     w.tile_diff, w.status, w.nstatus, lds > 0);
  const int nrb = tile_counts ? (cam.tiles_y + BIN_T / 64 - 1) / (BIN_T / 64) : 0;
  hipLaunchKernelGGL(k_bin_offsets, dim3(blocks + nrb), dim3(BIN_T), 0, st, n,
                     chunk, w.bin_sum, offsets, cap, status, w.tile_diff, cam.tiles_x,
                     cam.tiles_y, tile_counts);
  return hipGetLastError();
}

int32_t gs_wait_limit(int32_t fallback);

hipError_t gs_launch_schedule(const int32_t *ranges, const int32_t *counts, const CamK &cam,
                              int chunk_mode, int force_k, int force_h, double lambda_,
                              double beta, double eps, int nblocks, void *fwd_state,
                              int64_t *stats, int32_t *status, int64_t cap_pairs,
                              hipStream_t st);

// plan (or null): build the frame's tile schedule into plan->fwd_state as well,
// from the sort's tile counts: inside the 5-bit tile pass when the frame has
// one (257 to 8192 tiles), else in a schedule launch after the sort.
hipError_t gs_launch_sort(int n, const float *splats, const int32_t *offsets, int64_t cap,
                          const CamK &cam, uint64_t *sorted_keys, int32_t *sorted_ids,
                          int32_t *ranges, int32_t *status, void *ws, const SortPlan *plan,
                          hipStream_t st) {
  const Splat *sp = reinterpret_cast<const Splat *>(splats);
  const int ntiles = cam.tiles_x * cam.tiles_y;
  SortWs w = carve(reinterpret_cast<char *>(ws), n, cap, cam.tiles_x, cam.tiles_y);
  SortCtl *ctl = w.ctl;
  char *cb = reinterpret_cast<char *>(ctl);
  auto dhist = [&](int p) { return reinterpret_cast<const uint32_t *>(cb + offsetof(SortCtl, dhist)) + 512 * p; };
  const uint32_t *dhist2 = reinterpret_cast<const uint32_t *>(cb + offsetof(SortCtl, dhist2));
  auto tbase = [&](int p) { return reinterpret_cast<uint32_t *>(cb + offsetof(SortCtl, tbase)) + 256 * p; };
  auto ticket = [&](int p) { return reinterpret_cast<int32_t *>(cb + offsetof(SortCtl, tickets)) + p; };
  int32_t *err = reinterpret_cast<int32_t *>(cb + offsetof(SortCtl, err));
  const int32_t *m_dev = reinterpret_cast<const int32_t *>(cb + offsetof(SortCtl, m));
  const int32_t *i_dev = reinterpret_cast<const int32_t *>(cb + offsetof(SortCtl, npairs));
  const int capi = (int)cap;
  PassIn in{};
  in.ctl = ctl;
  in.status = status;
  in.spin_limit = gs_wait_limit(SPIN_LIMIT);

  // depth sort of the visible splats by key - (emin << 23): three passes of 9
  // bits, and a fourth over bits 27-31 that runs only when the keys' exponents
  // span 16 values or more (the third then hands its output to it); the last
  // pass also writes each splat's pair count in depth order. The first pass
  // has one extra workgroup that turns the binning pass's difference array
  // into tile counts, tile ranges and the tile-digit offsets.
  const int npd = (int)(parts_of(n, DS_PART) > 1 ? parts_of(n, DS_PART) : 1);
  const int b0 = 8;
  {
    PassIn a = in;
    a.dkey = w.dkey;
    a.offsets = offsets;
    a.cap = cap;
    a.tile_diff = w.tile_diff;
    a.tile_counts = w.tile_counts;
    a.ranges = ranges;
    a.tiles_x = cam.tiles_x;
    a.tiles_y = cam.tiles_y;
    a.b0 = b0;
    a.dhist_in = dhist(0);
    a.dhist_copies = 1;
    hipLaunchKernelGGL((k_onesweep<DS_THREADS, DS_ITEMS, 9, SRC_DEPTH0>), dim3(npd + 1),
                       dim3(DS_THREADS), 0, st, nullptr, nullptr, w.dk[1], w.dv[1], nullptr, n, 0,
                       nullptr, w.status, ticket(0), err, a);
  }
  {
    PassIn a = in;
    a.dhist_in = dhist(1);
    a.dhist_copies = 1;
    hipLaunchKernelGGL((k_onesweep<DS_THREADS, DS_ITEMS, 9, SRC_KEYS>), dim3(npd),
                       dim3(DS_THREADS), 0, st, w.dk[1], w.dv[1], w.dk[0], w.dv[0], m_dev, n, 9,
                       nullptr, w.status + w.pd, ticket(1), err, a);
  }
  {
    PassIn a = in;
    a.dhist_in = dhist2;
    a.dhist_copies = 8;
    a.offsets = offsets;
    a.cout = w.dcnt;
    a.wide_kout = w.dk[1];
    a.wide_vout = w.dv[1];
    hipLaunchKernelGGL((k_onesweep<DS_THREADS, DS_ITEMS, 9, SRC_KEYS>), dim3(npd),
                       dim3(DS_THREADS), 0, st, w.dk[0], w.dv[0], nullptr, w.dfinal, m_dev, n, 18,
                       nullptr, w.status + 2 * w.pd, ticket(2), err, a);
  }
  {
    PassIn a = in;
    a.dhist_in = reinterpret_cast<const uint32_t *>(cb + offsetof(SortCtl, dhist3));
    a.dhist_copies = 1;
    a.offsets = offsets;
    a.cout = w.dcnt;
    hipLaunchKernelGGL((k_onesweep<DS_THREADS, DS_ITEMS, 5, SRC_WIDE>), dim3(npd),
                       dim3(DS_THREADS), 0, st, w.dk[1], w.dv[1], nullptr, w.dfinal, m_dev, n, 27,
                       nullptr, w.status + 3 * w.pd, ticket(3), err, a);
  }
  const uint32_t *dval = w.dfinal;
  // pair offsets in depth order and the first splat of every tile partition
  const int nb = gs_div_up(n > 0 ? n : 1, SCAN_TILE);
  hipLaunchKernelGGL(k_dscan_reduce, dim3(nb), dim3(SCAN_T), 0, st, ctl, n, w.dcnt, w.bsum,
                     status);
  hipLaunchKernelGGL(k_dscan_apply, dim3(nb + 1), dim3(SCAN_T), 0, st, ctl, n, w.dcnt, w.bsum,
                     w.doff, w.part_first, status);
  int tbits = 1;
  while ((1 << tbits) < ntiles) tbits++;
  bool planned = false;  // the schedule was built inside a tile pass
  // tile passes: the first generates its partition's pairs itself
  const int npt = (int)(parts_of(cap, TS_PART) > 1 ? parts_of(cap, TS_PART) : 1);
  uint32_t *status_t0 = w.status + 4 * w.pd, *status_t1 = status_t0 + w.pt;
  uint32_t *ids_out = reinterpret_cast<uint32_t *>(sorted_ids);
  PassIn e = in;
  e.dval = dval;
  e.doff = w.doff;
  e.part_first = w.part_first;
  e.splats = sp;
  e.W = cam.width;
  e.H = cam.height;
  e.tiles_x = cam.tiles_x;
  e.tiles_y = cam.tiles_y;
  e.vty = cam.vty;
  e.views = cam.views;
  uint32_t *final_tiles = nullptr;
  if (tbits <= 8) {
    final_tiles = sorted_keys ? w.tk[1] : nullptr;
    hipLaunchKernelGGL((k_onesweep<TS_THREADS, TS_ITEMS, 8, SRC_EMIT>), dim3(npt), dim3(TS_THREADS),
                       0, st, nullptr, nullptr, final_tiles, ids_out, i_dev, capi, 0, tbase(0),
                       status_t0, ticket(4), err, e);
  } else {
    hipLaunchKernelGGL((k_onesweep<TS_THREADS, TS_ITEMS, 8, SRC_EMIT>), dim3(npt), dim3(TS_THREADS),
                       0, st, nullptr, nullptr, w.tk[0], w.tv[0], i_dev, capi, 0, tbase(0),
                       status_t0, ticket(4), err, e);
    final_tiles = sorted_keys ? w.tk[1] : nullptr;
    // the high digit has tbits - 8 significant bits: rank on 5 of them when
    // they fit (up to 8192 tiles), which cuts the ballots and the look-back
    if (tbits - b0 <= 5) {
      PassIn h = in;
      if (plan) {
        h.plan_state = reinterpret_cast<char *>(plan->fwd_state);
        h.plan_counts = w.tile_counts;
        h.tiles_x = cam.tiles_x;
        h.tiles_y = cam.tiles_y;
        h.plan_mode = plan->mode;
        h.plan_force_k = plan->force_k;
        h.plan_force_h = plan->force_h;
        h.plan_nblocks = plan->nblocks;
        h.plan_lambda = plan->lambda_;
        h.plan_beta = plan->beta;
        h.plan_eps = plan->eps;
        h.plan_cap = plan->cap;
        planned = true;
      }
      hipLaunchKernelGGL((k_onesweep<TS_THREADS, TS_ITEMS, 5, SRC_KEYS>), dim3(npt + (plan ? 1 : 0)),
                         dim3(TS_THREADS), 0, st, w.tk[0], w.tv[0], final_tiles, ids_out, i_dev,
                         capi, b0, tbase(1), status_t1, ticket(5), err, h);
    } else
      hipLaunchKernelGGL((k_onesweep<TS_THREADS, TS_ITEMS, 8, SRC_KEYS>), dim3(npt),
                         dim3(TS_THREADS), 0, st, w.tk[0], w.tv[0], final_tiles, ids_out, i_dev,
                         capi, b0, tbase(1), status_t1, ticket(5), err, in);
  }
  if (sorted_keys)
    hipLaunchKernelGGL(k_sorted_keys, dim3(gs_div_up(cap > 0 ? cap : 1, 256)), dim3(256), 0, st,
                       ctl, capi, final_tiles, reinterpret_cast<const uint32_t *>(sorted_ids), sp,
                       sorted_keys, status);
  hipError_t err_launch = hipGetLastError();
  if (err_launch == hipSuccess && plan && !planned)
    err_launch = gs_launch_schedule(nullptr, w.tile_counts, cam, plan->mode, plan->force_k,
                                    plan->force_h, plan->lambda_, plan->beta, plan->eps,
                                    plan->nblocks, plan->fwd_state, nullptr, status, plan->cap, st);
  return err_launch;
}
