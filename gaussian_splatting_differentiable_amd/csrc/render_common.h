// Shared by the schedule, forward and backward kernels: the work-item encoding,
// the forward-state layout, and the sub-tile geometry.
//
// Scheduling ("Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on
// GPUs", section 4): a persistent kernel whose workers take items from a queue
// advanced by one atomic add (4.1); tiles in longest-processing-time order by
// their pair count N_t (4.1); the heaviest h tiles split into k contiguous
// depth chunks (4.2) chosen per frame by the Eq. 6 cost model (4.4).
// Here a worker is one wavefront and an item is one 8x8 quarter of a tile (or
// of a chunk), so the queue holds 4 items per tile or chunk.
#pragma once
#include "gs_common.h"

#define GS_HK_MAX 4096        // maximum h*k (chunks of chunked tiles per frame)
#define GS_SLOTS_MAX 2048     // maximum h (k >= 2)
#define GS_SPIN_LIMIT (1 << 24)

// Item: kind (2 bits) | quad (2 bits) | chunk p (4 bits) | index (24 bits).
enum ItemKind { ITEM_PLAIN = 0, ITEM_PASS_A = 1, ITEM_PASS_B = 2 };

// Queues: one global queue for the chunk items (all pass A, then all pass B),
// then one queue per XCD group for the other quarters. Tiles are grouped into
// GS_GROUPS vertical strips of the image, so neighbouring tiles (which share
// splats) and the four quarters of one tile are served by the workers of one
// XCD and its L2; workers that empty their group's queue take from the others.
#define GS_GROUPS 8
#define GS_HEAD_STRIDE 16  // ints between two queue heads (one 64-byte line)

__host__ __device__ __forceinline__ int make_item(int kind, int quad, int p, int idx) {
  return (kind << 30) | (quad << 28) | (p << 24) | idx;
}
__device__ __forceinline__ int item_kind(int it) { return (it >> 30) & 3; }
__device__ __forceinline__ int item_quad(int it) { return (it >> 28) & 3; }
__device__ __forceinline__ int item_chunk(int it) { return (it >> 24) & 15; }
__device__ __forceinline__ int item_index(int it) { return it & 0xFFFFFF; }

struct PlanHdr {
  int32_t h, k;                 // chunked tiles and chunks per tile
  int32_t nA;                   // pass-A items = pass-B items = 4 h k
  int32_t nplain;               // quarters of the other tiles = 4 (T - h)
  int32_t err;                  // a bounded wait gave up (never expected)
  int32_t ntiles;
  int32_t qoff[GS_GROUPS + 1];  // group queues within the plain items
};

// Byte layout of fwd_state for T tiles.
struct FwdLayout {
  size_t hdr, heads, sub_last, order, counts, items, sat, doneA, doneB, chunk_last, PA, CB, TB,
      LB, total;
};

__host__ __device__ inline FwdLayout fwd_layout(int T) {
  FwdLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t r = off;
    off += (bytes + 255) / 256 * 256;
    return r;
  };
  const size_t cq = (size_t)GS_HK_MAX * 4;  // chunk items (per quad)
  L.hdr = take(sizeof(PlanHdr));
  L.heads = take(4 * (size_t)2 * (GS_GROUPS + 1) * GS_HEAD_STRIDE);
  L.sub_last = take(4 * (size_t)T * 4);
  L.order = take(4 * (size_t)T);
  L.counts = take(4 * (size_t)T);
  L.items = take(4 * ((size_t)T * 4 + 2 * cq));
  L.sat = take(4 * (size_t)GS_SLOTS_MAX * 4);
  L.doneA = take(4 * cq);
  L.doneB = take(4 * (size_t)GS_SLOTS_MAX * 4);
  L.chunk_last = take(4 * cq);
  L.PA = take(4 * cq * 64);
  L.CB = take(4 * cq * 64 * 3);
  L.TB = take(4 * cq * 64);
  L.LB = take(4 * cq * 64);
  L.total = off;
  return L;
}

struct FwdState {
  PlanHdr *hdr;
  int32_t *heads;  // [pass 0 fwd / 1 bwd][queue 0 chunks, 1.. groups] * GS_HEAD_STRIDE
  int32_t *sub_last, *order, *counts, *items, *sat, *doneA, *doneB, *chunk_last;
  float *PA, *CB, *TB;
  int32_t *LB;
};

__host__ __device__ inline FwdState fwd_state_at(void *base, int T) {
  const FwdLayout L = fwd_layout(T);
  char *b = reinterpret_cast<char *>(base);
  FwdState s;
  s.hdr = reinterpret_cast<PlanHdr *>(b + L.hdr);
  s.heads = reinterpret_cast<int32_t *>(b + L.heads);
  s.sub_last = reinterpret_cast<int32_t *>(b + L.sub_last);
  s.order = reinterpret_cast<int32_t *>(b + L.order);
  s.counts = reinterpret_cast<int32_t *>(b + L.counts);
  s.items = reinterpret_cast<int32_t *>(b + L.items);
  s.sat = reinterpret_cast<int32_t *>(b + L.sat);
  s.doneA = reinterpret_cast<int32_t *>(b + L.doneA);
  s.doneB = reinterpret_cast<int32_t *>(b + L.doneB);
  s.chunk_last = reinterpret_cast<int32_t *>(b + L.chunk_last);
  s.PA = reinterpret_cast<float *>(b + L.PA);
  s.CB = reinterpret_cast<float *>(b + L.CB);
  s.TB = reinterpret_cast<float *>(b + L.TB);
  s.LB = reinterpret_cast<int32_t *>(b + L.LB);
  return s;
}

__host__ __device__ __forceinline__ int32_t *queue_head(const FwdState &fs, int pass, int q) {
  return fs.heads + (pass * (GS_GROUPS + 1) + q) * GS_HEAD_STRIDE;
}

// Group (XCD strip) of a tile: vertical strips of the tile grid.
__host__ __device__ __forceinline__ int tile_group(int tile, int tiles_x) {
  return (tile % tiles_x) * GS_GROUPS / tiles_x;
}

// Index of (slot s, chunk p, quad q) among the chunk items.
__device__ __forceinline__ int chunk_index(int s, int p, int q, int k) { return (s * k + p) * 4 + q; }

// Chunk p of k over [start, end): equal contiguous pieces of ceil(N/k).
__device__ __forceinline__ void chunk_range(int start, int end, int p, int k, int &cs, int &ce) {
  const int N = end - start;
  const int csize = (N + k - 1) / k;
  cs = min(end, start + p * csize);
  ce = min(end, cs + csize);
}

struct SubTile {
  int tile, quad, x0, y0;
  float hx0, hx1, hy0, hy1;  // sample hull of the 8x8 quarter
  bool empty;
};

__device__ __forceinline__ SubTile subtile_of(int tile, int quad, const CamK &cam) {
  SubTile st;
  st.tile = tile;
  st.quad = quad;
  const int tx = tile % cam.tiles_x, ty = tile / cam.tiles_x;
  st.x0 = tx * 16 + (quad & 1) * 8;
  st.y0 = ty * 16 + (quad >> 1) * 8;
  st.empty = st.x0 >= cam.width || st.y0 >= cam.height;
  st.hx0 = (float)st.x0 + 0.5f;
  st.hx1 = (float)min(st.x0 + 7, cam.width - 1) + 0.5f;
  st.hy0 = (float)st.y0 + 0.5f;
  st.hy1 = (float)min(st.y0 + 7, cam.height - 1) + 0.5f;
  return st;
}

// Wave-uniform queue pop: one lane advances the head, every lane gets the ticket.
__device__ __forceinline__ int queue_pop(int32_t *head) {
  int t = 0;
  if (__lane_id() == 0) t = atomicAdd(head, 1);
  return __shfl(t, 0, GS_WAVE);
}

// Next item of a persistent worker: the chunk queue [0, nchunk) first, then its
// own group's queue, then the other groups'. Returns the index into items[]
// (relative to `base`), or -1 when everything is taken. `g` is the group
// currently being drained (starts at the worker's XCD).
__device__ __forceinline__ int next_item(const FwdState &fs, int pass, int nchunk, int &g,
                                         int &tried, bool &chunks_done) {
  if (!chunks_done) {
    const int t = queue_pop(queue_head(fs, pass, 0));
    if (t < nchunk) return t;
    chunks_done = true;
  }
  while (tried < GS_GROUPS) {
    const int q0 = fs.hdr->qoff[g], q1 = fs.hdr->qoff[g + 1];
    if (q1 > q0) {
      const int t = queue_pop(queue_head(fs, pass, 1 + g));
      if (q0 + t < q1) return nchunk + q0 + t;
    }
    g = (g + 1) % GS_GROUPS;
    tried++;
  }
  return -1;
}

// Spin on a flag with relaxed loads (no cache invalidation per probe); the
// caller issues one acquire fence after it succeeds.
__device__ __forceinline__ int ld_flag(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(int32_t *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
