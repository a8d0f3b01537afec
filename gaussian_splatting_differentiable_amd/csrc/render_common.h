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
#define GS_SPIN_LIMIT (1 << 20)  // probes of a bounded wait (seconds at the longest back-off)

// Item: kind (2 bits) | quad (2 bits) | chunk p (4 bits) | index (24 bits).
// The forward's items are quarters. The backward's: a whole plain tile
// (ITEM_PLAIN), one quarter of a plain tile (ITEM_QUARTER) or one quarter of
// a chunk (ITEM_PASS_B); for the first two, p = 0 is the whole walk and
// p = i + 1 its piece i between cuts.
enum ItemKind { ITEM_PLAIN = 0, ITEM_PASS_A = 1, ITEM_PASS_B = 2, ITEM_QUARTER = 3 };

// Queues: one per XCD group. Tiles are grouped into GS_GROUPS vertical strips of
// the image, so neighbouring tiles (which share splats) and the four quarters of
// one tile are served by the workers of one XCD and its L2. Group g's queue
// holds, in order, the pass-A items of its chunked tiles, their pass-B items,
// then the quarters of its other tiles (longest first); workers that empty
// their group's queue take from the others.
#define GS_GROUPS 8
#define GS_HEAD_STRIDE 16  // ints between two queue heads (one 64-byte line)
// One workgroup of 16 wave workers per CU (4 per SIMD): the waves of a CU share
// one LDS mask of drained queues.
#define GS_WAVES_PER_BLOCK 16

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
  int32_t qoff[GS_GROUPS + 1];  // group g's items are items[qoff[g], qoff[g+1])
  int32_t qa[GS_GROUPS];        // pass-A items at the front of group g (as many pass-B follow)
  // Items handed out without a queue pop: a worker's first item is the one at
  // its index within its group (in the forward only in groups without chunk
  // items, since a pass-B item waits on items in front of it).
  int32_t init_f[GS_GROUPS], init_b[GS_GROUPS];
  // The backward's items of group g are bitems[bwd_base(g), + nb[g]): at most
  // GS_PIECES per forward item of the group's plain and pass-B items.
  int32_t nb[GS_GROUPS];
  // The raster kernels run only when these are set: the frame's device status
  // was GS_OK when the schedule (forward) or the backward's preparation ran.
  int32_t run_f, run_b;
  int64_t nw;  // contributor words per quarter (from the state's capacity)
  // PLAN_READY while a plan built ahead of the forward (from the binning pass's
  // tile counts) waits for it; plan_pairs is the pair total it was built for,
  // the rest the knobs and worker count it was built with.
  int32_t planned, plan_pairs;
  int32_t plan_mode, plan_force_k, plan_force_h, plan_nblocks;
  float plan_lambda, plan_beta, plan_eps;
  // 1: the forward files each backward item into a bin of its walk length as
  // the item's walk ends (bcnt, blist); 0: the backward's preparation writes
  // bitems (frames with few tiles, whose walks it may cut into pieces)
  int32_t bmode;
  int32_t bexit;  // workgroups of a backward launch that have finished
};
static_assert(sizeof(PlanHdr) <= 256, "the plan header fills one 256-byte slot");
constexpr int32_t PLAN_READY = 0x504C414E;

// Contributor record of the forward pass ("What the 3DGS Literature Left on the
// Table", Step 4, kept as a bitmap instead of a compacted list): for every
// quarter q of a tile and every 64-entry batch m of the tile's list (batches are
// aligned to the tile's first entry; chunk boundaries are multiples of 64
// entries), one 64-bit word whose bit j says that some pixel of the quarter
// blended entry 64 m + j. Quarter q's words of tile t start at word
// (start_t >> 6) + t of array q: disjoint per tile, at most ceil(cap / 64) + T + 2
// words per quarter. The forward writes every batch it walks, so words below
// ceil(last hit / 64) are current; the backward ignores the rest.
__host__ __device__ inline int64_t contrib_words(int T, int64_t cap) {
  return (cap + 63) / 64 + T + 2;
}

// Cut points of a plain tile's walk. The backward may walk a long tile as
// pieces between cuts, side by side: the piece that ends at a cut starts from
// the state the forward pass left there: per pixel the transmittance T at the
// cut, and the colour of every segment of the walk (the entries between two
// cuts), so its accumulator is (the colours of the segments behind the cut) .
// dL/dC + T_final (bg . dL/dC + dL/dT), divided by T at the cut: the sum over
// everything behind the cut, per unit T, which walking back from the end would
// have reached there. Cut c lies before batch cut_batch(c) of the tile's list.
#define GS_NCUT 3
#define GS_PIECES (GS_NCUT + 1)
__host__ __device__ __forceinline__ int cut_batch(int c) { return 2 << c; }
// A tile's cut record: floats [(4 c + ch) * 256 + 64 q + l] hold, for cut c and
// pixel l of quarter q, ch 0 T at the cut and ch 1..3 the colour of the segment
// that ends there; floats [(4 GS_NCUT + ch) * 256 + 64 q + l] the colour of the
// segment after the last cut the walk reached. A quarter writes them when its
// walk reaches a cut; qcut[4 tile + q] counts the cuts it reached.
#define GS_CUT_FLOATS ((4 * GS_NCUT + 3) * 256)

// A frame with fewer tiles than half the workers (nblocks workgroups) keeps
// them busy only with smaller items: its backward walks plain tiles by
// quarters, and only such a frame records cuts and walks long quarters in
// pieces (with more tiles than that, the walks' start-up costs more than the
// longest walks do).
__host__ __device__ __forceinline__ bool few_tiles(int ntiles, int nblocks) {
  return 2 * ntiles < GS_WAVES_PER_BLOCK * nblocks;
}
// The forward state holds cut records for frames of up to GS_CUT_TILES_MAX
// tiles (a frame with few tiles on 256 compute units has fewer than 2048).
#define GS_CUT_TILES_MAX 2048
__host__ __device__ __forceinline__ bool records_cuts(int ntiles, int nblocks) {
  return few_tiles(ntiles, nblocks) && ntiles <= GS_CUT_TILES_MAX;
}

// Backward queue order. The forward pass knows every item's walk length (its
// last hit) when the walk ends, so the backward can serve its items longest
// first by that length ([LOAD-IMB] section 4.1 orders by N_t, which overstates
// the work of tiles whose pixels saturate early): items are kept in
// quarter-octave bins of the length, longest bin first.
constexpr int BO_BITS = 6, BO_BINS = 1 << BO_BITS;

__device__ __forceinline__ uint32_t order_bin(int len) {
  const int b = (int)(4.0f * __log2f((float)max(len, 0) + 1.0f));
  return (uint32_t)(BO_BINS - 1 - min(b, BO_BINS - 1));  // ascending bin = longest first
}

// A plain tile whose walk spans more entries than this is walked by quarters
// in the backward: on a long list whose batches hold few contributors each, a
// batch costs about one memory round trip for its records, and a whole tile
// visits every batch where any of its quarters has a contributor.
constexpr int SPLIT_WALK = 2048;

// Byte layout of fwd_state for T tiles and a pair capacity cap (the contributor
// bitmap comes last, so the capacity a state serves follows from its size).
struct FwdLayout {
  size_t hdr, heads, sub_last, order, counts, items, sat, doneA, doneB, chunk_last, PA, CB, TB,
      LB, HB, bitems, qcut, cut, tlen, bcnt, blist, contrib, total;
};

__host__ __device__ inline FwdLayout fwd_layout(int T, int64_t cap) {
  FwdLayout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t r = off;
    off += (bytes + 255) / 256 * 256;
    return r;
  };
  const size_t cq = (size_t)GS_HK_MAX * 4;  // chunk items (per quad)
  L.hdr = take(sizeof(PlanHdr));
  L.heads = take(4 * (size_t)2 * GS_GROUPS * GS_HEAD_STRIDE);
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
  L.HB = take(4 * cq * 64);
  L.bitems = take(4 * (size_t)GS_PIECES * ((size_t)T * 4 + 2 * cq));
  L.qcut = take(4 * (size_t)T * 4);
  L.cut = take(4 * (size_t)(T <= GS_CUT_TILES_MAX ? T : 0) * GS_CUT_FLOATS);
  L.tlen = take(8 * (size_t)T);
  L.bcnt = take(4 * (size_t)GS_GROUPS * BO_BINS);
  L.blist = take(4 * (size_t)BO_BINS * ((size_t)T * 4 + 2 * cq));
  L.contrib = take(8 * 4 * (size_t)contrib_words(T, cap));
  L.total = off;
  return L;
}

// The largest pair capacity whose forward state fits in `bytes` (-1 if none).
__host__ __device__ inline int64_t fwd_state_capacity(int T, size_t bytes) {
  const FwdLayout L = fwd_layout(T, 0);
  if (bytes < L.total) return -1;
  const int64_t words = (int64_t)((bytes - L.contrib) / 32);
  return (words - T - 2) * 64;
}

struct FwdState {
  PlanHdr *hdr;
  int32_t *heads;  // [pass 0 fwd / 1 bwd][group] * GS_HEAD_STRIDE
  int32_t *sub_last, *order, *counts, *items, *sat, *doneA, *doneB, *chunk_last;
  float *PA, *CB, *TB;
  int32_t *LB;
  int32_t *HB;      // pass B's per-pixel hit counts (only when the forward counts)
  int32_t *bitems;  // the backward's queue items, longest walk first within each group
  int32_t *qcut;    // per quarter: the cuts its forward walk reached
  float *cut;       // per tile: the cut record (GS_CUT_FLOATS)
  uint64_t *tlen;   // per tile: its quarters' walk lengths + 1, 16 bits each, as they end
  int32_t *bcnt;    // [group][bin] backward items filed so far
  int32_t *blist;   // the backward's items by group and bin (bin_base)
  uint64_t *contrib;  // [4][nw] contributor words
  int64_t nw;         // words per quarter: the schedule sets hdr->nw, kernels copy it here
};

// Only the contributor bitmap's word count depends on the state's capacity, and
// the bitmap comes last, so the arrays are found from T alone.
__host__ __device__ inline FwdState fwd_state_at(void *base, int T) {
  const FwdLayout L = fwd_layout(T, 0);
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
  s.HB = reinterpret_cast<int32_t *>(b + L.HB);
  s.bitems = reinterpret_cast<int32_t *>(b + L.bitems);
  s.qcut = reinterpret_cast<int32_t *>(b + L.qcut);
  s.cut = reinterpret_cast<float *>(b + L.cut);
  s.tlen = reinterpret_cast<uint64_t *>(b + L.tlen);
  s.bcnt = reinterpret_cast<int32_t *>(b + L.bcnt);
  s.blist = reinterpret_cast<int32_t *>(b + L.blist);
  s.contrib = reinterpret_cast<uint64_t *>(b + L.contrib);
  s.nw = 0;
  return s;
}

// First contributor word of quarter q of the tile whose list starts at `start`.
__host__ __device__ __forceinline__ uint64_t *contrib_base(const FwdState &fs, int q, int tile,
                                                         int start) {
  return fs.contrib + (int64_t)q * fs.nw + (start >> 6) + tile;
}

__host__ __device__ __forceinline__ int32_t *queue_head(const FwdState &fs, int pass, int g) {
  return fs.heads + (pass * GS_GROUPS + g) * GS_HEAD_STRIDE;
}

// First of group g's backward items in bitems[].
__host__ __device__ __forceinline__ int bwd_base(const PlanHdr *hd, int g) {
  return GS_PIECES * (hd->qoff[g] + hd->qa[g]);
}

// First slot of bin b of group g in blist[]: each bin of a group has room for
// every item of the group's forward queue (a backward item comes from one
// forward item: a whole tile from its quarter 0, a quarter or a chunk quarter
// from itself).
__host__ __device__ __forceinline__ int bin_base(const PlanHdr *hd, int g, int b) {
  return BO_BINS * hd->qoff[g] + b * (hd->qoff[g + 1] - hd->qoff[g]);
}


// Workers of group g when `nblocks` workgroups are launched (workgroup b runs on
// XCD b mod GS_GROUPS).
__host__ __device__ __forceinline__ int group_workers(int g, int nblocks) {
  return GS_WAVES_PER_BLOCK * ((nblocks - g + GS_GROUPS - 1) / GS_GROUPS);
}

// Group (XCD strip) of a tile: vertical strips of the tile grid.
__host__ __device__ __forceinline__ int tile_group(int tile, int tiles_x) {
  return (tile % tiles_x) * GS_GROUPS / tiles_x;
}

// Index of (slot s, chunk p, quad q) among the chunk items.
__device__ __forceinline__ int chunk_index(int s, int p, int q, int k) { return (s * k + p) * 4 + q; }

// Chunk p of k over [start, end): contiguous pieces of ceil(N/k) entries rounded
// up to a multiple of 64 (so every chunk starts on a contributor word; the last
// pieces may be shorter or empty).
__device__ __forceinline__ void chunk_range(int start, int end, int p, int k, int &cs, int &ce) {
  const int N = end - start;
  const int csize = ((N + k - 1) / k + 63) & ~63;
  cs = min(end, start + p * csize);
  ce = min(end, cs + csize);
}


struct SubTile {
  int tile, quad, x0, y0;    // x0, y0 in the coordinates of the tile's view
  int prow;                  // the view's first pixel row in the batch outputs
  float hx0, hx1, hy0, hy1;  // sample hull of the 8x8 quarter
  bool empty;
};

__device__ __forceinline__ SubTile subtile_of(int tile, int quad, const CamK &cam) {
  SubTile st;
  st.tile = tile;
  st.quad = quad;
  const int tx = tile % cam.tiles_x, tyb = tile / cam.tiles_x;
  const int view = tyb / cam.vty, ty = tyb - view * cam.vty;
  st.prow = view * cam.height;
  st.x0 = tx * 16 + (quad & 1) * 8;
  st.y0 = ty * 16 + (quad >> 1) * 8;
  st.empty = st.x0 >= cam.width || st.y0 >= cam.height;
  st.hx0 = (float)st.x0 + 0.5f;
  st.hx1 = (float)min(st.x0 + 7, cam.width - 1) + 0.5f;
  st.hy0 = (float)st.y0 + 0.5f;
  st.hy1 = (float)min(st.y0 + 7, cam.height - 1) + 0.5f;
  return st;
}

// A workgroup holds GS_WAVES_PER_BLOCK independent wave workers, each with its
// own slice of LDS.

__device__ __forceinline__ int wave_in_block() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / GS_WAVE);
}


// Wave-uniform queue pop: one lane advances the head, every lane gets the ticket.
__device__ __forceinline__ int queue_pop(int32_t *head) {
  int t = 0;
  if (__lane_id() == 0) t = atomicAdd(head, 1);
  return wave_first(t);
}

// Spin on a flag with relaxed loads (no cache invalidation per probe); the
// caller issues one acquire fence after it succeeds.
__device__ __forceinline__ int ld_flag(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A persistent worker: its home group (the XCD it runs on), its index within
// that group, its round, and what it knows of drained queues: its own
// findings and the LDS mask of its workgroup.
struct Worker {
  int home, wg, round;
  uint32_t known;     // groups this wave found empty
  uint32_t *drained;  // the workgroup's LDS mask of groups found empty
};

// Call from every thread of the workgroup, before any of its waves pops.
__device__ __forceinline__ Worker make_worker(uint32_t *drained) {
  if (threadIdx.x == 0) *drained = 0u;
  __syncthreads();
  Worker w;
  w.home = blockIdx.x % GS_GROUPS;
  // wave v of the group's j-th workgroup: consecutive items (the quarters of a
  // tile) go to different workgroups, as they would from a shared queue
  const int blocks = (gridDim.x - w.home + GS_GROUPS - 1) / GS_GROUPS;
  w.wg = wave_in_block() * blocks + (int)(blockIdx.x / GS_GROUPS);
  w.round = 0;
  w.known = 0u;
  w.drained = drained;
  return w;
}

// The lowest set slot of w, or 63 when w is empty (s_ff1 gives -1 there): the
// walk below then reads slot 63's record ahead and never uses it, which spares
// it a compare and two selects per entry.
__device__ __forceinline__ int next_slot(uint64_t w) {
  int j;
  __asm__("s_ff1_i32_b64 %0, %1" : "=s"(j) : "s"(w));
  return j & 63;
}

// w without slot j, and w with slot j (one scalar instruction each).
__device__ __forceinline__ uint64_t clear_slot(uint64_t w, int j) {
  __asm__("s_bitset0_b64 %0, %1" : "+s"(w) : "s"(j));
  return w;
}
__device__ __forceinline__ uint64_t set_slot(uint64_t w, int j) {
  __asm__("s_bitset1_b64 %0, %1" : "+s"(w) : "s"(j));
  return w;
}

// Walk a staged worklist (the set bits of w, lowest slot first) and call
// f(record, slot) on each until f returns false. The LDS read of the next
// entry's record is issued before f runs on the current one, so its latency
// overlaps the work on the current entry; two record buffers alternate, so no
// register copies are made.
template <class Rec, class F>
__device__ __forceinline__ void walk_worklist(uint64_t w, const Rec *sbuf, F &&f) {
  if (!w) return;
  int j0 = next_slot(w);
  w = clear_slot(w, j0);
  Rec s0 = sbuf[j0];
  for (;;) {
    const bool more1 = w != 0;
    const int j1 = next_slot(w);
    w = clear_slot(w, j1);  // an empty set stays empty
    const Rec s1 = sbuf[j1];
    const bool go1 = f(s0, j0);
    if (!more1) return;
    if (!go1) return;
    const bool more0 = w != 0;
    j0 = next_slot(w);
    w = clear_slot(w, j0);
    s0 = sbuf[j0];
    const bool go0 = f(s1, j1);
    if (!more0) return;
    if (!go0) return;
  }
}

// One pop on group g's queue: the item index, or -1 if the queue is empty (then
// g is recorded as drained in the wave and in the workgroup's LDS mask).
__device__ __forceinline__ int pop_group(const FwdState &fs, int pass, Worker &w, int g) {
  const PlanHdr *hd = fs.hdr;
  const int lo = pass ? bwd_base(hd, g) : hd->qoff[g];
  const int hi = pass ? lo + hd->nb[g] : hd->qoff[g + 1];
  if (lo < hi) {
    const int t = queue_pop(queue_head(fs, pass, g));
    if (lo + t < hi) return lo + t;
  }
  w.known |= 1u << g;
  if (__lane_id() == 0)
    __hip_atomic_fetch_or(w.drained, 1u << g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return -1;
}

// Next item (an index into items[], or bitems[] for the backward) of a worker,
// or -1 when every queue is empty. pass 0 (forward) serves every item of a
// group; pass 1 (backward) serves the nb[g] items that its preparation wrote
// from bwd_base(g) on. The first item comes without a pop: the queue heads
// start past the items handed out that way, so a frame's first wave of work
// does not serialise on the heads. After that the worker pops its home group,
// then the others nearest first (+1, -1, +2, ...), neighbouring strips sharing
// more splats.
//
// A pop on a drained head is a same-address atomic, and at the end of a frame
// every worker would make one per group: thousands of them, serialised on
// eight addresses, behind the pops of the workers still busy. So a pop that
// comes back empty is recorded in the workgroup's LDS mask and the other waves
// of the CU skip that queue; every bit records a pop that came back empty, so
// each round either returns an item or learns one more empty group.
__device__ __forceinline__ int next_item(const FwdState &fs, int pass, Worker &w) {
  const PlanHdr *hd = fs.hdr;
  if (w.round == 0) {
    const int init = pass ? hd->init_b[w.home] : hd->init_f[w.home];
    if (w.wg < init) return (pass ? bwd_base(hd, w.home) : hd->qoff[w.home]) + w.wg;
  }
  for (int c = 0; c < GS_GROUPS; c++) {
    const int g = (w.home + (c + 1) / 2 * ((c & 1) ? 1 : -1) + GS_GROUPS) % GS_GROUPS;
    if (w.known & (1u << g)) continue;
    const uint32_t dm = __hip_atomic_load(w.drained, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (wave_first((int)dm) & (1 << g)) {
      w.known |= 1u << g;
      continue;
    }
    const int t = pop_group(fs, pass, w, g);
    if (t >= 0) return t;
  }
  return -1;
}

// The backward's items filed in bins by the forward (bmode 1). Each workgroup
// keeps every group's bin starts in LDS: bpre[g][b] = items of group g in
// bins before b, bpre[g][BO_BINS] the group's total. Wave g < GS_GROUPS
// loads group g's counts (bin_count, issued first, beside the header's loads)
// and scans them; call bin_starts from every thread before make_worker (whose
// barrier publishes the table).
constexpr int BPRE = BO_BINS + 1;
__device__ __forceinline__ int bin_count(const FwdState &fs) {
  const int g = threadIdx.x >> 6;
  return g < GS_GROUPS ? fs.bcnt[g * BO_BINS + (threadIdx.x & 63)] : 0;
}
__device__ __forceinline__ void bin_starts(int v, int *bpre) {
  const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
  if (g < GS_GROUPS) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(v, d, 64);
      if (lane >= d) v += u;
    }
    bpre[g * BPRE + lane + 1] = v;
    if (lane == 0) bpre[g * BPRE] = 0;
  }
}

// Item at position c of group g's backward order (bins longest first).
__device__ __forceinline__ int bin_item(const FwdState &fs, const int *bpre, int g, int c) {
  const int lane = __lane_id();
  // bins that end at or before c come first (the starts are non-decreasing)
  const int b = __popcll(wave_ballot(bpre[g * BPRE + lane + 1] <= c));
  return fs.blist[bin_base(fs.hdr, g, b) + c - bpre[g * BPRE + b]];
}

// Next backward item from the bins into `it`; false when every group is
// served (an item's kind sits in its top bits, so no value of `it` is free to
// mark that). The same hand-out as next_item: the first item by the worker's
// index in its home group, then pops, home group first, with group g's head
// counting the pops past its static hand-out.
__device__ __forceinline__ bool next_bin_item(const FwdState &fs, const int *bpre, Worker &w,
                                              int nblocks, int &it) {
  if (w.round == 0) {
    const int tot = bpre[w.home * BPRE + BO_BINS];
    if (w.wg < min(tot, group_workers(w.home, nblocks))) {
      it = bin_item(fs, bpre, w.home, w.wg);
      return true;
    }
  }
  for (int c = 0; c < GS_GROUPS; c++) {
    const int g = (w.home + (c + 1) / 2 * ((c & 1) ? 1 : -1) + GS_GROUPS) % GS_GROUPS;
    if (w.known & (1u << g)) continue;
    const uint32_t dm = __hip_atomic_load(w.drained, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (wave_first((int)dm) & (1 << g)) {
      w.known |= 1u << g;
      continue;
    }
    const int tot = bpre[g * BPRE + BO_BINS];
    const int init = min(tot, group_workers(g, nblocks));
    if (init < tot) {
      const int pos = init + queue_pop(queue_head(fs, 1, g));
      if (pos < tot) {
        it = bin_item(fs, bpre, g, pos);
        return true;
      }
    }
    w.known |= 1u << g;
    if (__lane_id() == 0)
      __hip_atomic_fetch_or(w.drained, 1u << g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  return false;
}

__device__ __forceinline__ void st_flag(int32_t *p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
