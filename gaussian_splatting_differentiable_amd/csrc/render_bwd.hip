// gs_render_bwd: gradients of the blended image with respect to the 9
// screen-space splat parameters (centre x/y, conic a/b/c, opacity, r/g/b).
//
// "What the 3DGS Literature Left on the Table": Step 1 (a) per-pixel
// derivatives summed over a wave before global atomics; Step 1 (e) the scalar
// accumulator accum = c_behind . dL/dC; Step 2 the reduce-scatter that leaves
// the 9 sums on 9 lanes for one atomic instruction; Step 4 the walk from the
// last contributor back to the front over the contributors the forward pass
// recorded (here a bitmap per quarter and 64-entry batch), with no geometric
// sub-tile test; Step 5 branchless alpha = 0 predication for missed pixels and
// one canonical q shared with the forward pass; Step 6.1 two vertically
// adjacent pixels per lane (here four), sharing the column terms of q and summed
// in registers before the reduction; Step 6.3 the per-splat term
// alpha T (c . dL/dC - accum), with log2(o) folded into the exponent and o
// divided back out once after the sum; Step 6.4 the rows' offsets combined
// without per-row products by the row index.
// "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on GPUs",
// section 4: the same persistent longest-first queue as the forward pass; a
// chunk of a heavy tile is differentiated on its own from the forward pass's
// chunk state: it starts from the transmittance after its last processed
// splat, T_end, with accum = (sum over later chunks of C_chunk . dL/dC) / T_end.
//
// gfx950 mapping: one wavefront per item, a whole tile (or chunk): row q of 16
// lanes holds quarter q, lane s of the row column s mod 8 and rows 4 (s / 8) to
// 4 (s / 8) + 3, so a row's DPP exchanges reduce its quarter's sums. Each row
// walks its own quarter's contributors, so a step evaluates up to four splats.
// The item's non-empty batches come from one vector load of the contributor
// words; each batch stages only its contributors' records in LDS (the next
// batch's ids and records in flight) and is walked on the scalar unit.
#include <type_traits>

#include "render_common.h"
#include "wave_reduce.h"

namespace {

constexpr float NEG_HALF_LOG2E = -0.72134752044448170368f;

// The backward's preparation for frames with few tiles: one workgroup per
// group sorts the group's backward items (quarters, or their pieces between
// cuts) stably by the bin of their walk length.
constexpr int BO_T = 1024, BO_W = BO_T / 64;
constexpr int BO_IPL = 4;  // items per lane per span of the queue build

// Walk length of a backward item: its quarter's last hit, or the longest of
// the four for a whole tile.
__device__ __forceinline__ int item_len(const FwdState &fs, int it, int k) {
  const int idx = item_index(it), q = item_quad(it);
  switch (item_kind(it)) {
    case ITEM_PLAIN:
      return max(max(fs.sub_last[idx * 4], fs.sub_last[idx * 4 + 1]),
                 max(fs.sub_last[idx * 4 + 2], fs.sub_last[idx * 4 + 3]));
    case ITEM_QUARTER:
      return fs.sub_last[idx * 4 + q];
    default:
      return fs.chunk_last[chunk_index(idx, item_chunk(it), q, k)];
  }
}

// The backward item a forward item of the group's queue gives, or -1, and its
// walk length: a chunk's quarter (pass B) gives itself; a plain tile gives one
// whole-tile item (from its quarter 0), or one item per quarter when the frame
// has too few tiles to keep the workers busy or the tile's walk is long.
__device__ __forceinline__ int bwd_item(const FwdState &fs, int it, bool split, int k, int &len) {
  const int kind = item_kind(it), q = item_quad(it), idx = item_index(it);
  len = 0;
  if (kind == ITEM_PASS_B) {
    len = item_len(fs, it, k);
    return it;
  }
  if (kind != ITEM_PLAIN) return -1;
  const int4 v = *reinterpret_cast<const int4 *>(fs.sub_last + idx * 4);
  const int whole = max(max(v.x, v.y), max(v.z, v.w));
  if (split || whole > SPLIT_WALK) {
    len = q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
    return make_item(ITEM_QUARTER, q, 0, idx);
  }
  len = whole;
  return q == 0 ? it : -1;
}

__device__ __forceinline__ int ceil64(int v) { return (max(v, 0) + 63) >> 6; }

// Pieces of a plain walk of nb batches: one per cut below nb, and the rest.
__device__ __forceinline__ int pieces_of(int nb) {
  int p = 1;
#pragma unroll
  for (int c = 0; c < GS_NCUT; c++) p += cut_batch(c) < nb ? 1 : 0;
  return p;
}

// Batches [a, e) of piece i of a plain walk of nb batches; piece i < the last
// ends at cut i.
__device__ __forceinline__ void piece_range(int i, int nb, int &a, int &e) {
  a = i == 0 ? 0 : cut_batch(i - 1);
  e = i < GS_NCUT && cut_batch(i) < nb ? cut_batch(i) : nb;
}

// In a frame with few tiles, a plain walk is cut into pieces when it spans at
// least 3 batches and more than its group's batches per worker: only then can
// one walk outlast the rest of the frame's work, and each piece costs a walk's
// start-up (a chain of dependent loads) again.

// The backward's preparation in one launch: workgroup g < GS_GROUPS builds group
// g's backward queue: each of the forward's plain and pass-B items gives its
// backward items (a whole tile, or in a frame with few tiles (FEW) a quarter
// or its pieces between cuts, or the chunk quarter), stably sorted longest
// first; the others zero the gradient output. The frame runs only if its
// status is still GS_OK.
template <bool FEW>
__global__ void __launch_bounds__(BO_T) k_bwd_prep(char *__restrict__ state, int ntiles,
                                                  int nblocks, float *__restrict__ grads,
                                                  int64_t ng, const int32_t *__restrict__ status) {
  if (blockIdx.x >= GS_GROUPS) {
    const int64_t i = (int64_t)(blockIdx.x - GS_GROUPS) * BO_T + threadIdx.x;
    const int64_t n4 = ng / 4;
    if (i < n4) reinterpret_cast<float4 *>(grads)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < ng - 4 * n4) grads[4 * n4 + i] = 0.0f;
    return;
  }
  __shared__ int cnt[BO_W][BO_BINS];
  __shared__ int run;
  FwdState fs = fwd_state_at(state, ntiles);
  if (threadIdx.x == 0) {
    run = fs.hdr->run_f && *status == GS_OK;
    if (blockIdx.x == 0) fs.hdr->run_b = run;
  }
  __syncthreads();
  const int g = blockIdx.x, k = fs.hdr->k;
  const int lo = fs.hdr->qoff[g] + fs.hdr->qa[g], hi = run ? fs.hdr->qoff[g + 1] : lo;
  const int n = hi - lo;
  const int blo = bwd_base(fs.hdr, g);  // at most GS_PIECES backward items per forward item
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __shared__ int load;  // the group's walks in batches
  for (int i = threadIdx.x; i < BO_W * BO_BINS; i += BO_T) (&cnt[0][0])[i] = 0;
  if (threadIdx.x == 0) load = 0;
  __syncthreads();
  // the group's items in spans of BO_T * BO_IPL; wave w takes a contiguous
  // piece of each, and a lane's items and their loads go out together (a span
  // holds a garden-sized group, so its items stay in registers for the scatter)
  constexpr int SPAN = BO_T * BO_IPL;
  int itr[BO_IPL], ln[BO_IPL], np[BO_IPL];
  uint32_t dr[BO_IPL];  // the bin of the whole walk
#pragma unroll
  for (int j = 0; j < BO_IPL; j++) itr[j] = -1;
  int c0 = 0;
  auto load_span = [&](int o) {
    const int m = min(SPAN, n - o), per = (m + BO_W - 1) / BO_W;
    c0 = o + min(m, w * per);
    const int c1 = o + min(m, w * per + per);
    int raw[BO_IPL];
#pragma unroll
    for (int j = 0; j < BO_IPL; j++) {
      const int e = c0 + lane + 64 * j;
      raw[j] = e < c1 ? fs.items[lo + e] : -1;
    }
#pragma unroll
    for (int j = 0; j < BO_IPL; j++) {
      ln[j] = 0;
      itr[j] = raw[j] != -1 ? bwd_item(fs, raw[j], FEW, k, ln[j]) : -1;
      dr[j] = order_bin(ln[j]);
    }
  };
  // 1. the group's load: its walks' batches (a frame with few tiles cuts the
  //    walks longer than its batches per worker)
  if constexpr (FEW) {
    int mine = 0;
    for (int o = 0; o < n; o += SPAN) {
      load_span(o);
#pragma unroll
      for (int j = 0; j < BO_IPL; j++) mine += itr[j] != -1 ? ceil64(ln[j]) : 0;
    }
    if (mine) atomicAdd(&load, mine);
    __syncthreads();
  }
  const int64_t wl = group_workers(g, nblocks);
  const bool cuts = records_cuts(ntiles, nblocks);  // the forward recorded the cuts
  auto set_pieces = [&]() {
#pragma unroll
    for (int j = 0; j < BO_IPL; j++) {
      const int nb = ceil64(ln[j]);
      np[j] = itr[j] == -1 ? 0
              : FEW && cuts && item_kind(itr[j]) != ITEM_PASS_B && nb >= 3 &&
                        nb * wl > (int64_t)load
                  ? pieces_of(nb)
                  : 1;
    }
  };
  // piece i of item j (its walk length in entries sets its bin)
  auto piece = [&](int j, int i, uint32_t &bin) {
    if (np[j] == 1) {
      bin = dr[j];
      return itr[j];
    }
    int a, e;
    piece_range(i, ceil64(ln[j]), a, e);
    bin = order_bin(min(ln[j], 64 * e) - 64 * a);
    return itr[j] | ((i + 1) << 24);
  };
  // 2. counts per bin
  if (FEW && n <= SPAN) set_pieces();
  for (int o = 0; o < n; o += SPAN) {
    if (!FEW || n > SPAN) load_span(o);
    if constexpr (FEW) {
      if (n > SPAN) set_pieces();
#pragma unroll
      for (int j = 0; j < BO_IPL; j++)
        for (int i = 0; i < np[j]; i++) {
          uint32_t d;
          piece(j, i, d);
          atomicAdd(&cnt[w][d], 1);
        }
    } else {
#pragma unroll
      for (int j = 0; j < BO_IPL; j++)
        if (itr[j] != -1) atomicAdd(&cnt[w][dr[j]], 1);
    }
  }
  __syncthreads();
  __shared__ int btot[BO_BINS];
  if (threadIdx.x < BO_BINS) {
    int t = 0;
    for (int q = 0; q < BO_W; q++) t += cnt[q][threadIdx.x];
    btot[threadIdx.x] = t;
  }
  __syncthreads();
  if (threadIdx.x < BO_BINS) {
    // exclusive offsets in (bin, wave) order
    int run_ = 0;
    for (int d = 0; d < (int)threadIdx.x; d++) run_ += btot[d];
    for (int q = 0; q < BO_W; q++) {
      const int c = cnt[q][threadIdx.x];
      cnt[q][threadIdx.x] = run_;
      run_ += c;
    }
    if (threadIdx.x == BO_BINS - 1) {
      // the backward's own hand-out: the first items go to its workers without a pop
      const int nb = run_;
      const int init = min(nb, group_workers(g, nblocks));
      fs.hdr->nb[g] = nb;
      fs.hdr->init_b[g] = init;
      queue_head(fs, 1, g)[0] = init;
    }
  }
  __syncthreads();
  // 3. scatter, in the order the counts were taken
  const uint64_t lt = (1ull << lane) - 1ull;
  // piece i of a lane's item j (or the whole walk), ranked among the wave's
  // lanes with the same bin
  auto place = [&](int j, int i) {
    const bool valid = FEW ? i < np[j] : itr[j] != -1;
    uint32_t d = 0;
    int item = -1;
    if constexpr (FEW) {
      if (valid) item = piece(j, i, d);
    } else {
      d = valid ? dr[j] : 0u;
      item = itr[j];
    }
    uint64_t peers = wave_ballot(valid);
#pragma unroll
    for (int b = 0; b < BO_BITS; b++) {
      const uint64_t bal = wave_ballot((d >> b) & 1u);
      peers &= ((d >> b) & 1u) ? bal : ~bal;
    }
    if (valid) {
      const int below = __popcll(peers & lt);
      const int pos = cnt[w][d] + below;
      fs.bitems[blo + pos] = item;
      if (below == __popcll(peers) - 1) cnt[w][d] = pos + 1;
    }
  };
  for (int o = 0; o < n; o += SPAN) {
    if (n > SPAN) {
      load_span(o);
      if constexpr (FEW) set_pieces();
    }
#pragma unroll
    for (int j = 0; j < BO_IPL; j++) {
      place(j, 0);
      if constexpr (FEW) {
        if (wave_ballot(np[j] > 1))
          for (int i = 1; i < GS_PIECES; i++) place(j, i);
      }
    }
  }
}

constexpr int BATCH = GS_WAVE;  // entries per batch (one contributor word)

__device__ __forceinline__ bool valid_id(int id, int n) { return (unsigned)id < (unsigned)n; }

// This lane's list entry of a batch, if the batch's word marks it (else -1).
__device__ __forceinline__ int load_marked_id(const int32_t *__restrict__ sids, int64_t b,
                                              uint64_t word) {
  return (word >> __lane_id()) & 1ull ? sids[b + __lane_id()] : -1;
}

// The 64-bit contributor word of batch m held by lane m of the current round.
__device__ __forceinline__ uint64_t word_of(uint32_t lo, uint32_t hi, int m) {
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, m) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)lo, m);
}

// A staged entry (48 bytes): the record with 2b, log2(o) and 1/o in place of
// depth, pad and o. Slot 64 of a wave's stage is a dead entry (tau = -1, never
// hit) that a quarter with no entry left reads.
struct __align__(16) Staged {
  float4 p0;  // mx, my, a, b
  float4 p1;  // c, 1/o, r, g
  float4 p2;  // b (colour), tau, 2b, log2(o)
};
constexpr int SLOTS = BATCH + 1;

// The highest slot of w, removed from w; BATCH (the dead slot) when w is empty.
// s_flbit gives the leading zeros, -1 for an empty word, so 63 - f is 64 there,
// and clearing bit 64 mod 64 of an empty word leaves it empty.
__device__ __forceinline__ int take_top(uint64_t &w) {
  int f;
  __asm__("s_flbit_i32_b64 %0, %1" : "=s"(f) : "s"(w));
  const int j = 63 - f;
  __asm__("s_bitset0_b64 %0, %1" : "+s"(w) : "s"(j));
  return j;
}

// One batch's gradient sums, from the LDS accumulators to the output: 63 lanes
// take 7 slots' 9 sums at a time, so each atomic instruction writes 7 splats'
// rows of 9 consecutive floats (a line or two each), once per splat per batch
// whichever quarters blended it. rows[j]: slot j's gradient row (its byte
// offset, or its splat id when WIDE), -1 for a slot without an entry. The
// accumulators are left at zero.
template <bool WIDE>
__device__ __forceinline__ void flush(uint64_t staged, const int32_t *rows, float *gacc,
                                      float *__restrict__ grads) {
  const int lane = __lane_id();
  const int ds = lane / 9, c = lane - 9 * ds;  // slot within the group of 7, component
#pragma unroll
  for (int g0 = 0; g0 < BATCH; g0 += 7) {
    if (((staged >> g0) & 0x7Full) == 0) continue;
    const int slot = g0 + ds;
    if (lane < 63 && slot < BATCH) {
      const float v = gacc[9 * g0 + lane];
      gacc[9 * g0 + lane] = 0.0f;
      const int32_t row = rows[slot];
      if (row != -1) {
        if constexpr (WIDE)
          unsafeAtomicAdd(&grads[9 * (int64_t)row + c], v);
        else
          unsafeAtomicAdd(reinterpret_cast<float *>(reinterpret_cast<char *>(grads) +
                                                    ((uint32_t)row + 4u * (uint32_t)c)),
                          v);
      }
    }
  }
}

// Per-lane state: four vertically adjacent pixels of one column of a quarter.
struct Pix4 {
  float fx, fy[4];         // sample positions
  float T[4], acc[4];      // transmittance after the pixel's last entry; accumulator
  float g[4][3];           // dL/dC
  int last[4];             // entries the pixel consumed from the walk's start
};

// Walk the item's batches back to front. cw[q]: quarter q's contributor words
// at the walk's first batch; nbw[q]: how many of them are current (the rest
// were not written for this frame); list: the walk's first list position. The
// 16 lanes of row q of the wave hold quarter q's pixels and take its entries
// back to front, one per step: a step evaluates up to four different splats,
// one per quarter, and a quarter with no entry left reads the dead slot.
template <bool WIDE>
__device__ __forceinline__ void walk_back(const Splat *__restrict__ splats, int n,
                                          const int32_t *__restrict__ sids, int64_t list,
                                          const uint64_t *cw0, int64_t nw, const int nbw[4],
                                          Pix4 &x, Staged *stage, float *gacc2,
                                          int32_t *rows2, float *__restrict__ grads) {
  const int lane = __lane_id();
  const uint32_t shift = 8u * (uint32_t)(lane >> 4);  // this row's byte of the packed slots
  const int comp = comp_of_row_lane(lane);
  const bool lo2 = (lane & 2) == 0, lo1 = (lane & 1) == 0;
  float *gacc = gacc2;
  // the constant factor each owner lane applies to its sum after the reduction
  // (powers of two: exact): -1/2 for the two squared offsets
  const float post = (comp == 2 || comp == 4) ? -0.5f : 1.0f;
  const float4 *rec4 = reinterpret_cast<const float4 *>(splats);
  // the next batch's record of this lane, as three registers of four (kept out
  // of any aggregate: the compiler parks part of one in memory otherwise)
  float4 q0 = make_float4(0.f, 0.f, 0.f, 0.f), q1 = q0, q2 = q0;
  // x.last becomes, per batch, the limit last - (the batch's first position)
  int lbase = 0;
  // Two sets of accumulators and gradient rows alternate between batches: a
  // batch's sums are flushed after the next batch is staged, so the atomics
  // have that batch's walk to drain before the next wait on memory (one
  // counter covers loads and stores).
  int buf = 0;
  uint64_t pend = 0;  // the batch waiting for its flush (in set buf ^ 1)
  const int nbat = max(max(nbw[0], nbw[1]), max(nbw[2], nbw[3]));
  for (int r0 = (nbat - 1) & ~63; r0 >= 0; r0 -= 64) {
    // lane i holds the words of batch r0 + i, one per quarter
    const int m = r0 + lane;
    uint32_t wlo[4], whi[4];
    uint64_t any = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const uint64_t v = m < nbw[q] ? cw0[q * nw + m] : 0ull;
      wlo[q] = (uint32_t)v;
      whi[q] = (uint32_t)(v >> 32);
      any |= v;
    }
    uint64_t todo = wave_ballot(any != 0);
    if (!todo) continue;
    // every quarter's contributors of batch mb of this round
    auto any_word = [&](int mb) {
      uint64_t w = 0;
#pragma unroll
      for (int q = 0; q < 4; q++) w |= word_of(wlo[q], whi[q], mb);
      return w;
    };
    // pipeline: the records of the batch being staged and the ids of the next
    // non-empty batch are in flight while a batch is walked
    int mc = 63 - __builtin_clzll(todo);
    todo &= ~(1ull << mc);
    int idc = load_marked_id(sids, list + 64 * (int64_t)(r0 + mc), any_word(mc));
    {
      const int64_t ri = 3 * (int64_t)(valid_id(idc, n) ? idc : 0);
      q0 = rec4[ri];
      q1 = rec4[ri + 1];
      q2 = rec4[ri + 2];
    }
    int mn = -1, idn = -1;
    if (todo) {
      mn = 63 - __builtin_clzll(todo);
      todo &= ~(1ull << mn);
      idn = load_marked_id(sids, list + 64 * (int64_t)(r0 + mn), any_word(mn));
    }
    for (;;) {
      // whether any splat of the batch can reach the 0.99 clamp: o G < 0.99
      // whenever o <= 0.985 (G <= 1; the margin covers the rounding of
      // exp2(log2 o)), so most batches take the step without the clamp's
      // select and compare, with the same results bit for bit
      const bool bclamp = wave_ballot(valid_id(idc, n) && q1.y > 0.985f) != 0;
      {
        // 2b, log2(o) (the forward pass folds it the same way) and 1/o
        const float4 p1 = make_float4(q1.x, __builtin_amdgcn_rcpf(q1.y), q1.z, q1.w);
        const float4 p2 = make_float4(q2.x, q2.y, 2.0f * q0.w, __log2f(q1.y));
        stage[lane].p0 = q0;
        stage[lane].p1 = p1;
        stage[lane].p2 = p2;
        // the gradient row: its byte offset (rows of 36 bytes), or the id when WIDE
        rows2[BATCH * buf + lane] =
            valid_id(idc, n) ? (WIDE ? idc : (int)(36u * (uint32_t)idc)) : -1;
      }
      if (pend) flush<WIDE>(pend, rows2 + BATCH * (buf ^ 1), gacc2 + 9 * SLOTS * (buf ^ 1), grads);
      // records of the next batch, ids of the one after it
      idc = idn;
      {
        const int64_t rj = 3 * (int64_t)(valid_id(idc, n) ? idc : 0);
        q0 = rec4[rj];
        q1 = rec4[rj + 1];
        q2 = rec4[rj + 2];
      }
      int mnn = -1;
      idn = -1;
      if (todo) {
        mnn = 63 - __builtin_clzll(todo);
        todo &= ~(1ull << mnn);
        idn = load_marked_id(sids, list + 64 * (int64_t)(r0 + mnn), any_word(mnn));
      }
      wave_sync();
      // a pixel takes entry j only below its own stop: j < last - base (the
      // dead slot, j = 64, never hits)
      const int base = 64 * (r0 + mc);
#pragma unroll
      for (int k = 0; k < 4; k++) x.last[k] -= base - lbase;
      lbase = base;
      uint64_t wc[4];
#pragma unroll
      for (int q = 0; q < 4; q++) wc[q] = word_of(wlo[q], whi[q], mc);
      // steps of this batch: the most entries any quarter takes
      const int nsteps =
          max(max(__builtin_popcountll(wc[0]), __builtin_popcountll(wc[1])),
              max(__builtin_popcountll(wc[2]), __builtin_popcountll(wc[3])));
      auto step = [&](auto clamp_t, const Staged &s, int j) {
        constexpr bool CLAMP = decltype(clamp_t)::value;
        const float a = s.p0.z, b = s.p0.w, c = s.p1.x;
        // the column terms of the canonical q are shared by the lane's four rows
        const float dx = x.fx - s.p0.x;
        const float adxdx = (a * dx) * dx, b2dx = s.p2.z * dx;
        float mk[4], wk[4], dy0 = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const float dy = x.fy[k] - s.p0.y;
          if (k == 0) dy0 = dy;
          const float qk = __builtin_fmaf(c * dy, dy, __builtin_fmaf(b2dx, dy, adxdx));
          const bool h = j < x.last[k] && qk <= s.p2.y;
          // branchless: a missed pixel takes alpha = 0, which leaves T and accum
          // unchanged and contributes zero to every sum
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(qk, NEG_HALF_LOG2E, s.p2.w));
          const float oG = h ? e : 0.0f;  // o G
          const float al = CLAMP ? fminf(0.99f, oG) : oG;
          x.T[k] = x.T[k] * __builtin_amdgcn_rcpf(1.0f - al);  // T before this splat
          const float cg = __builtin_fmaf(s.p1.z, x.g[k][0],
                                          __builtin_fmaf(s.p1.w, x.g[k][1], s.p2.x * x.g[k][2]));
          const float d = cg - x.acc[k];  // dL/dalpha = T d
          x.acc[k] = __builtin_fmaf(al, d, x.acc[k]);
          wk[k] = al * x.T[k];
          // -2 dL/dq = alpha T d, which is also o G dL/dalpha: an unclamped
          // alpha is o G; a clamped alpha passes no gradient
          mk[k] = !CLAMP || oG < 0.99f ? wk[k] * d : 0.0f;
        }
        // the lane's rows, dy_k = dy0 + k: with M = sum m_k, R1 = sum k m_k and
        // R2 = sum k^2 m_k, Sy = sum m_k dy_k = M dy0 + R1 and Syy = sum m_k
        // dy_k^2 = dy0 (Sy + R1) + R2, and X = M dx: each derivative needs dx once
        const float M = (mk[0] + mk[1]) + (mk[2] + mk[3]);
        const float R1 = __builtin_fmaf(3.0f, mk[3], __builtin_fmaf(2.0f, mk[2], mk[1]));
        const float R2 = __builtin_fmaf(9.0f, mk[3], __builtin_fmaf(4.0f, mk[2], mk[1]));
        const float Sy = __builtin_fmaf(M, dy0, R1);
        const float X = M * dx;
        float gr[9];
        gr[0] = __builtin_fmaf(a, X, b * Sy);  // dq/dmx = -2 (a dx + b dy)
        gr[1] = __builtin_fmaf(b, X, c * Sy);  // dq/dmy = -2 (b dx + c dy)
        gr[2] = X * dx;                        // times -1/2 after the sum
        gr[3] = -(dx * Sy);
        gr[4] = __builtin_fmaf(dy0, Sy + R1, R2);  // times -1/2 after the sum
        gr[5] = M;                                 // divided by o after the sum
#pragma unroll
        for (int ch = 0; ch < 3; ch++)
          gr[6 + ch] = __builtin_fmaf(wk[3], x.g[3][ch],
                                      __builtin_fmaf(wk[2], x.g[2][ch],
                                                     __builtin_fmaf(wk[1], x.g[1][ch],
                                                                    wk[0] * x.g[0][ch])));
        float out = reduce_scatter9_row(gr, lo2, lo1);
        // finish the sum here, where its last exchange fuses into the add,
        // rather than inside the owner lanes' branch
        __asm__ volatile("" : "+v"(out));
        out *= comp == 5 ? s.p1.y : post;
        // the row's 9 sums go to the slot's accumulators in LDS (rows that took
        // the same splat add to the same ones; the dead slot collects zeros)
        if (comp >= 0) atomicAdd(&gacc[9 * SLOTS * buf + 9 * j + comp], out);
      };
      // the four quarters' slots of a step, packed a byte each on the scalar
      // unit; a lane takes its row's byte (one bit-field extract)
      auto next_slot4 = [&]() {
        const uint32_t j0 = (uint32_t)take_top(wc[0]), j1 = (uint32_t)take_top(wc[1]);
        const uint32_t j2 = (uint32_t)take_top(wc[2]), j3 = (uint32_t)take_top(wc[3]);
        const uint32_t packed = j0 | (j1 << 8) | (j2 << 16) | (j3 << 24);
        return (int)__builtin_amdgcn_ubfe(packed, shift, 8);
      };
      // the next step's reads from the stage go out before the current step
      // runs (two buffers alternate)
      auto walk = [&](auto clamp_t) {
        int left = nsteps;
        int j0 = next_slot4();
        Staged s0 = stage[j0];
        for (;;) {
          const int j1 = next_slot4();
          const Staged s1 = stage[j1];
          step(clamp_t, s0, j0);
          if (--left == 0) break;
          j0 = next_slot4();
          s0 = stage[j0];
          step(clamp_t, s1, j1);
          if (--left == 0) break;
        }
      };
      const uint64_t staged = wc[0] | wc[1] | wc[2] | wc[3];
      if (bclamp)
        walk(std::true_type{});
      else
        walk(std::false_type{});
      wave_sync();
      pend = staged;
      buf ^= 1;
      if (mn < 0) break;
      mc = mn;
      mn = mnn;
    }
  }
  if (pend) flush<WIDE>(pend, rows2 + BATCH * (buf ^ 1), gacc2 + 9 * SLOTS * (buf ^ 1), grads);
}

// WIDE: the gradient array is larger than 32-bit byte offsets reach (n above
// 119M), so the atomics take 64-bit addresses.
template <bool WIDE>
__global__ void __launch_bounds__(GS_WAVE * GS_WAVES_PER_BLOCK)
__attribute__((amdgpu_waves_per_eu(4))) k_render_bwd(
    const Splat *__restrict__ splats, int n, const int32_t *__restrict__ sorted_ids,
    const int2 *__restrict__ ranges, CamK cam, const float *__restrict__ Tfin,
    const int32_t *__restrict__ last, char *__restrict__ state, int ntiles,
    const float *__restrict__ dL, const float *__restrict__ dT, float *__restrict__ grads,
    const int32_t *__restrict__ status) {
  __shared__ Staged stage_all[GS_WAVES_PER_BLOCK][SLOTS];
  // per-slot gradient sums and gradient rows, two sets per wave
  __shared__ float gacc_all[GS_WAVES_PER_BLOCK][2 * 9 * SLOTS];
  __shared__ int32_t rows_all[GS_WAVES_PER_BLOCK][2 * BATCH];
  Staged *stage = stage_all[wave_in_block()];
  float *gacc = gacc_all[wave_in_block()];
  int32_t *rows = rows_all[wave_in_block()];
  FwdState fs = fwd_state_at(state, ntiles);
  const int bc = bin_count(fs);
  // the frame failed earlier: nothing to differentiate
  if (!fs.hdr->run_f || *status != GS_OK) return;
  // bins: the forward filed the items (frames with few tiles: the preparation
  // wrote bitems)
  const bool bins = fs.hdr->bmode != 0;
  __shared__ int bpre[GS_GROUPS * BPRE];
  if (bins) bin_starts(bc, bpre);
  for (int i = __lane_id(); i < 2 * 9 * SLOTS; i += GS_WAVE) gacc[i] = 0.0f;
  if (__lane_id() == 0) {
    Staged dead;
    dead.p0 = dead.p1 = dead.p2 = make_float4(0.f, 0.f, 0.f, 0.f);
    dead.p2.y = -1.0f;  // tau < 0: q <= tau never holds
    stage[BATCH] = dead;
  }
  fs.nw = fs.hdr->nw;
  const int k = fs.hdr->k;
  const int64_t P = (int64_t)cam.width * cam.height * cam.views;
  const int lane = __lane_id();
  // row q of the wave: quarter q of the tile; lane s of the row: column s mod 8,
  // rows 4 (s / 8) to 4 (s / 8) + 3 of the quarter
  const int quad = lane >> 4, col = lane & 7, r4 = 4 * ((lane >> 3) & 1);
  __shared__ uint32_t drained;
  __shared__ int waves_out;
  if (threadIdx.x == 0) waves_out = 0;
  Worker wk = make_worker(&drained);
  for (;;) {
    int it;
    if (bins) {
      if (!next_bin_item(fs, bpre, wk, gridDim.x, it)) break;
    } else {
      const int t = next_item(fs, 1, wk);
      if (t < 0) break;
      it = fs.bitems[t];
    }
    wk.round++;
    const int kind = item_kind(it), p = item_chunk(it);
    const int idx = item_index(it);
    const bool plain = kind == ITEM_PLAIN || kind == ITEM_QUARTER;
    const int tile = plain ? idx : fs.order[idx];
    // the quarters the item covers; the other rows have no pixels and no entries
    const uint32_t qm = kind == ITEM_PLAIN ? 0xFu : 1u << item_quad(it);
    const bool row_on = (qm >> quad) & 1u;
    const SubTile st = subtile_of(tile, quad, cam);  // this lane's quarter
    const int px = st.x0 + col;
    const int2 rg = ranges[tile];
    Pix4 x;
    x.fx = (float)px + 0.5f;
    bool in[4];
    int64_t pix[4];
    float ex[4];  // bg . dL/dC + dL/dT_final: what lies behind the last splat, per unit T
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int py = st.y0 + r4 + r;
      x.fy[r] = (float)py + 0.5f;
      in[r] = row_on && px < cam.width && py < cam.height;
      pix[r] = (int64_t)(st.prow + py) * cam.width + px;
      x.g[r][0] = x.g[r][1] = x.g[r][2] = 0.0f;
      ex[r] = 0.0f;
      if (in[r]) {
        x.g[r][0] = dL[pix[r]];
        x.g[r][1] = dL[P + pix[r]];
        x.g[r][2] = dL[2 * P + pix[r]];
        if (cam.bg_on) {
          ex[r] = fmaf(cam.bg[0], x.g[r][0], fmaf(cam.bg[1], x.g[r][1], cam.bg[2] * x.g[r][2]));
          if (dT) ex[r] += dT[pix[r]];
        }
      }
    }
    int nbw[4];
    if (plain) {
#pragma unroll
      for (int r = 0; r < 4; r++) {
        x.T[r] = in[r] ? Tfin[pix[r]] : 1.0f;
        x.last[r] = in[r] ? last[pix[r]] : 0;
        x.acc[r] = ex[r];
      }
      int nb = 0;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        nbw[q] = (qm >> q) & 1u ? ceil64(fs.sub_last[tile * 4 + q]) : 0;
        nb = max(nb, nbw[q]);
      }
      // piece p - 1 of the walk: batches [a, e); one that ends at a cut starts
      // from the forward pass's state there, in the quarters whose walk reached it
      int a = 0;
      if (p > 0) {
        int e;
        piece_range(p - 1, nb, a, e);
        const int c = p - 1;
        const int qc = row_on ? fs.qcut[tile * 4 + quad] : 0;
        if (e < nb && qc > c) {
          const float *cr = fs.cut + (size_t)tile * GS_CUT_FLOATS + 64 * quad + col + 8 * r4;
#pragma unroll
          for (int r = 0; r < 4; r++) {
            if (!in[r]) continue;
            const float *cp = cr + 8 * r;
            const float Tc = cp[4 * 256 * c];
            // the colour behind the cut: the segment after the last cut
            // reached, then those that end at cuts c + 1 .. qc - 1
            float cb[3];
#pragma unroll
            for (int ch = 0; ch < 3; ch++) cb[ch] = cp[4 * 256 * GS_NCUT + 256 * ch];
#pragma unroll
            for (int s2 = GS_NCUT - 1; s2 > 0; s2--)
              if (s2 > c && s2 < qc) {
#pragma unroll
                for (int ch = 0; ch < 3; ch++) cb[ch] += cp[4 * 256 * s2 + 256 * (ch + 1)];
              }
            float behind = __builtin_fmaf(cb[0], x.g[r][0],
                                          __builtin_fmaf(cb[1], x.g[r][1], cb[2] * x.g[r][2]));
            behind = __builtin_fmaf(x.T[r], ex[r], behind);
            // a pixel still blending at the cut has consumed every entry before it
            if (Tc >= 1e-4f) x.last[r] = 64 * e;
            x.acc[r] = behind / Tc;
            x.T[r] = Tc;
          }
        }
#pragma unroll
        for (int q = 0; q < 4; q++) nbw[q] = max(0, min(nbw[q], e) - a);
#pragma unroll
        for (int r = 0; r < 4; r++) x.last[r] -= 64 * a;
      }
      walk_back<WIDE>(splats, n, sorted_ids, rg.x + 64 * a, contrib_base(fs, 0, tile, rg.x) + a,
                      fs.nw, nbw, x, stage, gacc, rows, grads);
      continue;
    }
    // a chunk of a heavy tile: the lane's pixels are positions ql + 8 r of its
    // quarter's chunk state
    int cs, ce;
    chunk_range(rg.x, rg.y, p, k, cs, ce);
    const int ql = col + 8 * r4;
    const int ci = chunk_index(idx, p, quad, k);
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int64_t cp = (int64_t)ci * 64 + ql + 8 * r;
      int lb = in[r] ? fs.LB[cp] : -1;
      float Tc = 1.0f, ac = 0.0f;
      if (lb > 0) {
        Tc = fs.TB[cp];
        float behind = 0.0f;  // sum over later chunks of C . dL/dC
        for (int q2 = p + 1; q2 < k; q2++) {
          const int64_t c2 = (int64_t)chunk_index(idx, q2, quad, k) * 64 + ql + 8 * r;
          if (fs.LB[c2] < 0) break;
          behind = __builtin_fmaf(fs.CB[3 * c2], x.g[r][0],
                                  __builtin_fmaf(fs.CB[3 * c2 + 1], x.g[r][1],
                                                 __builtin_fmaf(fs.CB[3 * c2 + 2], x.g[r][2], behind)));
        }
        if (cam.bg_on) behind = fmaf(Tfin[pix[r]], ex[r], behind);
        ac = behind / Tc;
      } else {
        lb = 0;
      }
      x.T[r] = Tc;
      x.acc[r] = ac;
      x.last[r] = lb;
    }
#pragma unroll
    for (int q = 0; q < 4; q++)
      nbw[q] = (qm >> q) & 1u ? ceil64(fs.chunk_last[chunk_index(idx, p, q, k)]) : 0;
    walk_back<WIDE>(splats, n, sorted_ids, cs, contrib_base(fs, 0, tile, rg.x) + ((cs - rg.x) >> 6),
                    fs.nw, nbw, x, stage, gacc, rows, grads);
  }
  // The last wave out of the launch resets the bins' queue heads, so the
  // backward may run again on this state (every other wave has made its last
  // pop). A frame with few tiles has its heads set by its preparation, which
  // runs before every backward launch.
  if (bins && lane == 0 && atomicAdd(&waves_out, 1) == GS_WAVES_PER_BLOCK - 1 &&
      atomicAdd(&fs.hdr->bexit, 1) == (int)gridDim.x - 1) {
    for (int g = 0; g < GS_GROUPS; g++) queue_head(fs, 1, g)[0] = 0;
    fs.hdr->bexit = 0;
  }
}

// The overwritten gradient array's zeroing, for frames whose backward has no
// preparation.
__global__ void __launch_bounds__(256) k_zero(float *__restrict__ out, int64_t nout) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n4 = nout / 4;
  if (i < n4) reinterpret_cast<float4 *>(out)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i < nout - 4 * n4) out[4 * n4 + i] = 0.0f;
}

}  // namespace

hipError_t gs_launch_render_bwd(int n, const float *splats, const int32_t *sorted_ids,
                                const int32_t *ranges, const CamK &cam, const float *T,
                                const int32_t *last, void *fwd_state, const float *dL,
                                const float *dT, float *grads, bool accumulate, int32_t *status,
                                int workers_waves, hipEvent_t ev0, hipEvent_t ev1,
                                hipStream_t st) {
  const int64_t ng = 9 * (int64_t)n;
  const int ntiles = cam.tiles_x * cam.tiles_y;
  const int nblocks = workers_waves / GS_WAVES_PER_BLOCK;
  // accumulating: the caller's gradient array is the starting point, not zeroed
  // A frame with few tiles has its backward items ordered (and its long walks
  // cut) by the preparation, beside the zeroing; any other frame's forward
  // filed them, and only the zeroing remains.
  if (few_tiles(ntiles, nblocks)) {
    const int zero_blocks = accumulate ? 0 : (int)((ng / 4 + 4 + BO_T - 1) / BO_T);
    hipLaunchKernelGGL(k_bwd_prep<true>, dim3(GS_GROUPS + zero_blocks), dim3(BO_T), 0, st,
                       reinterpret_cast<char *>(fwd_state), ntiles, nblocks, grads, ng, status);
  } else if (!accumulate && ng > 0) {
    hipLaunchKernelGGL(k_zero, dim3(gs_div_up(ng / 4 + 4, 256)), dim3(256), 0, st, grads, ng);
  }
  if (ev0) {
    const hipError_t e = hipEventRecord(ev0, st);
    if (e != hipSuccess) return e;
  }
  const bool wide = 36 * (int64_t)n >= (int64_t)UINT32_MAX - 64;
  hipLaunchKernelGGL(wide ? k_render_bwd<true> : k_render_bwd<false>, dim3(nblocks),
                     dim3(GS_WAVE * GS_WAVES_PER_BLOCK), 0, st,
                     reinterpret_cast<const Splat *>(splats), n, sorted_ids,
                     reinterpret_cast<const int2 *>(ranges), cam, T, last,
                     reinterpret_cast<char *>(fwd_state), ntiles, dL, dT, grads, status);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev1) e = hipEventRecord(ev1, st);
  return e;
}
