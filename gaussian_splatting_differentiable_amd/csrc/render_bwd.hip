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
// adjacent pixels per lane, sharing the column terms of q and summed in
// registers before the reduction; Step 6.3 the per-splat term
// alpha T (c . dL/dC - accum), with log2(o) folded into the exponent and o
// divided back out once after the sum; Step 6.4 the two rows' offsets combined
// without per-row products by the row index.
// "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on GPUs",
// section 4: the same persistent longest-first queue as the forward pass; a
// chunk of a heavy tile is differentiated on its own from the forward pass's
// chunk state: it starts from the transmittance after its last processed
// splat, T_end, with accum = (sum over later chunks of C_chunk . dL/dC) / T_end.
//
// gfx950 mapping: one wavefront per item, an 8-column half of a tile (or of a
// chunk): lane l holds column l mod 8 and rows 2 (l / 8), 2 (l / 8) + 1, so
// lanes 0-31 cover the half's upper quarter and lanes 32-63 its lower one. The
// item's non-empty batches come from one vector load of its contributor words;
// each batch stages only its contributors' records in LDS (the next batch's
// ids and records in flight) and walks them back to front on the scalar unit.
#include <type_traits>

#include "render_common.h"
#include "wave_reduce.h"

namespace {

constexpr float NEG_HALF_LOG2E = -0.72134752044448170368f;

// Backward queue order. The forward pass leaves every item's walk length (the
// quarter's or chunk's last hit), so the backward can serve its items longest
// first exactly ([LOAD-IMB] section 4.1 orders by N_t, which overstates the work
// of tiles whose pixels saturate early). One workgroup per group sorts the
// group's backward items stably by a quarter-octave bucket of that length.
constexpr int BO_T = 1024, BO_W = BO_T / 64, BO_BITS = 6, BO_BINS = 1 << BO_BITS;

// Walk length of a backward item: the longer of its two quarters' last hits.
__device__ __forceinline__ int item_len(const FwdState &fs, int it, int k) {
  const int half = item_quad(it), idx = item_index(it);
  if (item_kind(it) == ITEM_PLAIN)
    return max(fs.sub_last[idx * 4 + half], fs.sub_last[idx * 4 + half + 2]);
  const int p = item_chunk(it);
  return max(fs.chunk_last[chunk_index(idx, p, half, k)],
             fs.chunk_last[chunk_index(idx, p, half + 2, k)]);
}

__device__ __forceinline__ uint32_t order_bin(int len) {
  const int b = (int)(4.0f * __log2f((float)max(len, 0) + 1.0f));
  return (uint32_t)(BO_BINS - 1 - min(b, BO_BINS - 1));  // ascending bin = longest first
}

// The backward's preparation in one launch: workgroup g < GS_GROUPS builds group
// g's backward queue: the forward's plain and pass-B items of quarters 0 and 1
// become the left and right halves (each covers quarters h and h + 2), stably
// sorted longest first; the others zero the gradient output. The frame runs only
// if its status is still GS_OK.
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
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < BO_W * BO_BINS; i += BO_T) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int chunk = (n + BO_W - 1) / BO_W;
  const int c0 = min(n, w * chunk), c1 = min(n, c0 + chunk);
  for (int e = c0 + lane; e < c1; e += 64) {
    const int it = fs.items[lo + e];
    if (item_quad(it) < 2) atomicAdd(&cnt[w][order_bin(item_len(fs, it, k))], 1);
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
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int base = c0; base < c1; base += 64) {
    const int e = base + lane;
    const int it = e < c1 ? fs.items[lo + e] : 0;
    const bool valid = e < c1 && item_quad(it) < 2;
    const uint32_t d = valid ? order_bin(item_len(fs, it, k)) : 0u;
    uint64_t peers = wave_ballot(valid);
#pragma unroll
    for (int b = 0; b < BO_BITS; b++) {
      const uint64_t bal = wave_ballot((d >> b) & 1u);
      peers &= ((d >> b) & 1u) ? bal : ~bal;
    }
    if (valid) {
      const int below = __popcll(peers & lt);
      const int pos = cnt[w][d] + below;
      fs.bitems[lo + pos] = it;
      if (below == __popcll(peers) - 1) cnt[w][d] = pos + 1;
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

// A staged entry (64 bytes): the record with 2b, log2(o) and 1/o in place of
// depth, pad and o, and the splat id. Slot 64 of a wave's stage is a dead
// entry (tau = -1, never hit) that a half with no entry left reads.
struct __align__(16) Staged {
  float4 p0;  // mx, my, a, b
  float4 p1;  // c, 1/o, r, g
  float4 p2;  // b (colour), tau, 2b, log2(o)
  int4 p3;    // id, live (1) or dead (0), -, -
};
constexpr int SLOTS = BATCH + 1;

__device__ __forceinline__ int top_bit(uint64_t w) { return w ? 63 - __builtin_clzll(w) : BATCH; }
__device__ __forceinline__ bool has_bit(uint64_t w, int j) { return j < BATCH && ((w >> j) & 1ull); }

// The next step of a batch's walk: the entries the upper and lower quarter take
// (BATCH, the dead slot, for none), removed from their words. Each quarter
// takes its own entries back to front. An entry both quarters blended is taken
// by both in the same step (shared: the halves' sums are added and written
// once); otherwise the higher entry goes to its quarter, and the other quarter
// takes its own next entry in the same step unless that entry is still to come
// for the first quarter too (then it waits, so that the two meet on it).
struct Pair {
  int jt, jb;
  bool shared;
};
__device__ __forceinline__ Pair next_pair(uint64_t &wt, uint64_t &wb) {
  Pair p;
  const int ht = top_bit(wt), hb = top_bit(wb);
  p.shared = ht == hb && ht < BATCH;
  if (p.shared || ht > hb) {
    p.jt = ht;
    p.jb = p.shared ? hb : (has_bit(wt, hb) ? BATCH : hb);
  } else {
    p.jb = hb;
    p.jt = has_bit(wb, ht) ? BATCH : ht;
  }
  if (p.jt < BATCH) wt &= ~(1ull << p.jt);
  if (p.jb < BATCH) wb &= ~(1ull << p.jb);
  return p;
}

// Per-lane state of the two pixels of a lane (rows 0 and 1 of its pair).
struct Pix2 {
  float fx, fy0, fy1;        // sample positions
  float T0, T1, acc0, acc1;  // transmittance after the pixel's last entry; accumulator
  float g00, g01, g02, g10, g11, g12;  // dL/dC of the two pixels
  int last0, last1;          // entries the pixel consumed from the walk's start
};

// Walk the item's batches back to front. cw_top / cw_bot: the contributor words
// of the two quarters at the walk's first batch; nb_top / nb_bot: how many of
// them are current (the rest were not written for this frame); list: the walk's
// first list position. Lanes 0-31 (the upper quarter) and 32-63 (the lower
// one) take the entries of their own quarter's word, back to front (next_pair):
// a step evaluates one splat for both halves or two different splats, one per
// half, and a half with no entry in the step reads the dead slot.
template <bool WIDE>
__device__ __forceinline__ void walk_back(const Splat *__restrict__ splats, int n,
                                          const int32_t *__restrict__ sids, int64_t list,
                                          const uint64_t *__restrict__ cw_top, int nb_top,
                                          const uint64_t *__restrict__ cw_bot, int nb_bot,
                                          Pix2 &x, Staged *stage, float *__restrict__ grads) {
  const int lane = __lane_id();
  const bool top = lane < 32;
  const int upper = top ? 1 : 0;
  const int comp = comp_of_half_lane(lane);
  const int comp4 = 4 * comp;
  // the constant factor each owner lane applies to its sum after the reduction
  // (powers of two: exact): -1/2 for the two squared offsets
  const float post = (comp == 2 || comp == 4) ? -0.5f : 1.0f;
  float zero = 0.0f;
  __asm__ volatile("" : "+v"(zero));  // a register, not a constant, for the unpaired swap
  const float4 *rec4 = reinterpret_cast<const float4 *>(splats);
  // the next batch's record of this lane, as three registers of four (kept out
  // of any aggregate: the compiler parks part of one in memory otherwise)
  float4 q0 = make_float4(0.f, 0.f, 0.f, 0.f), q1 = q0, q2 = q0;
  const int nbat = max(nb_top, nb_bot);
  for (int r0 = (nbat - 1) & ~63; r0 >= 0; r0 -= 64) {
    // lane i holds the words of batch r0 + i, one per quarter
    const int m = r0 + lane;
    const uint64_t wtv = m < nb_top ? cw_top[m] : 0ull;
    const uint64_t wbv = m < nb_bot ? cw_bot[m] : 0ull;
    const uint32_t tlo = (uint32_t)wtv, thi = (uint32_t)(wtv >> 32);
    const uint32_t blo = (uint32_t)wbv, bhi = (uint32_t)(wbv >> 32);
    uint64_t todo = wave_ballot((wtv | wbv) != 0);
    if (!todo) continue;
    // pipeline: the records of the batch being staged and the ids of the next
    // non-empty batch are in flight while a batch is walked
    int mc = 63 - __builtin_clzll(todo);
    todo &= ~(1ull << mc);
    uint64_t wt = word_of(tlo, thi, mc), wb = word_of(blo, bhi, mc);
    int idc = load_marked_id(sids, list + 64 * (int64_t)(r0 + mc), wt | wb);
    {
      const int64_t ri = 3 * (int64_t)(valid_id(idc, n) ? idc : 0);
      q0 = rec4[ri];
      q1 = rec4[ri + 1];
      q2 = rec4[ri + 2];
    }
    int mn = -1, idn = -1;
    uint64_t wtn = 0, wbn = 0;
    if (todo) {
      mn = 63 - __builtin_clzll(todo);
      todo &= ~(1ull << mn);
      wtn = word_of(tlo, thi, mn);
      wbn = word_of(blo, bhi, mn);
      idn = load_marked_id(sids, list + 64 * (int64_t)(r0 + mn), wtn | wbn);
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
        // the gradient row's byte offset (rows of 36 bytes; only when it fits)
        stage[lane].p3 = make_int4(idc, valid_id(idc, n) ? 1 : 0, WIDE ? 0 : (int)(36u * (uint32_t)idc), 0);
      }
      // records of the next batch, ids of the one after it
      idc = idn;
      {
        const int64_t rj = 3 * (int64_t)(valid_id(idc, n) ? idc : 0);
        q0 = rec4[rj];
        q1 = rec4[rj + 1];
        q2 = rec4[rj + 2];
      }
      int mnn = -1;
      uint64_t wtnn = 0, wbnn = 0;
      idn = -1;
      if (todo) {
        mnn = 63 - __builtin_clzll(todo);
        todo &= ~(1ull << mnn);
        wtnn = word_of(tlo, thi, mnn);
        wbnn = word_of(blo, bhi, mnn);
        idn = load_marked_id(sids, list + 64 * (int64_t)(r0 + mnn), wtnn | wbnn);
      }
      wave_sync();
      const int base = 64 * (r0 + mc);
      // a pixel takes entry j only below its own stop: j < last - base, here
      // on the slot's byte offset in the stage, 64 j (the dead slot, j = 64,
      // never hits)
      const int lim0 = 64 * (x.last0 - base), lim1 = 64 * (x.last1 - base);
      auto step = [&](auto clamp_t, const Staged &s, int j, bool shared) {
        constexpr bool CLAMP = decltype(clamp_t)::value;
        const float a = s.p0.z, b = s.p0.w, c = s.p1.x;
        // the column terms of the canonical q are shared by the lane's two rows
        const float dx = x.fx - s.p0.x;
        const float adx = a * dx;
        const float adxdx = adx * dx, b2dx = s.p2.z * dx;
        const float dy0 = x.fy0 - s.p0.y, dy1 = x.fy1 - s.p0.y;
        const float cdy0 = c * dy0, cdy1 = c * dy1;
        const float qa = __builtin_fmaf(cdy0, dy0, __builtin_fmaf(b2dx, dy0, adxdx));
        const float qb = __builtin_fmaf(cdy1, dy1, __builtin_fmaf(b2dx, dy1, adxdx));
        const bool h0 = j < lim0 && qa <= s.p2.y;  // j: the slot's byte offset
        const bool h1 = j < lim1 && qb <= s.p2.y;
        // branchless: a missed pixel takes alpha = 0, which leaves T and accum
        // unchanged and contributes zero to every sum
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(qa, NEG_HALF_LOG2E, s.p2.w));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(qb, NEG_HALF_LOG2E, s.p2.w));
        const float oG0 = h0 ? e0 : 0.0f, oG1 = h1 ? e1 : 0.0f;  // o G
        const float al0 = CLAMP ? fminf(0.99f, oG0) : oG0;
        const float al1 = CLAMP ? fminf(0.99f, oG1) : oG1;
        x.T0 = x.T0 * __builtin_amdgcn_rcpf(1.0f - al0);  // T before this splat
        x.T1 = x.T1 * __builtin_amdgcn_rcpf(1.0f - al1);
        const float cg0 = __builtin_fmaf(s.p1.z, x.g00, __builtin_fmaf(s.p1.w, x.g01, s.p2.x * x.g02));
        const float cg1 = __builtin_fmaf(s.p1.z, x.g10, __builtin_fmaf(s.p1.w, x.g11, s.p2.x * x.g12));
        const float d0 = cg0 - x.acc0, d1 = cg1 - x.acc1;  // dL/dalpha = T d
        x.acc0 = __builtin_fmaf(al0, d0, x.acc0);
        x.acc1 = __builtin_fmaf(al1, d1, x.acc1);
        const float w0 = al0 * x.T0, w1 = al1 * x.T1;
        // -2 dL/dq = alpha T d, which is also o G dL/dalpha: an unclamped alpha
        // is o G; a clamped alpha passes no gradient
        const float m0 = !CLAMP || oG0 < 0.99f ? w0 * d0 : 0.0f;
        const float m1 = !CLAMP || oG1 < 0.99f ? w1 * d1 : 0.0f;
        // the lane's two rows, dy1 = dy0 + 1: with M = m0 + m1,
        // Sy = m0 dy0 + m1 dy1 = M dy0 + m1 and Syy = m0 dy0^2 + m1 dy1^2 =
        // dy0 (Sy + m1) + m1, and X = M dx, each derivative needs dx once
        const float M = m0 + m1;
        const float Sy = __builtin_fmaf(M, dy0, m1);
        const float X = M * dx;
        float gr[9];
        gr[0] = __builtin_fmaf(a, X, b * Sy);  // dq/dmx = -2 (a dx + b dy)
        gr[1] = __builtin_fmaf(b, X, c * Sy);  // dq/dmy = -2 (b dx + c dy)
        gr[2] = X * dx;                        // times -1/2 after the sum
        gr[3] = -(dx * Sy);
        gr[4] = __builtin_fmaf(dy0, Sy + m1, m1);  // times -1/2 after the sum
        gr[5] = M;                                 // divided by o after the sum
        gr[6] = __builtin_fmaf(w1, x.g10, w0 * x.g00);
        gr[7] = __builtin_fmaf(w1, x.g11, w0 * x.g01);
        gr[8] = __builtin_fmaf(w1, x.g12, w0 * x.g02);
        float out = reduce_scatter9_half(gr, zero);
        // one splat in both halves: add the lower half's sums to the upper's
        // (the owners sit at the same place in both halves), written once
        if (shared) out = swap_sum32(out, out);
        // finish the sum here, where its last exchange fuses into the add,
        // rather than inside the owner lanes' branch
        __asm__ volatile("" : "+v"(out));
        out *= comp == 5 ? s.p1.y : post;
        if (comp >= 0 && s.p3.y && (top || !shared)) {
          if constexpr (WIDE)
            unsafeAtomicAdd(&grads[9 * (int64_t)s.p3.x + comp], out);
          else
            unsafeAtomicAdd(reinterpret_cast<float *>(reinterpret_cast<char *>(grads) +
                                                      ((uint32_t)s.p3.z + (uint32_t)comp4)),
                            out);
        }
      };
      // the next step's reads from the stage go out before the current step
      // runs (two buffers alternate)
      // a lane's slot is jt in the upper half and jb in the lower one: its
      // byte offset 64 jb + upper (64 (jt - jb)), one 24-bit multiply-add on
      // the vector unit (the rest is scalar)
      const char *stage_b = reinterpret_cast<const char *>(stage);
      auto slot_off = [&](const Pair &p) {
        int t;
        __asm__("v_mul_i32_i24 %0, %1, %2" : "=v"(t) : "s"(64 * (p.jt - p.jb)), "v"(upper));
        return t + 64 * p.jb;
      };
      auto at = [&](int off) { return *reinterpret_cast<const Staged *>(stage_b + off); };
      auto walk = [&](auto clamp_t) {
        Pair pc = next_pair(wt, wb);
        int j0 = slot_off(pc);
        bool sh0 = pc.shared;
        Staged s0 = at(j0);
        for (;;) {
          const bool more1 = (wt | wb) != 0;
          pc = next_pair(wt, wb);
          const int j1 = slot_off(pc);
          const bool sh1 = pc.shared;
          const Staged s1 = at(j1);
          step(clamp_t, s0, j0, sh0);
          if (!more1) break;
          const bool more0 = (wt | wb) != 0;
          pc = next_pair(wt, wb);
          j0 = slot_off(pc);
          sh0 = pc.shared;
          s0 = at(j0);
          step(clamp_t, s1, j1, sh1);
          if (!more0) break;
        }
      };
      if (bclamp)
        walk(std::true_type{});
      else
        walk(std::false_type{});
      wave_sync();
      if (mn < 0) break;
      mc = mn;
      wt = wtn;
      wb = wbn;
      mn = mnn;
      wtn = wtnn;
      wbn = wbnn;
    }
  }
}

__device__ __forceinline__ int ceil64(int v) { return (max(v, 0) + 63) >> 6; }

// WIDE: the gradient array is larger than 32-bit byte offsets reach (n above
// 119M), so the atomics take 64-bit addresses.
template <bool WIDE>
__global__ void __launch_bounds__(GS_WAVE * GS_WAVES_PER_BLOCK)
__attribute__((amdgpu_waves_per_eu(4))) k_render_bwd(
    const Splat *__restrict__ splats, int n, const int32_t *__restrict__ sorted_ids,
    const int2 *__restrict__ ranges, CamK cam, const float *__restrict__ Tfin,
    const int32_t *__restrict__ last, char *__restrict__ state, int ntiles,
    const float *__restrict__ dL, const float *__restrict__ dT, float *__restrict__ grads) {
  __shared__ Staged stage_all[GS_WAVES_PER_BLOCK][SLOTS];
  Staged *stage = stage_all[wave_in_block()];
  FwdState fs = fwd_state_at(state, ntiles);
  if (!fs.hdr->run_b) return;  // the frame failed earlier: nothing to differentiate
  if (__lane_id() == 0) {
    Staged dead;
    dead.p0 = dead.p1 = dead.p2 = make_float4(0.f, 0.f, 0.f, 0.f);
    dead.p2.y = -1.0f;  // tau < 0: q <= tau never holds
    dead.p3 = make_int4(0, 0, 0, 0);
    stage[BATCH] = dead;
  }
  fs.nw = fs.hdr->nw;
  const int k = fs.hdr->k;
  const int64_t P = (int64_t)cam.width * cam.height * cam.views;
  const int lane = __lane_id();
  const int col = lane & 7, rp = lane >> 3;
  __shared__ uint32_t drained;
  Worker wk = make_worker(&drained);
  for (;;) {
    const int t = next_item(fs, 1, wk);
    if (t < 0) break;
    wk.round++;
    const int it = fs.bitems[t];
    const int kind = item_kind(it), half = item_quad(it), p = item_chunk(it);
    const int idx = item_index(it);
    const int tile = kind == ITEM_PLAIN ? idx : fs.order[idx];
    const SubTile st = subtile_of(tile, half, cam);  // the half's upper quarter
    if (st.empty) continue;
    const int px = st.x0 + col, py0 = st.y0 + 2 * rp, py1 = py0 + 1;
    const bool in0 = px < cam.width && py0 < cam.height;
    const bool in1 = px < cam.width && py1 < cam.height;
    const int64_t pix0 = (int64_t)(st.prow + py0) * cam.width + px;
    const int64_t pix1 = pix0 + cam.width;
    const int2 rg = ranges[tile];
    Pix2 x;
    x.fx = (float)px + 0.5f;
    x.fy0 = (float)py0 + 0.5f;
    x.fy1 = (float)py1 + 0.5f;
    x.g00 = x.g01 = x.g02 = x.g10 = x.g11 = x.g12 = 0.f;
    // what lies behind the last blended splat, per unit of final transmittance:
    // the background's bg . dL/dC and dL/dT_final (0 when neither is given)
    float ex0 = 0.f, ex1 = 0.f;
    if (in0) {
      x.g00 = dL[pix0];
      x.g01 = dL[P + pix0];
      x.g02 = dL[2 * P + pix0];
      if (cam.bg_on) {
        ex0 = fmaf(cam.bg[0], x.g00, fmaf(cam.bg[1], x.g01, cam.bg[2] * x.g02));
        if (dT) ex0 += dT[pix0];
      }
    }
    if (in1) {
      x.g10 = dL[pix1];
      x.g11 = dL[P + pix1];
      x.g12 = dL[2 * P + pix1];
      if (cam.bg_on) {
        ex1 = fmaf(cam.bg[0], x.g10, fmaf(cam.bg[1], x.g11, cam.bg[2] * x.g12));
        if (dT) ex1 += dT[pix1];
      }
    }
    const int qtop = half, qbot = half + 2;
    if (kind == ITEM_PLAIN) {
      x.T0 = in0 ? Tfin[pix0] : 1.0f;
      x.T1 = in1 ? Tfin[pix1] : 1.0f;
      x.last0 = in0 ? last[pix0] : 0;
      x.last1 = in1 ? last[pix1] : 0;
      x.acc0 = ex0;
      x.acc1 = ex1;
      walk_back<WIDE>(splats, n, sorted_ids, rg.x, contrib_base(fs, qtop, tile, rg.x),
                ceil64(fs.sub_last[tile * 4 + qtop]), contrib_base(fs, qbot, tile, rg.x),
                ceil64(fs.sub_last[tile * 4 + qbot]), x, stage, grads);
      continue;
    }
    // a chunk of a heavy tile: the lane's two pixels lie in one quarter, at
    // positions ql and ql + 8 of that quarter's chunk state
    int cs, ce;
    chunk_range(rg.x, rg.y, p, k, cs, ce);
    const int q = rp < 4 ? qtop : qbot;
    const int ql = col + 8 * ((2 * rp) & 7);
    const int ci = chunk_index(idx, p, q, k);
    float Tc[2] = {1.0f, 1.0f}, ac[2] = {0.f, 0.f};
    int lc[2] = {0, 0};
    const bool inr[2] = {in0, in1};
    const float exr[2] = {ex0, ex1};
    const int64_t pixr[2] = {pix0, pix1};
    const float gr0[2] = {x.g00, x.g10}, gr1[2] = {x.g01, x.g11}, gr2[2] = {x.g02, x.g12};
#pragma unroll
    for (int r = 0; r < 2; r++) {
      const int64_t cp = (int64_t)ci * 64 + ql + 8 * r;
      int lb = inr[r] ? fs.LB[cp] : -1;
      if (lb > 0) {
        Tc[r] = fs.TB[cp];
        float behind = 0.0f;  // sum over later chunks of C . dL/dC
        for (int q2 = p + 1; q2 < k; q2++) {
          const int64_t c2 = (int64_t)chunk_index(idx, q2, q, k) * 64 + ql + 8 * r;
          if (fs.LB[c2] < 0) break;
          behind = __builtin_fmaf(fs.CB[3 * c2], gr0[r],
                                  __builtin_fmaf(fs.CB[3 * c2 + 1], gr1[r],
                                                 __builtin_fmaf(fs.CB[3 * c2 + 2], gr2[r], behind)));
        }
        if (cam.bg_on) behind = fmaf(Tfin[pixr[r]], exr[r], behind);
        ac[r] = behind / Tc[r];
      } else {
        lb = 0;
      }
      lc[r] = lb;
    }
    x.T0 = Tc[0];
    x.T1 = Tc[1];
    x.acc0 = ac[0];
    x.acc1 = ac[1];
    x.last0 = lc[0];
    x.last1 = lc[1];
    const uint64_t *cw0 = contrib_base(fs, qtop, tile, rg.x) + ((cs - rg.x) >> 6);
    const uint64_t *cw1 = contrib_base(fs, qbot, tile, rg.x) + ((cs - rg.x) >> 6);
    walk_back<WIDE>(splats, n, sorted_ids, cs, cw0, ceil64(fs.chunk_last[chunk_index(idx, p, qtop, k)]),
              cw1, ceil64(fs.chunk_last[chunk_index(idx, p, qbot, k)]), x, stage, grads);
  }
}

}  // namespace

hipError_t gs_launch_render_bwd(int n, const float *splats, const int32_t *sorted_ids,
                                const int32_t *ranges, const CamK &cam, const float *T,
                                const int32_t *last, void *fwd_state, const float *dL,
                                const float *dT, float *grads, int32_t *status, int workers_waves,
                                hipEvent_t ev0, hipEvent_t ev1, hipStream_t st) {
  const int64_t ng = 9 * (int64_t)n;
  const int ntiles = cam.tiles_x * cam.tiles_y;
  const int nblocks = workers_waves / GS_WAVES_PER_BLOCK;
  const int zero_blocks = (int)((ng / 4 + 4 + BO_T - 1) / BO_T);
  hipLaunchKernelGGL(k_bwd_prep, dim3(GS_GROUPS + zero_blocks), dim3(BO_T), 0, st,
                     reinterpret_cast<char *>(fwd_state), ntiles, nblocks, grads, ng, status);
  if (ev0) {
    const hipError_t e = hipEventRecord(ev0, st);
    if (e != hipSuccess) return e;
  }
  const bool wide = 36 * (int64_t)n >= (int64_t)UINT32_MAX - 64;
  hipLaunchKernelGGL(wide ? k_render_bwd<true> : k_render_bwd<false>, dim3(nblocks),
                     dim3(GS_WAVE * GS_WAVES_PER_BLOCK), 0, st,
                     reinterpret_cast<const Splat *>(splats), n, sorted_ids,
                     reinterpret_cast<const int2 *>(ranges), cam, T, last,
                     reinterpret_cast<char *>(fwd_state), ntiles, dL, dT, grads);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev1) e = hipEventRecord(ev1, st);
  return e;
}
