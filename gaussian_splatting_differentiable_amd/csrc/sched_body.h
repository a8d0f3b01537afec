// Per-frame tile schedule: longest-processing-time order, the chunking policy
// and the work queues of the persistent raster kernels, as a device function
// for the schedule's own launch (sched.hip) and for the sort's last tile pass,
// which builds it in a spare workgroup (sort.hip).
//
// "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on GPUs":
// section 4.1 orders the tiles by descending pair count N_t (a radix sort of the
// tile indices that leaves the Gaussian data in place); section 4.3 chunks the
// heaviest tiles and schedules the rest in that order; section 4.4, Eq. 6 picks
// the number of chunked tiles h and chunks per tile k per frame. Chunks are
// composed exactly here (a transmittance pass, then a blending pass from the
// exact incoming transmittance), so a split tile is walked twice and the model
// charges that:
//   avg = ((N_total + S_h) + lambda h k) / K,  S_h = N_1 + ... + N_h,
//   l = max(2 N_1 / k, N_{h+1}),  T(h,k) = max(avg, l) + beta l,
// k in {2,4,8,16}, first strict minimum over (k, h), enabled only when at least
// eps below the no-chunking estimate max(N_total / K, N_1) + beta N_1. Here h k
// is also capped at GS_HK_MAX. The policy arithmetic is fp64 in one fixed order
// and every translation unit that includes this file is compiled with
// -ffp-contract=off, so a host copy of the policy returns the same (h, k).
//
// One workgroup of 1024 threads does everything; T <= 65535 tiles, in LDS up to
// 8192 tiles.
#pragma once
#include "render_common.h"

namespace {
namespace sched_impl {

constexpr int NT = 1024, NW = NT / 64;

// Block-wide maximum and sum, in one exchange.
__device__ __forceinline__ void block_max_sum(uint32_t &mx, long long &sum) {
  __shared__ uint32_t wm[NW];
  __shared__ long long wsum[NW];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, d, 64));
    sum += __shfl_xor(sum, d, 64);
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    wm[threadIdx.x >> 6] = mx;
    wsum[threadIdx.x >> 6] = sum;
  }
  __syncthreads();
  mx = 0;
  sum = 0;
#pragma unroll
  for (int w = 0; w < NW; w++) {
    mx = max(mx, wm[w]);
    sum += wsum[w];
  }
  __syncthreads();
}

// Block-wide exclusive prefix sum of one value per thread; `total` gets the sum.
template <typename V>
__device__ __forceinline__ V block_excl_scan(V v, V &total) {
  __shared__ V ws[NW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  V inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const V t = __shfl_up(inc, d, 64);
    if (lane >= d) inc += t;
  }
  __syncthreads();
  if (lane == 63) ws[w] = inc;
  __syncthreads();
  V before = 0, tot = 0;
#pragma unroll
  for (int q = 0; q < NW; q++) {
    const V x = ws[q];
    before += q < w ? x : V(0);
    tot += x;
  }
  total = tot;
  __syncthreads();
  return before + inc - v;
}

// Per-lane register batch of the single-workgroup passes below: a wave loads
// RB_ROUNDS rounds of 64 elements before it uses any of them, so each batch
// costs one global-memory round trip instead of one per round.
constexpr int RB_ROUNDS = 8;

// One stable LSD pass (8-bit digit at `shift`) of (key, val) over n elements in
// global memory, by one workgroup. Wave w owns the contiguous chunk
// [w*chunk, (w+1)*chunk); a first sweep counts digits per wave, a second sweep
// ranks each round of 64 with a ballot match and scatters.
__device__ void block_radix_pass(const uint32_t *__restrict__ kin, const int32_t *__restrict__ vin,
                                 uint32_t *__restrict__ kout, int32_t *__restrict__ vout, int n,
                                 int shift) {
  __shared__ int cnt[NW][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < NW * 256; i += NT) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int chunk = (n + NW - 1) / NW;
  const int c0 = min(n, w * chunk), c1 = min(n, c0 + chunk);
  for (int base = c0; base < c1; base += 64 * RB_ROUNDS) {
    uint32_t kk[RB_ROUNDS];
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++) {
      const int e = base + 64 * r + lane;
      kk[r] = e < c1 ? kin[e] : 0u;
    }
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++)
      if (base + 64 * r + lane < c1) atomicAdd(&cnt[w][(kk[r] >> shift) & 255], 1);
  }
  __syncthreads();
  // offsets in (digit, wave) order: thread t scans the counts of digit t / 4
  // in waves 4 (t % 4) .. 4 (t % 4) + 3, then one block scan joins them
  static_assert(NW * 256 == 4 * NT, "four (digit, wave) counts per thread");
  const int dg = threadIdx.x >> 2, q0 = 4 * (threadIdx.x & 3);
  int cc[4], loc = 0;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    cc[j] = cnt[q0 + j][dg];
    loc += cc[j];
  }
  int all;
  int run = block_excl_scan<int>(loc, all);
#pragma unroll
  for (int j = 0; j < 4; j++) {
    cnt[q0 + j][dg] = run;
    run += cc[j];
  }
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int base = c0; base < c1; base += 64 * RB_ROUNDS) {
    uint32_t kk[RB_ROUNDS];
    int32_t vv[RB_ROUNDS];
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++) {
      const int e = base + 64 * r + lane;
      kk[r] = e < c1 ? kin[e] : 0u;
      vv[r] = e < c1 ? vin[e] : 0;
    }
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++) {
      const bool valid = base + 64 * r + lane < c1;
      const uint32_t d = (kk[r] >> shift) & 255u;
      uint64_t peers = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 8; b++) {
        const uint64_t bal = __ballot((d >> b) & 1u);
        peers &= ((d >> b) & 1u) ? bal : ~bal;
      }
      if (valid) {
        const int below = __popcll(peers & lt);
        const int pos = cnt[w][d] + below;
        kout[pos] = kk[r];
        vout[pos] = vv[r];
        if (below == __popcll(peers) - 1) cnt[w][d] = pos + 1;
      }
    }
  }
  __syncthreads();
}

constexpr int NCLS = 2 * GS_GROUPS;  // (group, chunked?) classes of the LPT positions
constexpr int HMAX = GS_HK_MAX / 2;  // the largest h of any policy candidate
// Frames of up to TL tiles are scheduled in LDS: the sort buffers, the policy's
// prefix sums and the queue partition live in one dynamic LDS block, so the
// workgroup makes a handful of global round trips instead of two per pass.
constexpr int TL = 8192;
constexpr size_t POLICY_BYTES = 8 * (HMAX + 1) + 4 * (HMAX + 1);
constexpr size_t LDS_BYTES = 16 * (size_t)TL;  // four arrays of TL words

// The block's lexicographic minimum of (best, idx), by two LDS atomics on an
// order-preserving 64-bit image of the (non-NaN) doubles.
__device__ __forceinline__ void block_min_idx(double &best, int &idx) {
  __shared__ unsigned long long sb;
  __shared__ int si;
  if (threadIdx.x == 0) {
    sb = ~0ull;
    si = 0x7FFFFFFF;
  }
  __syncthreads();
  const unsigned long long u = (unsigned long long)__double_as_longlong(best);
  const unsigned long long key = (u >> 63) ? ~u : (u | (1ull << 63));
  unsigned long long wmin = key;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const unsigned long long o = __shfl_xor(wmin, d, 64);
    wmin = o < wmin ? o : wmin;
  }
  if ((threadIdx.x & 63) == 0) atomicMin(&sb, wmin);
  __syncthreads();
  if (key == sb) atomicMin(&si, idx);
  __syncthreads();
  const unsigned long long kb = sb;
  best = __longlong_as_double((long long)((kb >> 63) ? (kb & ~(1ull << 63)) : ~kb));
  idx = si;
  __syncthreads();
}

// Stable partition of the LPT positions e in [0, T) by class
// c(e) = 2 group(order[e]) + (e >= h): perm lists the positions class by class,
// each class in LPT order; ccount/cstart get the class sizes and starts.
__device__ void class_partition(const int32_t *order, int T, int h, int tiles_x, int32_t *perm,
                                int *ccount, int *cstart) {
  __shared__ int pc[NW][NCLS];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x < NW * NCLS) (&pc[0][0])[threadIdx.x] = 0;
  __syncthreads();
  const int chunk = (T + NW - 1) / NW;
  const int c0 = min(T, w * chunk), c1 = min(T, c0 + chunk);
  auto cls = [&](int e) { return 2 * tile_group(order[e], tiles_x) + (e >= h ? 1 : 0); };
  for (int e = c0 + lane; e < c1; e += 64) atomicAdd(&pc[w][cls(e)], 1);
  __syncthreads();
  {
    // offsets in (class, wave) order
    static_assert(NCLS * NW <= NT, "one (class, wave) count per thread");
    const int c = threadIdx.x / NW, q = threadIdx.x % NW;
    const bool mine = threadIdx.x < NCLS * NW;
    const int v = mine ? pc[q][c] : 0;
    int all;
    const int ex = block_excl_scan<int>(v, all);
    if (mine) {
      pc[q][c] = ex;
      if (q == 0) cstart[c] = ex;
    }
    __syncthreads();
    if (threadIdx.x < NCLS) {
      const int cc = threadIdx.x;
      ccount[cc] = (cc + 1 < NCLS ? cstart[cc + 1] : T) - cstart[cc];
    }
  }
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int base = c0; base < c1; base += 64) {
    const int e = base + lane;
    const bool valid = e < c1;
    const int c = valid ? cls(e) : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const uint64_t bal = __ballot((c >> b) & 1);
      peers &= ((c >> b) & 1) ? bal : ~bal;
    }
    if (valid) {
      const int below = __popcll(peers & lt);
      const int pos = pc[w][c] + below;
      perm[pos] = e;
      if (below == __popcll(peers) - 1) pc[w][c] = pos + 1;
    }
  }
  __syncthreads();
}

// The plan of a frame that does not run: no items in any queue.
__device__ void empty_plan(const FwdState &fs) {
  if (threadIdx.x <= GS_GROUPS) fs.hdr->qoff[threadIdx.x] = 0;
  if (threadIdx.x < GS_GROUPS) {
    fs.hdr->qa[threadIdx.x] = fs.hdr->init_f[threadIdx.x] = fs.hdr->init_b[threadIdx.x] = 0;
    fs.hdr->nb[threadIdx.x] = 0;
    queue_head(fs, 0, threadIdx.x)[0] = queue_head(fs, 1, threadIdx.x)[0] = 0;
  }
  for (int i = threadIdx.x; i < GS_GROUPS * BO_BINS; i += blockDim.x) fs.bcnt[i] = 0;
  if (threadIdx.x == 0) {
    fs.hdr->h = 0;
    fs.hdr->k = 1;
    fs.hdr->nA = fs.hdr->nplain = 0;
    fs.hdr->bmode = 1;
    fs.hdr->bexit = 0;
  }
}

// LDS: the frame has at most TL tiles and its working arrays live in LDS (an
// instantiation of its own, so that every access to them is an LDS access).
// Two callers:
//   counts == null (the forward call): the tile counts come from the ranges.
//     If a plan built ahead for this frame waits in the state (planned), the
//     kernel only checks it against the frame (tile grid and pair total) and
//     the frame's status, and hands it over;
//   counts != null (the plan built ahead, beside the sort): the per-tile
//     counts of the binning pass; the plan is marked as waiting.
// dyn: LDS_BYTES of LDS for the working arrays when LDS, else POLICY_BYTES.
// Every thread of a workgroup of NT threads calls it.
template <bool LDS>
__device__ void schedule_frame(const int2 *__restrict__ ranges,
                               const int32_t *__restrict__ counts_in, int T, int tiles_x,
                               int chunk_mode, int force_k, int force_h, double lambda_,
                               double beta, double eps, int nblocks, char *__restrict__ fwd_state,
                               unsigned long long *__restrict__ stats,
                               int32_t *__restrict__ status, int64_t cap_pairs, uint32_t *dyn) {
  FwdState fs = fwd_state_at(fwd_state, T);
  const bool ahead = counts_in != nullptr;
  // 0. the frame runs only if every earlier call of it succeeded and its pairs
  //    fit the state's contributor bitmap; otherwise the plan is empty
  __shared__ int run, handed;
  if (threadIdx.x == 0) {
    // every word this decision reads is loaded at once (one memory round trip)
    const int st = *status;
    const int64_t npairs = T > 0 && !ahead ? (int64_t)ranges[T - 1].y : 0;
    const PlanHdr hd = *fs.hdr;
    handed = 0;
    const bool waiting =
        (hd.planned == PLAN_READY) & (hd.ntiles == T) & (hd.nw == contrib_words(T, cap_pairs)) &
        (hd.plan_mode == chunk_mode) & (hd.plan_force_k == force_k) &
        (hd.plan_force_h == force_h) & (hd.plan_nblocks == nblocks) &
        (hd.plan_lambda == lambda_) & (hd.plan_beta == beta) & (hd.plan_eps == eps);
    if (!ahead && waiting) {
      // built ahead: valid for any frame of this grid (a plan only orders and
      // splits the tiles), checked against the pair total to catch a stale one
      const bool same = npairs == (int64_t)hd.plan_pairs;
      if (st == GS_OK && !same) report_status(status, GS_ERR_WORKSPACE);
      run = hd.run_f && st == GS_OK && same;
      handed = 1;
      fs.hdr->planned = 0;
      if (run && stats) atomicAdd(&stats[3], (unsigned long long)hd.h);
    } else {
      run = st == GS_OK && npairs <= cap_pairs;
      if (st == GS_OK && npairs > cap_pairs) report_status(status, GS_ERR_WORKSPACE);
      fs.hdr->planned = 0;
    }
    fs.hdr->run_f = run;
    fs.hdr->run_b = 0;
    fs.hdr->nw = contrib_words(T, cap_pairs);
    fs.hdr->err = 0;
    fs.hdr->ntiles = T;
  }
  __syncthreads();
  if (!run) empty_plan(fs);
  if (!run || handed) return;
  const double workers = (double)(nblocks * GS_WAVES_PER_BLOCK) / 4.0;  // four waves per tile
  // working arrays: LDS for frames of up to TL tiles, else the forward state's
  // item and bound arrays (written for real only after they served here)
  constexpr bool lds = LDS;
  uint32_t *key = lds ? dyn : reinterpret_cast<uint32_t *>(fs.counts);
  int32_t *ord = lds ? reinterpret_cast<int32_t *>(dyn + TL) : fs.order;
  uint32_t *tmp_k = lds ? dyn + 2 * TL : reinterpret_cast<uint32_t *>(fs.items);
  int32_t *tmp_v = lds ? reinterpret_cast<int32_t *>(dyn + 3 * TL) : fs.items + T;
  // 1. counts and the (bit-limited) descending key
  uint32_t mx = 0;
  long long tot = 0;
  for (int t0 = threadIdx.x; t0 < T; t0 += NT * RB_ROUNDS) {
    int2 rr[RB_ROUNDS];
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++) {
      const int t = t0 + r * NT;
      rr[r] = t >= T ? make_int2(0, 0) : (ahead ? make_int2(0, counts_in[t]) : ranges[t]);
    }
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++) {
      const int t = t0 + r * NT;
      if (t < T) {
        const uint32_t c = (uint32_t)max(0, rr[r].y - rr[r].x);
        key[t] = c;
        ord[t] = t;
        mx = max(mx, c);
        tot += c;
      }
    }
  }
  block_max_sum(mx, tot);
  if (ahead && tot > cap_pairs) {
    // built ahead: the pair total is known only now
    if (threadIdx.x == 0) {
      if (*status == GS_OK) report_status(status, GS_ERR_WORKSPACE);
      fs.hdr->run_f = 0;
    }
    empty_plan(fs);
    return;
  }
  int bits = 0;
  while (bits < 32 && (mx >> bits) != 0u) bits++;
  const uint32_t full = bits >= 32 ? 0xFFFFFFFFu : ((1u << bits) - 1u);
  __syncthreads();
  for (int t = threadIdx.x; t < T; t += NT) key[t] = full - key[t];  // ascending key = descending N_t
  __syncthreads();
  // 2. stable LSD passes (ties keep ascending tile id)
  const int npass = (bits + 7) / 8;
  for (int pass = 0; pass < npass; pass++) {
    const bool even = (pass & 1) == 0;
    block_radix_pass(even ? key : tmp_k, even ? ord : tmp_v, even ? tmp_k : key,
                     even ? tmp_v : ord, T, 8 * pass);
  }
  if (npass & 1) {
    for (int t = threadIdx.x; t < T; t += NT) {
      key[t] = tmp_k[t];
      ord[t] = tmp_v[t];
    }
    __syncthreads();
  }
  // sorted counts: the forward state keeps them and the LPT order
  int32_t *cnts = lds ? reinterpret_cast<int32_t *>(tmp_k) : fs.counts;
  for (int t = threadIdx.x; t < T; t += NT) {
    const int32_t c = (int32_t)(full - key[t]);
    cnts[t] = c;
    if (lds) {
      fs.counts[t] = c;
      fs.order[t] = ord[t];
    }
  }
  __syncthreads();

  // 3. chunking policy
  int h = 0, k = 1;
  if (chunk_mode == 2) {
    k = force_k <= 2 ? 2 : (force_k <= 4 ? 4 : (force_k <= 8 ? 8 : 16));
    h = force_h <= 0 ? T : min(force_h, T);
    h = min(h, GS_HK_MAX / k);
  } else if (chunk_mode == 1 && T > 0) {
    // sS[h] = N_1 + ... + N_h (exact), sN[h] = N_{h+1} (0 past the last tile)
    long long *sS = reinterpret_cast<long long *>(dyn);
    int *sN = reinterpret_cast<int *>(sS + HMAX + 1);
    {
      static_assert(HMAX == 2 * NT, "two prefix entries per thread");
      const int i0 = 2 * threadIdx.x;
      const long long a = i0 < T ? cnts[i0] : 0, b = i0 + 1 < T ? cnts[i0 + 1] : 0;
      long long all;
      const long long before = block_excl_scan<long long>(a + b, all);
      sS[i0 + 1] = before + a;
      sS[i0 + 2] = before + a + b;
      sN[i0] = (int)a;
      sN[i0 + 1] = (int)b;
      if (threadIdx.x == 0) {
        sS[0] = 0;
        sN[HMAX] = HMAX < T ? cnts[HMAX] : 0;
      }
    }
    __syncthreads();
    const double Nt = (double)tot, N1 = (double)cnts[0];
    const double T0 = fmax(Nt / workers, N1) + beta * N1;
    // candidates in (k ascending, h ascending) order
    int len[4], off[5];
    off[0] = 0;
    for (int q = 0; q < 4; q++) {
      len[q] = min(T, GS_HK_MAX / (2 << q));
      off[q + 1] = off[q] + len[q];
    }
    double best = 3.0e300;
    int bidx = 0x7FFFFFFF;
    for (int i = threadIdx.x; i < off[4]; i += NT) {
      const int q = i < off[1] ? 0 : (i < off[2] ? 1 : (i < off[3] ? 2 : 3));
      const int kk = 2 << q;
      const int hh = i - off[q] + 1;
      const double next = hh < T ? (double)sN[hh] : 0.0;
      const double l = fmax((2.0 * N1) / (double)kk, next);
      const double avg = ((Nt + (double)sS[hh]) + (lambda_ * (double)hh) * (double)kk) / workers;
      const double est = fmax(avg, l) + beta * l;
      if (est < best || (est == best && i < bidx)) {
        best = est;
        bidx = i;
      }
    }
    block_min_idx(best, bidx);
    if (bidx != 0x7FFFFFFF && best <= (1.0 - eps) * T0) {
      const int q = bidx < off[1] ? 0 : (bidx < off[2] ? 1 : (bidx < off[3] ? 2 : 3));
      k = 2 << q;
      h = bidx - off[q] + 1;
    }
    __syncthreads();
  }
  if (h == 0) k = 1;
  const int bins = few_tiles(T, nblocks) ? 0 : 1;

  // 4. queues. The LPT positions e in [0, T) fall into classes (group of the
  //    tile, chunked iff e < h); a stable partition by class keeps the LPT order
  //    inside every class.
  int32_t *perm = lds ? reinterpret_cast<int32_t *>(dyn + 2 * TL) : fs.sub_last;
  __shared__ int ccount[NCLS], cstart[NCLS], qoff[GS_GROUPS + 1];
  class_partition(ord, T, h, tiles_x, perm, ccount, cstart);
  if (threadIdx.x == 0) {
    int q = 0;
    for (int g = 0; g < GS_GROUPS; g++) {
      qoff[g] = q;
      q += 8 * k * ccount[2 * g] + 4 * ccount[2 * g + 1];
    }
    qoff[GS_GROUPS] = q;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < T; i += NT) {
    const int e = perm[i];
    const int tile = ord[e];
    const int c = 2 * tile_group(tile, tiles_x) + (e >= h ? 1 : 0);
    const int g = c >> 1, r = i - cstart[c];
    if ((c & 1) == 0) {  // chunked: LPT slot e
      const int a0 = qoff[g] + 4 * k * r, b0 = a0 + 4 * k * ccount[c];
      for (int p = 0; p < k; p++)
        for (int q = 0; q < 4; q++) {
          fs.items[a0 + 4 * p + q] = make_item(ITEM_PASS_A, q, p, e);
          fs.items[b0 + 4 * p + q] = make_item(ITEM_PASS_B, q, p, e);
        }
    } else {
      const int p0 = qoff[g] + 8 * k * ccount[c - 1] + 4 * r;
      for (int q = 0; q < 4; q++) fs.items[p0 + q] = make_item(ITEM_PLAIN, q, 0, tile);
    }
  }
  const int nA = 4 * h * k;
  for (int i = threadIdx.x; i < nA; i += NT) fs.doneA[i] = 0;
  for (int i = threadIdx.x; i < 4 * h; i += NT) {
    fs.sat[i] = k;
    fs.doneB[i] = 0;
  }
  if (threadIdx.x < GS_GROUPS) {
    const int g = threadIdx.x;
    const int len = qoff[g + 1] - qoff[g], qa = 4 * k * ccount[2 * g];
    const int W = group_workers(g, nblocks);
    // A pass-B item waits on pass-A items, so every item in front of it must be
    // held by a running worker: a group with chunk items hands out nothing
    // without a pop in the forward pass. The backward never waits.
    const int init_f = qa > 0 ? 0 : min(len, W);
    const int init_b = min(len - qa, W);
    fs.hdr->qa[g] = qa;
    fs.hdr->init_f[g] = init_f;
    fs.hdr->init_b[g] = init_b;
    queue_head(fs, 0, g)[0] = init_f;
    // the backward's head counts pops past its static hand-out, which a frame
    // with few tiles learns from its preparation (that sets the head) and any
    // other from the forward's bins
    queue_head(fs, 1, g)[0] = bins ? 0 : init_b;
  }
  // the forward files the backward's items by bin as their walks end
  for (int i = threadIdx.x; i < GS_GROUPS * BO_BINS; i += NT) fs.bcnt[i] = 0;
  for (int t = threadIdx.x; t < T; t += NT) fs.tlen[t] = 0ull;
  if (threadIdx.x <= GS_GROUPS) fs.hdr->qoff[threadIdx.x] = qoff[threadIdx.x];
  if (threadIdx.x == 0) {
    fs.hdr->bmode = bins;
    fs.hdr->bexit = 0;
    fs.hdr->h = h;
    fs.hdr->k = k;
    fs.hdr->nA = nA;
    fs.hdr->nplain = 4 * (T - h);
    if (stats) atomicAdd(&stats[3], (unsigned long long)h);
    if (ahead) {
      fs.hdr->plan_pairs = (int32_t)tot;
      fs.hdr->plan_mode = chunk_mode;
      fs.hdr->plan_force_k = force_k;
      fs.hdr->plan_force_h = force_h;
      fs.hdr->plan_nblocks = nblocks;
      fs.hdr->plan_lambda = lambda_;
      fs.hdr->plan_beta = beta;
      fs.hdr->plan_eps = eps;
      fs.hdr->planned = PLAN_READY;
    }
  }
}

}  // namespace sched_impl
}  // namespace
