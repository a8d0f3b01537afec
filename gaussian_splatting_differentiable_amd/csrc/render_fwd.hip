// gs_render_fwd: front-to-back alpha blending of 16x16 tiles.
//
// "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on GPUs",
// section 2.1, Eq. 2-3: alpha = o exp(-q/2); C = sum c alpha T; a pixel stops
// blending once T falls below 1e-4. Section 4: a persistent kernel takes work
// from a longest-first queue; the heaviest tiles are split into contiguous
// depth chunks (Eq. 4-5) with saturation signalling.
// "What the 3DGS Literature Left on the Table": Step 1 (b) the alpha >= 1/255
// cutoff as q <= tau; Step 1 (c) sub-tile culling of staged splat batches with a
// ballot and a find-first-set worklist; Step 1 (e) base-2 exponential; Step 5
// branchless blending with one canonical q shared with the backward; Step 6.3
// log2(o) folded into the exponent.
//
// gfx950 mapping: one workgroup of 16 wavefronts per CU, each a persistent worker
// that pops items (an 8x8 quarter of a tile or of a chunk) until the queues are
// empty. A worker walks its list in batches of 64 splats staged in LDS (one
// record per lane, three 16-byte loads, the next batch in flight while the
// current one is blended); each lane tests its staged splat against the
// quarter's sample rectangle and the ballot of those tests is the worklist,
// walked on the scalar unit with the next entry's record read ahead.
//
// Exact chunking (a reading of section 4.2: chunks that start at T = 1 can stop
// later than the sequential renderer, so the composition is made exact):
//   pass A, chunk p: per pixel the product P_p of (1 - alpha) over the chunk,
//     stopping once P_p < 1e-4; if every pixel of the quarter stops, the chunk
//     lowers sat[] with atomicMin and later chunks give up (checked per batch).
//   pass B, chunk p: waits for pass A of chunks 0..p-1 (queued earlier, so
//     already taken by running workers), starts from T_in = prod_{q<p} P_q and
//     blends with the exact stop rule, writing (C, T, consumed) of the chunk.
//   the last pass-B worker of a quarter sums the chunk colours (Eq. 5 with the
//     transmittance already applied) and writes the pixel outputs.
#include "render_common.h"

namespace {

constexpr float NEG_HALF_LOG2E = -0.72134752044448170368f;
constexpr float T_STOP = 1e-4f;
constexpr int BATCH = GS_WAVE;  // splats per staged batch

struct Px {
  float fx, fy;
  bool inside;
  int p;  // pixel index (fewer than 2^31 / 3 pixels: at most 65535 tiles)
};

__device__ __forceinline__ Px pixel_of(const SubTile &st, const CamK &cam) {
  Px x;
  const int lane = __lane_id();
  const int px = st.x0 + (lane & 7), py = st.y0 + (lane >> 3);
  x.inside = px < cam.width && py < cam.height;
  x.fx = (float)px + 0.5f;
  x.fy = (float)py + 0.5f;
  x.p = (st.prow + py) * cam.width + px;
  return x;
}

// An id outside [0, n) (which only a frame whose sort failed could hold) is an
// empty slot: it is neither read nor blended.
__device__ __forceinline__ bool valid_id(int id, int n) { return (unsigned)id < (unsigned)n; }

// Stage one splat record for the worklist: 2b and log2(o) replace b and pad.
__device__ __forceinline__ bool stage(Splat s, const SubTile &st, Splat *slot) {
  const bool cand = rect_may_hit(s.p0.x, s.p0.y, s.p0.z, s.p0.w, s.p1.x, s.p2.y, st.hx0, st.hx1,
                                 st.hy0, st.hy1);
  s.p0.w = 2.0f * s.p0.w;
  s.p2.w = __log2f(s.p1.y);
  *slot = s;
  return cand;
}

// Two-stage load pipeline over a splat list: ids two batches ahead, records one
// batch ahead, so neither the id load nor the dependent record load stalls the
// batch being blended. Slots past the end carry id -1 (and read record 0).
struct Pipe {
  int idc;     // id of this lane's slot in the batch whose records are in rec
  int idn;     // id of its slot in the batch after it
  Splat rec;
};

__device__ __forceinline__ int load_id(const int32_t *__restrict__ sids, int b, int ce) {
  const int e = b + __lane_id();
  return e < ce ? sids[e] : -1;
}

__device__ __forceinline__ void pipe_start(Pipe &pp, const Splat *__restrict__ splats,
                                           const int32_t *__restrict__ sids, int cs, int ce,
                                           int n) {
  pp.idc = load_id(sids, cs, ce);
  pp.rec = splats[valid_id(pp.idc, n) ? pp.idc : 0];
  pp.idn = load_id(sids, cs + BATCH, ce);
}

// After the batch at b is staged: start the records of b + BATCH and the ids of
// b + 2 BATCH.
__device__ __forceinline__ void pipe_advance(Pipe &pp, const Splat *__restrict__ splats,
                                             const int32_t *__restrict__ sids, int b, int ce,
                                             int n) {
  pp.idc = pp.idn;
  pp.rec = splats[valid_id(pp.idc, n) ? pp.idc : 0];
  pp.idn = load_id(sids, b + 2 * BATCH, ce);
}

struct Blend {
  float C0, C1, C2, T;
  int consumed;  // list entries consumed (relative to the range start)
  int wlast;     // 1 + last position any lane hit (relative), 0 if none
  int nh;        // this lane's hits (counted only when STATS)
};

// Blend [cs, ce) into pixels that start with transmittance T0. Branchless per
// entry: a lane that misses (or has stopped) takes alpha = 0, which leaves its
// colour and T unchanged bit for bit. A lane is alive exactly while its T is at
// least 1e-4 (lanes outside the image start at T = 0); the wave carries the
// alive lanes as a scalar mask, so the hit mask is that mask AND the ballot of
// q <= tau, and a lane stops where it was hit and the new ballot of T >= 1e-4
// drops it (one vector compare each, the rest on the scalar unit).
// A batch whose staged opacities are all at most 0.985 cannot reach the 0.99
// clamp (alpha <= o), so its entries are blended without the min.
// cw: the quarter's contributor word of the range's first batch; every batch
// walked writes its word (bit j: some lane blended entry j of the batch).
// CUTS (plain tiles of a frame with few tiles): cutp is this lane's pixel in
// the tile's cut record; a walk that reaches a cut writes T there and the colour blended since
// the previous cut, then blends on from zero, and writes the colour after its
// last cut at the end; ncut counts the cuts reached. Every segment is a sum of
// non-negative terms, so the backward's sums of the segments behind a cut keep
// full relative precision (a difference of running totals would not); the
// returned colour is the sum of the segments.
template <bool STATS, bool CUTS>
__device__ __forceinline__ Blend blend_range(const Splat *__restrict__ splats,
                                             const int32_t *__restrict__ sids, int cs, int ce,
                                             int n, const SubTile &st, const Px &x, float T0,
                                             Splat *sbuf, uint64_t *__restrict__ cw,
                                             float *__restrict__ cutp, int &ncut,
                                             uint32_t &nhits, uint32_t &nsteps,
                                             uint32_t &nhsteps) {
  Blend r;
  r.C0 = r.C1 = r.C2 = 0.0f;
  r.T = x.inside ? T0 : 0.0f;
  r.consumed = r.T >= T_STOP ? ce - cs : 0;
  r.wlast = 0;
  r.nh = 0;
  uint64_t alive = wave_ballot(r.T >= T_STOP);
  const int lane = __lane_id();
  Pipe pp;
  if (alive && cs < ce) pipe_start(pp, splats, sids, cs, ce, n);
  ncut = 0;
  float D0 = 0.0f, D1 = 0.0f, D2 = 0.0f;  // the segments before the last cut reached
  for (int b = cs; b < ce && alive; b += BATCH) {
    if (CUTS && ncut < GS_NCUT && b - cs == BATCH * cut_batch(ncut)) {
      float *c = cutp + 4 * 256 * ncut;
      c[0] = r.T;
      c[256] = r.C0;
      c[512] = r.C1;
      c[768] = r.C2;
      D0 += r.C0;
      D1 += r.C1;
      D2 += r.C2;
      r.C0 = r.C1 = r.C2 = 0.0f;
      ncut++;
    }
    const bool cand = stage(pp.rec, st, &sbuf[lane]) && valid_id(pp.idc, n);
    const uint64_t work = wave_ballot(cand);
    const bool clamp = wave_ballot(cand && pp.rec.p1.y > 0.985f) != 0;
    pipe_advance(pp, splats, sids, b, ce, n);
    wave_sync();
    const int base = b - cs;
    uint64_t bm = 0;  // the batch's entries that some lane blended
    auto step = [&](const Splat &s, int j, auto clamp_tag) {
      constexpr bool CLAMP = decltype(clamp_tag)::value;
      const int pos = base + j;
      const float dx = x.fx - s.p0.x, dy = x.fy - s.p0.y;
      const float q = canon_q(s.p0.z, s.p0.w, s.p1.x, dx, dy);
      const uint64_t hm = alive & wave_ballot(q <= s.p2.y);
      if constexpr (STATS) nsteps++;
      if (!hm) return true;  // no lane hits: nothing changes
      const bool hit = __builtin_amdgcn_inverse_ballot_w64(hm);
      if constexpr (STATS) {
        nhits += __popcll(hm);
        nhsteps++;
        r.nh += hit ? 1 : 0;
      }
      bm = set_slot(bm, j);
      const float ex = __builtin_amdgcn_exp2f(__builtin_fmaf(q, NEG_HALF_LOG2E, s.p2.w));
      const float al = hit ? (CLAMP ? fminf(0.99f, ex) : ex) : 0.0f;
      const float w = al * r.T;
      r.C0 = __builtin_fmaf(w, s.p1.z, r.C0);
      r.C1 = __builtin_fmaf(w, s.p1.w, r.C1);
      r.C2 = __builtin_fmaf(w, s.p2.x, r.C2);
      r.T = r.T - w;
      const uint64_t now = wave_ballot(r.T >= T_STOP);
      const uint64_t died = hm & ~now;
      if (died) r.consumed = __builtin_amdgcn_inverse_ballot_w64(died) ? pos + 1 : r.consumed;
      alive = now;
      return alive != 0;
    };
    if (clamp)
      walk_worklist(work, sbuf, [&](const Splat &s, int j) {
        return step(s, j, std::true_type{});
      });
    else
      walk_worklist(work, sbuf, [&](const Splat &s, int j) {
        return step(s, j, std::false_type{});
      });
    if (bm) r.wlast = base + 64 - __builtin_clzll(bm);  // 1 + the last entry any lane blended
    if (lane == 0) cw[base >> 6] = bm;
    wave_sync();
  }
  if (CUTS && ncut > 0) {
    float *c = cutp + 4 * 256 * GS_NCUT;
    c[0] = r.C0;
    c[256] = r.C1;
    c[512] = r.C2;
    r.C0 += D0;
    r.C1 += D1;
    r.C2 += D2;
  }
  return r;
}

// Pass A: transmittance product over the chunk; gives up when sat < chunk.
// Lanes outside the image start at P = 0 (dead), as in blend_range.
template <bool STATS>
__device__ __forceinline__ float product_range(const Splat *__restrict__ splats,
                                               const int32_t *__restrict__ sids, int cs, int ce,
                                               int n, const SubTile &st, const Px &x,
                                               Splat *sbuf, const int32_t *sat, int chunk,
                                               bool &gave_up, uint32_t &nsteps) {
  float P = x.inside ? 1.0f : 0.0f;
  uint64_t alive = wave_ballot(P >= T_STOP);
  gave_up = false;
  const int lane = __lane_id();
  Pipe pp;
  if (alive && cs < ce) pipe_start(pp, splats, sids, cs, ce, n);
  // sat is read one batch late: the load goes out with the batch prefetch, so
  // waiting for it costs nothing beyond the wait for the prefetch itself
  int satv = chunk;
  for (int b = cs; b < ce && alive; b += BATCH) {
    if (satv < chunk) {
      gave_up = true;
      break;
    }
    const bool cand = stage(pp.rec, st, &sbuf[lane]) && valid_id(pp.idc, n);
    const uint64_t work = wave_ballot(cand);
    pipe_advance(pp, splats, sids, b, ce, n);
    const int satn = __hip_atomic_load(sat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wave_sync();
    walk_worklist(work, sbuf, [&](const Splat &s, int) {
      const float dx = x.fx - s.p0.x, dy = x.fy - s.p0.y;
      const float q = canon_q(s.p0.z, s.p0.w, s.p1.x, dx, dy);
      const uint64_t hm = alive & wave_ballot(q <= s.p2.y);
      if constexpr (STATS) nsteps++;
      if (!hm) return true;
      const float ex = __builtin_amdgcn_exp2f(__builtin_fmaf(q, NEG_HALF_LOG2E, s.p2.w));
      const float al = __builtin_amdgcn_inverse_ballot_w64(hm) ? fminf(0.99f, ex) : 0.0f;
      P = P - al * P;
      alive = wave_ballot(P >= T_STOP);
      return alive != 0;
    });
    satv = satn;
    wave_sync();
  }
  return P;
}

// Every lane's earlier stores become visible device-wide before lane 0 publishes.
__device__ __forceinline__ void wave_release() {
  __threadfence();
  wave_sync();
}

__device__ __forceinline__ float ld_f(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_i(const int32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The backward's queue, filed as the forward's walks end (frames whose
// backward has no preparation): quarter `quad` of a plain tile adds its walk
// length to the tile's length word; the quarter that completes the word files
// the tile's backward items in the bins of their walks: the whole tile
// (walked by the longest of its quarters), or, when that walk is long, its
// four quarters. One returning atomic per quarter, one more per filed item.
__device__ __forceinline__ void file_plain(const FwdState &fs, int tile, int quad, int wlast,
                                           int tiles_x) {
  const int lane = __lane_id();
  const uint64_t mine = (uint64_t)(min(wlast, 65534) + 1) << (16 * quad);
  uint64_t old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_or(&fs.tlen[tile], mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t o = ((uint64_t)(uint32_t)wave_first((int)(old >> 32)) << 32) |
                     (uint32_t)wave_first((int)(uint32_t)old);
  const int seen = ((o & 0xFFFFull) != 0) + (((o >> 16) & 0xFFFFull) != 0) +
                   (((o >> 32) & 0xFFFFull) != 0) + ((o >> 48) != 0);
  if (seen != 3) return;  // another quarter of the tile is still walking
  const uint64_t all = o | mine;
  const int l0 = (int)(all & 0xFFFFull) - 1, l1 = (int)((all >> 16) & 0xFFFFull) - 1;
  const int l2 = (int)((all >> 32) & 0xFFFFull) - 1, l3 = (int)(all >> 48) - 1;
  const int whole = max(max(l0, l1), max(l2, l3));
  const bool split = whole > SPLIT_WALK;
  if (split ? lane < 4 : lane == 0) {
    const int len = !split ? whole : lane == 0 ? l0 : lane == 1 ? l1 : lane == 2 ? l2 : l3;
    const int item = split ? make_item(ITEM_QUARTER, lane, 0, tile) : make_item(ITEM_PLAIN, 0, 0, tile);
    const int g = tile_group(tile, tiles_x);
    const uint32_t b = order_bin(len);
    const int pos = atomicAdd(&fs.bcnt[g * BO_BINS + b], 1);
    fs.blist[bin_base(fs.hdr, g, b) + pos] = item;
  }
}

// A chunk's quarter is a backward item of its own (pass B's item).
__device__ __forceinline__ void file_chunk(const FwdState &fs, int item, int tile, int wlast,
                                           int tiles_x) {
  if (__lane_id() != 0) return;
  const int g = tile_group(tile, tiles_x);
  const uint32_t b = order_bin(wlast);
  const int pos = atomicAdd(&fs.bcnt[g * BO_BINS + b], 1);
  fs.blist[bin_base(fs.hdr, g, b) + pos] = item;
}

// A worker with no tile left clears its own slice of the caller's array (the
// gradient array a backward of this frame adds into): slices of whole float4s
// by worker index, so no counter is shared and a late worker adds only its
// slice's stores to the end of the launch.
__device__ __forceinline__ void clear_slice(float *__restrict__ out, int64_t nout) {
  const int lane = __lane_id();
  const int64_t workers = (int64_t)gridDim.x * GS_WAVES_PER_BLOCK;
  const int64_t w = (int64_t)blockIdx.x * GS_WAVES_PER_BLOCK + wave_in_block();
  const int64_t n4 = nout / 4;                      // whole float4s
  const int64_t per = (n4 + workers - 1) / workers;  // float4s per worker
  const int64_t a = min(n4, w * per), e = min(n4, a + per);
  float4 *o4 = reinterpret_cast<float4 *>(out);
  for (int64_t i = a + lane; i < e; i += 64) o4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (w == workers - 1 && lane < nout - 4 * n4) out[4 * n4 + lane] = 0.0f;  // the ragged end
}

// A plan built ahead that the forward checks itself (no hand-over launch): the
// knobs and worker count it must have been built with, and the state's
// contributor words per quarter.
struct PlanKey {
  int planned;  // 1: check the waiting plan in the launch
  int mode, force_k, force_h, nblocks;
  float lambda_, beta, eps;
  long long nw;
};

// Whether this frame runs. planned: thread 0 of every workgroup checks the
// plan built ahead against the frame (the same decision everywhere: the tile
// grid, the knobs, the pair total against the tile ranges, the status), and
// workgroup 0 records it for the backward; a mismatch is GS_ERR_WORKSPACE.
// Otherwise the hand-over (or the schedule it built) decided.
__device__ __forceinline__ bool frame_runs(const FwdState &fs, const PlanKey &key, int T,
                                           const int2 *__restrict__ ranges,
                                           unsigned long long *__restrict__ stats,
                                           int32_t *__restrict__ status) {
  if (!key.planned) return fs.hdr->run_f != 0;
  __shared__ int s_run;
  if (threadIdx.x == 0) {
    const int st = *status;
    const int64_t npairs = T > 0 ? (int64_t)ranges[T - 1].y : 0;
    const PlanHdr *hd = fs.hdr;
    const bool match = (hd->planned == PLAN_READY) & (hd->ntiles == T) & (hd->nw == key.nw) &
                       (hd->plan_mode == key.mode) & (hd->plan_force_k == key.force_k) &
                       (hd->plan_force_h == key.force_h) & (hd->plan_nblocks == key.nblocks) &
                       (hd->plan_lambda == key.lambda_) & (hd->plan_beta == key.beta) &
                       (hd->plan_eps == key.eps) & (npairs == (int64_t)hd->plan_pairs);
    if (st == GS_OK && !match) report_status(status, GS_ERR_WORKSPACE);
    const bool run = hd->run_f && st == GS_OK && match;
    if (blockIdx.x == 0) {
      fs.hdr->run_f = run;
      if (run && stats) atomicAdd(&stats[3], (unsigned long long)hd->h);
    }
    s_run = run;
  }
  __syncthreads();
  return s_run != 0;
}

// STATS: count hits, tested entries and sub-tile hits (only when the caller asks
// for them: the counters cost a few scalar instructions per entry). CUTS: the
// frame has few tiles, and its plain walks record their state at the cuts.
template <bool STATS, bool CUTS>
__global__ void __launch_bounds__(GS_WAVE * GS_WAVES_PER_BLOCK)
__attribute__((amdgpu_waves_per_eu(4))) k_render_fwd(
    const Splat *__restrict__ splats, int n, const int32_t *__restrict__ sorted_ids,
    const int2 *__restrict__ ranges, CamK cam, float *__restrict__ rgb, float *__restrict__ Tout,
    int32_t *__restrict__ last, char *__restrict__ state, int T,
    unsigned long long *__restrict__ stats, int32_t *__restrict__ pixel_hits,
    int32_t *__restrict__ status, int spin_limit, float *__restrict__ clear, int64_t nclear,
    PlanKey key) {
  __shared__ Splat sbuf_all[GS_WAVES_PER_BLOCK][BATCH];
  Splat *sbuf = sbuf_all[wave_in_block()];
  FwdState fs = fwd_state_at(state, T);
  // a frame that failed earlier has an empty plan: its workers only clear
  const bool run = frame_runs(fs, key, T, ranges, stats, status);
  const bool bins = fs.hdr->bmode != 0;
  fs.nw = fs.hdr->nw;
  const int k = fs.hdr->k;
  const int P = cam.width * cam.height * cam.views;
  const int lane = __lane_id();
  uint32_t nhits = 0, nsteps = 0, nhsteps = 0;  // per worker; far below 2^32
  __shared__ uint32_t drained;
  Worker wk = make_worker(&drained);
  for (;;) {
    const int t = run ? next_item(fs, 0, wk) : -1;
    if (t < 0) break;
    wk.round++;
    const int it = fs.items[t];
    const int kind = item_kind(it), quad = item_quad(it), p = item_chunk(it);
    const int idx = item_index(it);
    const int tile = kind == ITEM_PLAIN ? idx : fs.order[idx];
    const SubTile st = subtile_of(tile, quad, cam);
    const int2 rg = ranges[tile];
    const Px x = pixel_of(st, cam);
    if (kind == ITEM_PLAIN) {
      if (st.empty) {
        if (lane == 0) {
          fs.sub_last[tile * 4 + quad] = 0;
          fs.qcut[tile * 4 + quad] = 0;
        }
        if (bins) file_plain(fs, tile, quad, 0, cam.tiles_x);
        continue;
      }
      int ncut = 0;
      Blend r;
      if constexpr (CUTS)
        r = blend_range<STATS, true>(splats, sorted_ids, rg.x, rg.y, n, st, x, 1.0f, sbuf,
                                     contrib_base(fs, quad, tile, rg.x),
                                     fs.cut + (size_t)tile * GS_CUT_FLOATS + 64 * quad + lane,
                                     ncut, nhits, nsteps, nhsteps);
      else
        r = blend_range<STATS, false>(splats, sorted_ids, rg.x, rg.y, n, st, x, 1.0f, sbuf,
                                      contrib_base(fs, quad, tile, rg.x), nullptr, ncut, nhits,
                                      nsteps, nhsteps);
      if (x.inside) {
        rgb[x.p] = cam.bg_on ? fmaf(r.T, cam.bg[0], r.C0) : r.C0;
        rgb[P + x.p] = cam.bg_on ? fmaf(r.T, cam.bg[1], r.C1) : r.C1;
        rgb[2 * P + x.p] = cam.bg_on ? fmaf(r.T, cam.bg[2], r.C2) : r.C2;
        Tout[x.p] = r.T;
        last[x.p] = r.consumed;
        if (STATS && pixel_hits) pixel_hits[x.p] += r.nh;
      }
      if (lane == 0) {
        fs.sub_last[tile * 4 + quad] = r.wlast;
        fs.qcut[tile * 4 + quad] = ncut;
      }
      if (bins) file_plain(fs, tile, quad, r.wlast, cam.tiles_x);
      continue;
    }
    int cs, ce;
    chunk_range(rg.x, rg.y, p, k, cs, ce);
    const int ci = chunk_index(idx, p, quad, k);
    int32_t *sat = &fs.sat[idx * 4 + quad];
    if (kind == ITEM_PASS_A) {
      float Pp = 0.0f;
      if (!st.empty) {
        bool gave_up = false;
        Pp = product_range<STATS>(splats, sorted_ids, cs, ce, n, st, x, sbuf, sat, p, gave_up,
                                  nsteps);
        if (gave_up) Pp = 0.0f;  // an earlier chunk already took every pixel below 1e-4
        // every pixel of the quarter below the threshold: later chunks may give up
        if (!gave_up && wave_ballot(x.inside && Pp >= T_STOP) == 0 && lane == 0) atomicMin(sat, p);
      }
      fs.PA[(int64_t)ci * 64 + lane] = Pp;
      wave_release();
      if (lane == 0) st_flag(&fs.doneA[ci], 1);
      continue;
    }
    // pass B: wait for pass A of the earlier chunks of this quarter
    float Tin = 1.0f;
    int ok = 1;
    if (lane == 0) {
      for (int q = 0; q < p && ok; q++) {
        int spins = 0;
        while (ld_flag(&fs.doneA[chunk_index(idx, q, quad, k)]) == 0) {
          if (++spins > spin_limit) {
            atomicOr(&fs.hdr->err, 1);
            report_status(status, GS_ERR_TIMEOUT);
            ok = 0;
            break;
          }
          // back off: a few quick probes, then about 8k cycles between probes,
          // so thousands of waiting waves do not load the L2 with probes
          if (spins < 64)
            __builtin_amdgcn_s_sleep(4);
          else
            __builtin_amdgcn_s_sleep(127);
        }
      }
    }
    ok = wave_first(ok);
    __threadfence();  // acquire: the producers' PA stores are visible from here
    for (int q = 0; q < p; q++)
      Tin = ok ? Tin * ld_f(&fs.PA[(int64_t)chunk_index(idx, q, quad, k) * 64 + lane]) : 0.0f;
    Blend r;
    r.C0 = r.C1 = r.C2 = 0.0f;
    r.T = Tin;
    r.consumed = -1;
    r.wlast = 0;
    r.nh = 0;
    const bool skip = st.empty || ld_i(sat) < p;
    if (!skip) {
      int ncut = 0;
      r = blend_range<STATS, false>(splats, sorted_ids, cs, ce, n, st, x, Tin, sbuf,
                             contrib_base(fs, quad, tile, rg.x) + ((cs - rg.x) >> 6), nullptr,
                             ncut, nhits, nsteps, nhsteps);
      if (!(x.inside && Tin >= T_STOP)) r.consumed = -1;  // stopped before this chunk
    }
    const int64_t cp = (int64_t)ci * 64 + lane;
    fs.CB[3 * cp] = r.C0;
    fs.CB[3 * cp + 1] = r.C1;
    fs.CB[3 * cp + 2] = r.C2;
    fs.TB[cp] = r.T;
    fs.LB[cp] = r.consumed;
    if (STATS) fs.HB[cp] = r.nh;
    if (lane == 0) fs.chunk_last[ci] = r.wlast;
    if (bins) file_chunk(fs, it, tile, r.wlast, cam.tiles_x);
    wave_release();
    int prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(&fs.doneB[idx * 4 + quad], 1, __ATOMIC_ACQ_REL,
                                    __HIP_MEMORY_SCOPE_AGENT);
    prev = wave_first(prev);
    if (prev != k - 1 || st.empty) continue;
    // the last finisher of this quarter composes the chunks in depth order. The
    // image ends at the first chunk after which T is below 1e-4; a later chunk
    // that pass A's products still let through (rounding at a knife edge) is
    // marked as not reached, so the backward takes exactly the composed chunks.
    __threadfence();
    float C0 = 0.f, C1 = 0.f, C2 = 0.f, Tf = 1.0f;
    int lastv = 0, nhv = 0, qend = k;
    for (int q = 0; q < k; q++) {
      const int64_t c2 = (int64_t)chunk_index(idx, q, quad, k) * 64 + lane;
      const int lb = ld_i(&fs.LB[c2]);
      if (lb < 0) {
        qend = q;
        break;
      }
      C0 += ld_f(&fs.CB[3 * c2]);
      C1 += ld_f(&fs.CB[3 * c2 + 1]);
      C2 += ld_f(&fs.CB[3 * c2 + 2]);
      Tf = ld_f(&fs.TB[c2]);
      if (STATS) nhv += ld_i(&fs.HB[c2]);
      int qs, qe;
      chunk_range(rg.x, rg.y, q, k, qs, qe);
      lastv = qs - rg.x + lb;
      if (Tf < T_STOP) {
        qend = q + 1;
        break;
      }
    }
    for (int q = qend; q < k; q++) fs.LB[(int64_t)chunk_index(idx, q, quad, k) * 64 + lane] = -1;
    if (x.inside) {
      rgb[x.p] = cam.bg_on ? fmaf(Tf, cam.bg[0], C0) : C0;
      rgb[P + x.p] = cam.bg_on ? fmaf(Tf, cam.bg[1], C1) : C1;
      rgb[2 * P + x.p] = cam.bg_on ? fmaf(Tf, cam.bg[2], C2) : C2;
      Tout[x.p] = Tf;
      last[x.p] = lastv;
      if (STATS && pixel_hits) pixel_hits[x.p] += nhv;
    }
  }
  if (clear) clear_slice(clear, nclear);
  if (STATS && stats && lane == 0) {
    atomicAdd(&stats[0], (unsigned long long)nhits);
    atomicAdd(&stats[1], nsteps * (unsigned long long)GS_WAVE);
    atomicAdd(&stats[2], (unsigned long long)nhsteps);
  }
}

}  // namespace

hipError_t gs_launch_schedule(const int32_t *ranges, const int32_t *counts, const CamK &cam,
                              int chunk_mode, int force_k, int force_h, double lambda_,
                              double beta, double eps, int nblocks, void *fwd_state,
                              int64_t *stats, int32_t *status, int64_t cap_pairs,
                              hipStream_t st);

int32_t gs_wait_limit(int32_t fallback);

hipError_t gs_launch_render_fwd(int n, const float *splats, const int32_t *sorted_ids,
                                const int32_t *ranges, const CamK &cam, const gs_sched &sched,
                                float *rgb, float *T, int32_t *last, void *fwd_state,
                                int64_t cap_pairs, int64_t *stats, int32_t *pixel_hits,
                                int32_t *status, int workers_waves, float *clear,
                                int64_t nclear, hipEvent_t ev0, hipEvent_t ev1, hipStream_t st) {
  const int ntiles = cam.tiles_x * cam.tiles_y;
  const int nblocks = workers_waves / GS_WAVES_PER_BLOCK;
  PlanKey key;
  key.planned = sched.planned;
  key.mode = sched.chunk_mode;
  key.force_k = sched.force_k;
  key.force_h = sched.force_h;
  key.nblocks = nblocks;
  key.lambda_ = sched.lambda_;
  key.beta = sched.beta;
  key.eps = sched.eps;
  key.nw = contrib_words(ntiles, cap_pairs);
  hipError_t e = hipSuccess;
  // a plan built ahead is checked inside the launch; otherwise the schedule
  // hands a waiting plan over, or builds one
  if (!sched.planned)
    e = gs_launch_schedule(ranges, nullptr, cam, sched.chunk_mode, sched.force_k, sched.force_h,
                           sched.lambda_, sched.beta, sched.eps, nblocks, fwd_state, stats, status,
                           cap_pairs, st);
  if (e != hipSuccess) return e;
  // persistent workers, GS_WAVES_PER_BLOCK per workgroup; workers that find the
  // queues empty exit at once
  if (ev0 && (e = hipEventRecord(ev0, st)) != hipSuccess) return e;
  const bool count = stats || pixel_hits, cuts = records_cuts(ntiles, nblocks);
  auto kern = count ? (cuts ? k_render_fwd<true, true> : k_render_fwd<true, false>)
                    : (cuts ? k_render_fwd<false, true> : k_render_fwd<false, false>);
  hipLaunchKernelGGL(kern, dim3(nblocks),
                     dim3(GS_WAVE * GS_WAVES_PER_BLOCK), 0, st,
                     reinterpret_cast<const Splat *>(splats), n, sorted_ids,
                     reinterpret_cast<const int2 *>(ranges), cam, rgb, T, last,
                     reinterpret_cast<char *>(fwd_state), ntiles,
                     reinterpret_cast<unsigned long long *>(stats), pixel_hits, status,
                     gs_wait_limit(GS_SPIN_LIMIT), clear, clear ? nclear : (int64_t)0, key);
  e = hipGetLastError();
  if (e == hipSuccess && ev1) e = hipEventRecord(ev1, st);
  return e;
}
