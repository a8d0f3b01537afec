// gs_render_bwd: gradients of the blended image with respect to the 9
// screen-space splat parameters (centre x/y, conic a/b/c, opacity, r/g/b).
//
// "What the 3DGS Literature Left on the Table": Step 1 (a) per-pixel
// derivatives summed over a wave before global atomics; Step 1 (e) the scalar
// accumulator accum = c_behind . dL/dC; Step 2 the reduce-scatter that leaves
// the 9 sums on 9 lanes for one atomic instruction; Step 4 the walk from the
// last contributor back to the front; Step 5 branchless alpha = 0 predication
// for missed pixels and one canonical q shared with the forward pass; Step 6.3
// the per-splat term alpha T (c . dL/dC - accum), with log2(o) folded into the
// exponent and o divided back out once after the sum.
// "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on GPUs",
// section 4: the same persistent longest-first queue as the forward pass; a
// chunk of a heavy tile is differentiated on its own from the forward pass's
// chunk state: it starts from the transmittance after its last processed
// splat, T_end, with accum = (sum over later chunks of C_chunk . dL/dC) / T_end.
//
// gfx950 mapping: one wavefront per item (an 8x8 quarter), LDS-staged batches
// of 64 splats walked back to front with the next batch fetched ahead; the
// per-wave cull ballot skips splats that miss the quarter and a second ballot
// skips splats no live pixel hits.
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

__device__ __forceinline__ uint32_t order_bin(const FwdState &fs, int it, int k) {
  const int quad = item_quad(it), idx = item_index(it);
  const int len = item_kind(it) == ITEM_PLAIN
                      ? fs.sub_last[idx * 4 + quad]
                      : fs.chunk_last[chunk_index(idx, item_chunk(it), quad, k)];
  const int b = (int)(4.0f * __log2f((float)max(len, 0) + 1.0f));
  return (uint32_t)(BO_BINS - 1 - min(b, BO_BINS - 1));  // ascending bin = longest first
}

// The backward's preparation in one launch: workgroup g < GS_GROUPS orders
// group g's items and rewinds its queue; the others zero the gradient output.
__global__ void __launch_bounds__(BO_T) k_bwd_prep(char *__restrict__ state, int ntiles,
                                                  int nblocks, float *__restrict__ grads,
                                                  int64_t ng) {
  if (blockIdx.x >= GS_GROUPS) {
    const int64_t i = (int64_t)(blockIdx.x - GS_GROUPS) * BO_T + threadIdx.x;
    const int64_t n4 = ng / 4;
    if (i < n4) reinterpret_cast<float4 *>(grads)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < ng - 4 * n4) grads[4 * n4 + i] = 0.0f;
    return;
  }
  __shared__ int cnt[BO_W][BO_BINS];
  FwdState fs = fwd_state_at(state, ntiles);
  const int g = blockIdx.x, k = fs.hdr->k;
  const int lo = fs.hdr->qoff[g] + fs.hdr->qa[g], hi = fs.hdr->qoff[g + 1];
  const int n = hi - lo;
  // the backward's own hand-out: the first items go to its workers without a pop
  if (threadIdx.x == 0) {
    const int init = min(n, group_workers(g, nblocks));
    fs.hdr->init_b[g] = init;
    queue_head(fs, 1, g)[0] = init;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < BO_W * BO_BINS; i += BO_T) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int chunk = (n + BO_W - 1) / BO_W;
  const int c0 = min(n, w * chunk), c1 = min(n, c0 + chunk);
  for (int e = c0 + lane; e < c1; e += 64) atomicAdd(&cnt[w][order_bin(fs, fs.items[lo + e], k)], 1);
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
    int run = 0;
    for (int d = 0; d < (int)threadIdx.x; d++) run += btot[d];
    for (int q = 0; q < BO_W; q++) {
      const int c = cnt[q][threadIdx.x];
      cnt[q][threadIdx.x] = run;
      run += c;
    }
  }
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int base = c0; base < c1; base += 64) {
    const int e = base + lane;
    const bool valid = e < c1;
    const int it = valid ? fs.items[lo + e] : 0;
    const uint32_t d = valid ? order_bin(fs, it, k) : 0u;
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

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d, GS_WAVE));
  return wave_first(v);
}

constexpr int BATCH = GS_WAVE;  // splats per staged batch

// Two-stage load pipeline for the back-to-front walk: the ids of the batch
// after next and the records of the next batch are in flight while a batch is
// processed. Slots outside the range carry id -1 (and read record 0).
__device__ __forceinline__ int load_id(const int32_t *__restrict__ sids, int lo, int hi) {
  const int e = lo + __lane_id();
  return e < hi ? sids[e] : -1;
}

// Walk positions [cs, cs + kmax) back to front for one quarter. Lane state:
// T (transmittance after the lane's last consumed entry), accum, and lastp,
// the number of entries the lane consumed from cs. Each staged record carries
// 1/o, 2b and log2(o) in place of o, depth and pad, so the per-entry work has
// no reciprocal of o, no doubling and no logarithm.
__device__ __forceinline__ void walk_back(const Splat *__restrict__ splats,
                                          const int32_t *__restrict__ sids, int cs, int kmax,
                                          const SubTile &st, float fx, float fy, int lastp,
                                          float T, float accum, float g0, float g1, float g2,
                                          Splat *sbuf, int *sid, float *__restrict__ grads) {
  const int lane = __lane_id();
  const int comp = comp_of_lane(lane);
  // the constant factor each owner lane applies to its sum after the reduction
  // (a power of two: exact): -1/2 for the two squared offsets
  const float post = (comp == 2 || comp == 4) ? -0.5f : 1.0f;
  int hiE = cs + kmax;
  int lo = max(cs, hiE - BATCH);
  int idc = -1, idn = -1;
  // the next batch's record of this lane, as three registers of four (kept out
  // of any aggregate: the compiler parked part of one in memory and waited for
  // its load right after issuing it)
  const float4 *rec4 = reinterpret_cast<const float4 *>(splats);
  float4 r0 = make_float4(0.f, 0.f, 0.f, 0.f), r1 = r0, r2 = r0;
  if (hiE > cs) {
    idc = load_id(sids, lo, hiE);
    const int64_t ri = 3 * (int64_t)(idc >= 0 ? idc : 0);
    r0 = rec4[ri];
    r1 = rec4[ri + 1];
    r2 = rec4[ri + 2];
    idn = load_id(sids, max(cs, lo - BATCH), lo);
  }
  while (hiE > cs) {
    Splat s;
    s.p0 = r0;
    s.p1 = r1;
    s.p2 = r2;
    const bool cand = idc >= 0 && rect_may_hit(s.p0.x, s.p0.y, s.p0.z, s.p0.w, s.p1.x, s.p2.y,
                                                st.hx0, st.hx1, st.hy0, st.hy1);
    s.p2.w = __log2f(s.p1.y);  // the forward pass folds log2(o) the same way
    s.p2.z = 2.0f * s.p0.w;
    s.p1.y = __builtin_amdgcn_rcpf(s.p1.y);
    sbuf[lane] = s;
    sid[lane] = idc;
    const uint64_t work = wave_ballot(cand);
    const int nhi = lo, nlo = max(cs, lo - BATCH);
    // records of [nlo, nhi), ids of the batch below it
    idc = idn;
    {
      const int64_t ri = 3 * (int64_t)(idc >= 0 ? idc : 0);
      r0 = rec4[ri];
      r1 = rec4[ri + 1];
      r2 = rec4[ri + 2];
    }
    idn = load_id(sids, max(cs, nlo - BATCH), nlo);
    wave_sync();
    const int base = lo - cs;
    walk_worklist<true>(work, sbuf, [&](const Splat &s, int j) {
      const int rel = base + j;
      const float a = s.p0.z, b = s.p0.w, c = s.p1.x;
      const float dx = fx - s.p0.x, dy = fy - s.p0.y;
      const float adx = a * dx, cdy = c * dy;
      // canon_q with the staged 2b
      const float q = __builtin_fmaf(cdy, dy, __builtin_fmaf(s.p2.z * dx, dy, adx * dx));
      const bool inr = rel < lastp, inq = q <= s.p2.y;
      if (!(wave_ballot(inr) & wave_ballot(inq))) return true;
      const bool hit = inr && inq;
      // branchless: a missed pixel takes alpha = 0, which leaves T and accum
      // unchanged and contributes zero to every sum
      const float ex = __builtin_amdgcn_exp2f(__builtin_fmaf(q, NEG_HALF_LOG2E, s.p2.w));
      const float oG = hit ? ex : 0.0f;  // o G
      const float al = fminf(0.99f, oG);
      T = T * __builtin_amdgcn_rcpf(1.0f - al);  // T before this splat
      const float cg = __builtin_fmaf(s.p1.z, g0, __builtin_fmaf(s.p1.w, g1, s.p2.x * g2));
      const float diff = cg - accum;
      const float dal = T * diff;  // dL/dalpha
      accum = __builtin_fmaf(al, diff, accum);
      const float w = al * T;
      const bool live_g = oG < 0.99f;  // a clamped alpha passes no gradient
      // -2 dL/dq, which is also o G dL/dalpha: an unclamped alpha is o G
      const float m = live_g ? al * dal : 0.0f;
      float gr[9];
      gr[0] = m * __builtin_fmaf(b, dy, adx);  // dq/dmx = -2 (a dx + b dy)
      gr[1] = m * __builtin_fmaf(b, dx, cdy);
      gr[2] = m * (dx * dx);                   // times -1/2 after the sum
      gr[3] = -(m * (dx * dy));
      gr[4] = m * (dy * dy);                   // times -1/2 after the sum
      gr[5] = m;                               // divided by o after the sum
      gr[6] = w * g0;
      gr[7] = w * g1;
      gr[8] = w * g2;
      float out = reduce_scatter9(gr);
      // finish the sum here, where its last exchange fuses into the add,
      // rather than inside the owner lanes' branch
      __asm__ volatile("" : "+v"(out));
      out *= comp == 5 ? s.p1.y : post;
      if (comp >= 0) unsafeAtomicAdd(&grads[9 * (int64_t)sid[j] + comp], out);
      return true;
    });
    wave_sync();
    hiE = nhi;
    lo = nlo;
  }
}

__global__ void __launch_bounds__(GS_WAVE * GS_WAVES_PER_BLOCK)
__attribute__((amdgpu_waves_per_eu(4))) k_render_bwd(
    const Splat *__restrict__ splats, const int32_t *__restrict__ sorted_ids,
    const int2 *__restrict__ ranges, CamK cam, const float *__restrict__ Tfin,
    const int32_t *__restrict__ last, char *__restrict__ state, int ntiles,
    const float *__restrict__ dL, const float *__restrict__ dT, float *__restrict__ grads) {
  __shared__ Splat sbuf_all[GS_WAVES_PER_BLOCK][BATCH];
  __shared__ int sid_all[GS_WAVES_PER_BLOCK][BATCH];
  Splat *sbuf = sbuf_all[wave_in_block()];
  int *sid = sid_all[wave_in_block()];
  FwdState fs = fwd_state_at(state, ntiles);
  const int k = fs.hdr->k;
  const int64_t P = (int64_t)cam.width * cam.height * cam.views;
  const int lane = __lane_id();
  __shared__ uint32_t drained;
  Worker wk = make_worker(&drained);
  for (;;) {
    const int t = next_item(fs, 1, wk);
    if (t < 0) break;
    wk.round++;
    const int it = fs.bitems[t];
    const int kind = item_kind(it), quad = item_quad(it), p = item_chunk(it);
    const int idx = item_index(it);
    const int tile = kind == ITEM_PLAIN ? idx : fs.order[idx];
    const SubTile st = subtile_of(tile, quad, cam);
    if (st.empty) continue;
    const int px = st.x0 + (lane & 7), py = st.y0 + (lane >> 3);
    const bool inside = px < cam.width && py < cam.height;
    const int64_t pix = (int64_t)(st.prow + py) * cam.width + px;
    const int2 rg = ranges[tile];
    float g0 = 0.f, g1 = 0.f, g2 = 0.f;
    // what lies behind the last blended splat, per unit of final transmittance:
    // the background's bg . dL/dC and dL/dT_final (0 when neither is given)
    float extra = 0.f;
    if (inside) {
      g0 = dL[pix];
      g1 = dL[P + pix];
      g2 = dL[2 * P + pix];
      if (cam.bg_on) {
        extra = fmaf(cam.bg[0], g0, fmaf(cam.bg[1], g1, cam.bg[2] * g2));
        if (dT) extra += dT[pix];
      }
    }
    const float fx = (float)px + 0.5f, fy = (float)py + 0.5f;
    if (kind == ITEM_PLAIN) {
      float T = 1.0f;
      int lastp = 0;
      if (inside) {
        T = Tfin[pix];
        lastp = last[pix];
      }
      const int kmax = min(wave_max(lastp), fs.sub_last[tile * 4 + quad]);
      walk_back(splats, sorted_ids, rg.x, kmax, st, fx, fy, lastp, T, extra, g0, g1, g2, sbuf,
                sid, grads);
      continue;
    }
    // a chunk of a heavy tile
    int cs, ce;
    chunk_range(rg.x, rg.y, p, k, cs, ce);
    const int ci = chunk_index(idx, p, quad, k);
    const int64_t cp = (int64_t)ci * 64 + lane;
    int lb = inside ? fs.LB[cp] : -1;
    float T = 1.0f, accum = 0.0f;
    if (lb > 0) {
      T = fs.TB[cp];
      float behind = 0.0f;  // sum over later chunks of C . dL/dC
      for (int q = p + 1; q < k; q++) {
        const int64_t c2 = (int64_t)chunk_index(idx, q, quad, k) * 64 + lane;
        if (fs.LB[c2] < 0) break;
        behind = __builtin_fmaf(fs.CB[3 * c2], g0,
                                __builtin_fmaf(fs.CB[3 * c2 + 1], g1,
                                               __builtin_fmaf(fs.CB[3 * c2 + 2], g2, behind)));
      }
      if (cam.bg_on) behind = fmaf(Tfin[pix], extra, behind);
      accum = behind / T;
    } else {
      lb = 0;
    }
    const int kmax = min(wave_max(lb), fs.chunk_last[ci]);
    walk_back(splats, sorted_ids, cs, kmax, st, fx, fy, lb, T, accum, g0, g1, g2, sbuf, sid,
              grads);
  }
}

}  // namespace

hipError_t gs_launch_render_bwd(const float *splats, const int32_t *sorted_ids,
                                const int32_t *ranges, const CamK &cam, const float *T,
                                const int32_t *last, void *fwd_state, const float *dL,
                                const float *dT, float *grads, int n, int workers_waves,
                                hipEvent_t ev0, hipEvent_t ev1, hipStream_t st) {
  const int64_t ng = 9 * (int64_t)n;
  const int ntiles = cam.tiles_x * cam.tiles_y;
  const int nblocks = workers_waves / GS_WAVES_PER_BLOCK;
  const int zero_blocks = (int)((ng / 4 + 4 + BO_T - 1) / BO_T);
  hipLaunchKernelGGL(k_bwd_prep, dim3(GS_GROUPS + zero_blocks), dim3(BO_T), 0, st,
                     reinterpret_cast<char *>(fwd_state), ntiles, nblocks, grads, ng);
  if (ev0) {
    const hipError_t e = hipEventRecord(ev0, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_render_bwd, dim3(nblocks),
                     dim3(GS_WAVE * GS_WAVES_PER_BLOCK), 0, st,
                     reinterpret_cast<const Splat *>(splats), sorted_ids,
                     reinterpret_cast<const int2 *>(ranges), cam, T, last,
                     reinterpret_cast<char *>(fwd_state), ntiles, dL, dT, grads);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && ev1) e = hipEventRecord(ev1, st);
  return e;
}
