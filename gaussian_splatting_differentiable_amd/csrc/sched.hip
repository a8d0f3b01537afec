// Per-frame tile schedule: longest-processing-time order, the chunking policy
// and the work queues of the persistent raster kernels.
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
// and this TU is compiled with -ffp-contract=off, so a host copy of the policy
// returns the same (h, k).
//
// One workgroup of 1024 threads does everything; T <= 65535 tiles.
#include "render_common.h"

namespace {

constexpr int NT = 1024, NW = NT / 64;

__device__ __forceinline__ uint32_t block_max(uint32_t v) {
  __shared__ uint32_t ws[NW];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, d, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < NW; w++) t = max(t, ws[w]);
  __syncthreads();
  return t;
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
  // offsets in (digit, wave) order: within a digit over the waves, then the
  // digit totals scanned by the whole block
  int dtot = 0;
  if (threadIdx.x < 256) {
    for (int q = 0; q < NW; q++) {
      const int c = cnt[q][threadIdx.x];
      cnt[q][threadIdx.x] = dtot;
      dtot += c;
    }
  }
  int all;
  const int dbase = block_excl_scan<int>(dtot, all);
  if (threadIdx.x < 256)
    for (int q = 0; q < NW; q++) cnt[q][threadIdx.x] += dbase;
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

__global__ void __launch_bounds__(NT) k_schedule(const int2 *__restrict__ ranges, int T, int tiles_x,
                                                 int chunk_mode, int force_k, int force_h,
                                                 double lambda_, double beta, double eps,
                                                 int nblocks, char *__restrict__ fwd_state,
                                                 unsigned long long *__restrict__ stats) {
  FwdState fs = fwd_state_at(fwd_state, T);
  const double workers = (double)(nblocks * GS_WAVES_PER_BLOCK) / 4.0;  // four waves per tile
  uint32_t *tmp_k = reinterpret_cast<uint32_t *>(fs.items);
  int32_t *tmp_v = fs.items + T;
  uint32_t *key = reinterpret_cast<uint32_t *>(fs.counts);
  // 1. counts and the (bit-limited) descending key
  uint32_t mx = 0;
  for (int t0 = threadIdx.x; t0 < T; t0 += NT * RB_ROUNDS) {
    int2 rr[RB_ROUNDS];
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++) {
      const int t = t0 + r * NT;
      rr[r] = t < T ? ranges[t] : make_int2(0, 0);
    }
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++) {
      const int t = t0 + r * NT;
      if (t < T) {
        const uint32_t c = (uint32_t)max(0, rr[r].y - rr[r].x);
        key[t] = c;
        fs.order[t] = t;
        mx = max(mx, c);
      }
    }
  }
  mx = block_max(mx);
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
    block_radix_pass(even ? key : tmp_k, even ? fs.order : tmp_v, even ? tmp_k : key,
                     even ? tmp_v : fs.order, T, 8 * pass);
  }
  if (npass & 1) {
    for (int t = threadIdx.x; t < T; t += NT) {
      key[t] = tmp_k[t];
      fs.order[t] = tmp_v[t];
    }
    __syncthreads();
  }
  for (int t0 = threadIdx.x; t0 < T; t0 += NT * RB_ROUNDS) {
    uint32_t kk[RB_ROUNDS];
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++) kk[r] = t0 + r * NT < T ? key[t0 + r * NT] : 0u;
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++)
      if (t0 + r * NT < T) fs.counts[t0 + r * NT] = (int32_t)(full - kk[r]);
  }
  __syncthreads();

  // 3. chunking policy
  int h = 0, k = 1;
  if (chunk_mode == 2) {
    k = force_k <= 2 ? 2 : (force_k <= 4 ? 4 : (force_k <= 8 ? 8 : 16));
    h = force_h <= 0 ? T : min(force_h, T);
    h = min(h, GS_HK_MAX / k);
  } else if (chunk_mode == 1 && T > 0) {
    constexpr int HMAX = GS_HK_MAX / 2;  // the largest h of any candidate
    __shared__ long long sS[HMAX + 1];   // sS[h] = N_1 + ... + N_h (exact)
    __shared__ int sN[HMAX + 1];         // sN[h] = N_{h+1} (0 past the last tile)
    __shared__ double s_best[NT];
    __shared__ int s_idx[NT];
    long long total_ll = 0;
    for (int t = threadIdx.x; t < T; t += NT) total_ll += fs.counts[t];
    long long tot;
    (void)block_excl_scan<long long>(total_ll, tot);
    {
      static_assert(HMAX == 2 * NT, "two prefix entries per thread");
      const int i0 = 2 * threadIdx.x;
      const long long a = i0 < T ? fs.counts[i0] : 0, b = i0 + 1 < T ? fs.counts[i0 + 1] : 0;
      long long all;
      const long long before = block_excl_scan<long long>(a + b, all);
      sS[i0 + 1] = before + a;
      sS[i0 + 2] = before + a + b;
      sN[i0] = (int)a;
      sN[i0 + 1] = (int)b;
      if (threadIdx.x == 0) {
        sS[0] = 0;
        sN[HMAX] = HMAX < T ? fs.counts[HMAX] : 0;
      }
    }
    __syncthreads();
    const double Nt = (double)tot, N1 = (double)fs.counts[0];
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
    s_best[threadIdx.x] = best;
    s_idx[threadIdx.x] = bidx;
    __syncthreads();
    for (int sft = NT / 2; sft > 0; sft >>= 1) {
      if ((int)threadIdx.x < sft) {
        const double ob = s_best[threadIdx.x + sft];
        const int oi = s_idx[threadIdx.x + sft];
        if (ob < s_best[threadIdx.x] || (ob == s_best[threadIdx.x] && oi < s_idx[threadIdx.x])) {
          s_best[threadIdx.x] = ob;
          s_idx[threadIdx.x] = oi;
        }
      }
      __syncthreads();
    }
    const int bi = s_idx[0];
    if (bi != 0x7FFFFFFF && s_best[0] <= (1.0 - eps) * T0) {
      const int q = bi < off[1] ? 0 : (bi < off[2] ? 1 : (bi < off[3] ? 2 : 3));
      k = 2 << q;
      h = bi - off[q] + 1;
    }
    __syncthreads();
  }
  if (h == 0) k = 1;

  // 4. queues. The LPT positions e in [0, T) fall into classes (group of the
  //    tile, chunked iff e < h); a stable partition by class keeps the LPT order
  //    inside every class. The per-quarter bounds array (written by the forward
  //    pass later) holds the partition's temporaries.
  uint32_t *ck = reinterpret_cast<uint32_t *>(fs.sub_last);
  int32_t *cv = fs.sub_last + T;
  uint32_t *ck2 = reinterpret_cast<uint32_t *>(fs.sub_last + 2 * T);
  int32_t *perm = fs.sub_last + 3 * T;
  __shared__ int ccount[NCLS], cstart[NCLS], qoff[GS_GROUPS + 1];
  if (threadIdx.x < NCLS) ccount[threadIdx.x] = 0;
  __syncthreads();
  for (int e0 = threadIdx.x; e0 < T; e0 += NT * RB_ROUNDS) {
    int tl[RB_ROUNDS];
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++) {
      const int e = e0 + r * NT;
      tl[r] = e < T ? fs.order[e] : 0;
    }
#pragma unroll
    for (int r = 0; r < RB_ROUNDS; r++) {
      const int e = e0 + r * NT;
      if (e < T) {
        const uint32_t c = 2u * (uint32_t)tile_group(tl[r], tiles_x) + (e >= h ? 1u : 0u);
        ck[e] = c;
        cv[e] = e;
        atomicAdd(&ccount[c], 1);
      }
    }
  }
  __syncthreads();
  block_radix_pass(ck, cv, ck2, perm, T, 0);
  if (threadIdx.x == 0) {
    int run = 0, q = 0;
    for (int c = 0; c < NCLS; c++) {
      cstart[c] = run;
      run += ccount[c];
    }
    for (int g = 0; g < GS_GROUPS; g++) {
      qoff[g] = q;
      q += 8 * k * ccount[2 * g] + 4 * ccount[2 * g + 1];
    }
    qoff[GS_GROUPS] = q;
  }
  __syncthreads();
  for (int i0 = threadIdx.x; i0 < T; i0 += NT * RB_ROUNDS) {
    int ee[RB_ROUNDS], cc[RB_ROUNDS], tl[RB_ROUNDS];
#pragma unroll
    for (int u = 0; u < RB_ROUNDS; u++) {
      const int i = i0 + u * NT;
      ee[u] = i < T ? perm[i] : 0;
      cc[u] = i < T ? (int)ck2[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < RB_ROUNDS; u++) tl[u] = fs.order[ee[u]];
#pragma unroll
    for (int u = 0; u < RB_ROUNDS; u++) {
    const int i = i0 + u * NT;
    if (i >= T) continue;
    const int e = ee[u];
    const int c = cc[u];
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
      const int tile = tl[u];
      for (int q = 0; q < 4; q++) fs.items[p0 + q] = make_item(ITEM_PLAIN, q, 0, tile);
    }
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
    queue_head(fs, 1, g)[0] = init_b;
  }
  if (threadIdx.x <= GS_GROUPS) fs.hdr->qoff[threadIdx.x] = qoff[threadIdx.x];
  if (threadIdx.x == 0) {
    fs.hdr->h = h;
    fs.hdr->k = k;
    fs.hdr->nA = nA;
    fs.hdr->nplain = 4 * (T - h);
    fs.hdr->err = 0;
    fs.hdr->ntiles = T;
    if (stats) atomicAdd(&stats[3], (unsigned long long)h);
  }
}

}  // namespace

hipError_t gs_launch_schedule(const int32_t *ranges, const CamK &cam, int chunk_mode, int force_k,
                              int force_h, double lambda_, double beta, double eps, int nblocks,
                              void *fwd_state, int64_t *stats, hipStream_t st) {
  const int T = cam.tiles_x * cam.tiles_y;
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(NT), 0, st, reinterpret_cast<const int2 *>(ranges), T,
                     cam.tiles_x, chunk_mode, force_k, force_h, lambda_, beta, eps, nblocks,
                     reinterpret_cast<char *>(fwd_state),
                     reinterpret_cast<unsigned long long *>(stats));
  return hipGetLastError();
}
