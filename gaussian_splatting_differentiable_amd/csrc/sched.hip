// Per-frame tile schedule: longest-processing-time order, the chunking policy
// and the persistent work queue.
//
// "Mitigating SM-Level Load Imbalance in 3D Gaussian Splatting on GPUs":
// section 4.1 orders the tiles by descending pair count N_t (a radix sort of the
// tile indices that leaves the Gaussian data in place); section 4.3 chunks the
// heaviest tiles and schedules the rest in that order; section 4.4, Eq. 6 picks
// the number of chunked tiles h and chunks per tile k per frame:
//   l(h,k) = max(N_1/k, N_{h+1});  T(h,k) = max((N_total + lambda h k)/K, l) + beta l,
// k in {2,4,8,16}, first strict minimum over (k, h), enabled only when at least
// eps below the no-chunking estimate. Here h k is also capped at GS_HK_MAX.
// The policy arithmetic is fp64 in one fixed order and this TU is compiled with
// -ffp-contract=off, so a host copy of the policy returns the same (h, k).
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

// One stable LSD pass (8-bit digit at `shift`) of (key, val) over n elements in
// global memory, by one workgroup. Wave w owns the contiguous chunk
// [w*chunk, (w+1)*chunk); a first sweep counts digits per wave, a second sweep
// ranks each round of 64 with a ballot match and scatters.
__device__ void block_radix_pass(const uint32_t *kin, const int32_t *vin, uint32_t *kout,
                                 int32_t *vout, int n, int shift) {
  __shared__ int cnt[NW][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < NW * 256; i += NT) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int chunk = (n + NW - 1) / NW;
  const int c0 = min(n, w * chunk), c1 = min(n, c0 + chunk);
  for (int e = c0 + lane; e < c1; e += 64) atomicAdd(&cnt[w][(kin[e] >> shift) & 255], 1);
  __syncthreads();
  // exclusive offsets in (digit, wave) order
  __shared__ int dtot[256];
  if (threadIdx.x < 256) {
    int tot = 0;
    for (int q = 0; q < NW; q++) {
      const int c = cnt[q][threadIdx.x];
      cnt[q][threadIdx.x] = tot;
      tot += c;
    }
    dtot[threadIdx.x] = tot;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int d = 0; d < 256; d++) {
      const int t = dtot[d];
      dtot[d] = run;
      run += t;
    }
  }
  __syncthreads();
  if (threadIdx.x < 256)
    for (int q = 0; q < NW; q++) cnt[q][threadIdx.x] += dtot[threadIdx.x];
  __syncthreads();
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int base = c0; base < c1; base += 64) {
    const int e = base + lane;
    const bool valid = e < c1;
    const uint32_t k = valid ? kin[e] : 0u;
    const int32_t v = valid ? vin[e] : 0;
    const uint32_t d = (k >> shift) & 255u;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; b++) {
      const uint64_t bal = __ballot((d >> b) & 1u);
      peers &= ((d >> b) & 1u) ? bal : ~bal;
    }
    if (valid) {
      const int below = __popcll(peers & lt);
      const int pos = cnt[w][d] + below;
      kout[pos] = k;
      vout[pos] = v;
      if (below == __popcll(peers) - 1) cnt[w][d] = pos + 1;
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(NT) k_schedule(const int2 *__restrict__ ranges, int T, int tiles_x,
                                                 int chunk_mode, int force_k, int force_h,
                                                 double lambda_, double beta, double eps,
                                                 double workers, char *__restrict__ fwd_state,
                                                 unsigned long long *__restrict__ stats) {
  FwdState fs = fwd_state_at(fwd_state, T);
  uint32_t *tmp_k = reinterpret_cast<uint32_t *>(fs.items);
  int32_t *tmp_v = fs.items + T;
  uint32_t *key = reinterpret_cast<uint32_t *>(fs.counts);
  // 1. counts and the (bit-limited) descending key
  uint32_t mx = 0;
  for (int t = threadIdx.x; t < T; t += NT) {
    const int2 r = ranges[t];
    const uint32_t c = (uint32_t)max(0, r.y - r.x);
    key[t] = c;
    fs.order[t] = t;
    mx = max(mx, c);
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
  for (int t = threadIdx.x; t < T; t += NT) fs.counts[t] = (int32_t)(full - key[t]);
  __syncthreads();

  // 3. chunking policy
  int h = 0, k = 1;
  if (chunk_mode == 2) {
    k = force_k <= 2 ? 2 : (force_k <= 4 ? 4 : (force_k <= 8 ? 8 : 16));
    h = force_h <= 0 ? T : min(force_h, T);
    h = min(h, GS_HK_MAX / k);
  } else if (chunk_mode == 1 && T > 0) {
    __shared__ double s_best[NT];
    __shared__ int s_idx[NT];
    long long total_ll = 0;
    for (int t = threadIdx.x; t < T; t += NT) total_ll += fs.counts[t];
    __shared__ long long s_tot[NW];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) total_ll += __shfl_xor(total_ll, d, 64);
    if ((threadIdx.x & 63) == 0) s_tot[threadIdx.x >> 6] = total_ll;
    __syncthreads();
    long long tot = 0;
    for (int w = 0; w < NW; w++) tot += s_tot[w];
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
      const double next = hh < T ? (double)fs.counts[hh] : 0.0;
      const double l = fmax(N1 / (double)kk, next);
      const double avg = (Nt + (lambda_ * (double)hh) * (double)kk) / workers;
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

  // 4. queues: pass-A chunk items, pass-B chunk items, then the quarters of the
  //    other tiles grouped by image strip (a stable partition of the LPT order)
  const int nA = 4 * h * k;
  for (int i = threadIdx.x; i < nA; i += NT) {
    const int s = i / (4 * k), rem = i % (4 * k);
    const int p = rem >> 2, q = rem & 3;
    fs.items[i] = make_item(ITEM_PASS_A, q, p, s);
    fs.items[nA + i] = make_item(ITEM_PASS_B, q, p, s);
    fs.doneA[i] = 0;
  }
  __shared__ int gcnt[GS_GROUPS][NT];
  __shared__ int goff[GS_GROUPS + 1];
  const int rest = T - h;
  const int seg = (rest + NT - 1) / NT;
  const int e0 = h + min(rest, (int)threadIdx.x * seg), e1 = h + min(rest, ((int)threadIdx.x + 1) * seg);
  for (int g = 0; g < GS_GROUPS; g++) gcnt[g][threadIdx.x] = 0;
  for (int e = e0; e < e1; e++) gcnt[tile_group(fs.order[e], tiles_x)][threadIdx.x]++;
  __syncthreads();
  if (threadIdx.x < GS_GROUPS) {
    int run = 0;
    for (int t = 0; t < NT; t++) {
      const int c = gcnt[threadIdx.x][t];
      gcnt[threadIdx.x][t] = run;
      run += c;
    }
    goff[threadIdx.x + 1] = run;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    goff[0] = 0;
    for (int g = 0; g < GS_GROUPS; g++) goff[g + 1] += goff[g];
  }
  __syncthreads();
  for (int e = e0; e < e1; e++) {
    const int tile = fs.order[e];
    const int g = tile_group(tile, tiles_x);
    const int pos = 2 * nA + 4 * (goff[g] + gcnt[g][threadIdx.x]++);
    for (int q = 0; q < 4; q++) fs.items[pos + q] = make_item(ITEM_PLAIN, q, 0, tile);
  }
  for (int i = threadIdx.x; i < 4 * h; i += NT) {
    fs.sat[i] = k;
    fs.doneB[i] = 0;
  }
  for (int i = threadIdx.x; i < 2 * (GS_GROUPS + 1); i += NT) fs.heads[i * GS_HEAD_STRIDE] = 0;
  if (threadIdx.x <= GS_GROUPS) fs.hdr->qoff[threadIdx.x] = 4 * goff[threadIdx.x];
  if (threadIdx.x == 0) {
    fs.hdr->h = h;
    fs.hdr->k = k;
    fs.hdr->nA = nA;
    fs.hdr->nplain = 4 * rest;
    fs.hdr->err = 0;
    fs.hdr->ntiles = T;
    if (stats) atomicAdd(&stats[3], (unsigned long long)h);
  }
}

}  // namespace

hipError_t gs_launch_schedule(const int32_t *ranges, const CamK &cam, int chunk_mode, int force_k,
                              int force_h, double lambda_, double beta, double eps, double workers,
                              void *fwd_state, int64_t *stats, hipStream_t st) {
  const int T = cam.tiles_x * cam.tiles_y;
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(NT), 0, st, reinterpret_cast<const int2 *>(ranges), T,
                     cam.tiles_x, chunk_mode, force_k, force_h, lambda_, beta, eps, workers,
                     reinterpret_cast<char *>(fwd_state),
                     reinterpret_cast<unsigned long long *>(stats));
  return hipGetLastError();
}
