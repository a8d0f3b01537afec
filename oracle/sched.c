/* Oracle: per-frame chunking policy. TEST INFRASTRUCTURE ONLY.
 *
 * [LOAD-IMB] section 4.4, Eq. 6 (garbled in extraction; reading below), with
 * the cost of exact chunk composition folded in.
 * With tile counts N_1 >= N_2 >= ... and N_total = sum_t N_t, the page's model
 * charges the average workload over K concurrent workers plus a fixed cost
 * lambda per chunk, and the longest remaining unit:
 *   T(h, k) = max(avg, l) + beta l.
 * Chunks here are composed exactly (a transmittance pass over every chunk,
 * then a blending pass from the exact incoming transmittance), so a split tile
 * is walked twice and a chunk's blending waits for the transmittance of the
 * chunks in front of it. The model therefore charges
 *   avg = ((N_total + S_h) + lambda h k) / K,  S_h = N_1 + ... + N_h,
 *   l   = max(2 N_1 / k, N_{h+1}).
 * The policy searches k in {2, 4, 8, 16} and h = 1..T, keeps the first strict
 * minimum (k ascending, then h ascending), and chunks only if that minimum is at
 * least eps (10%) below the no-chunking estimate T(0) = max(N_total / K, N_1) + beta N_1.
 * Candidates are limited to h k <= max_items (the number of chunk partials a frame
 * can hold).
 * All arithmetic is fp64 in this exact order (S_h summed exactly in int64), so a
 * device copy can match it bit for bit. lambda and beta are not printed on the
 * page: parity for their values is unpinned.
 */
#include <math.h>
#include "oracle.h"
#ifdef _OPENMP
#include <omp.h>
#endif

void or_chunk_policy(int ntiles, const int32_t *counts_desc, double workers, double lambda_,
                     double beta, double eps, int max_items, int32_t *h_out, int32_t *k_out) {
  *h_out = 0;
  *k_out = 1;
  if (ntiles <= 0) return;
  int64_t total = 0;
  for (int t = 0; t < ntiles; t++) total += counts_desc[t];
  const double Nt = (double)total, N1 = (double)counts_desc[0];
  const double T0 = fmax(Nt / workers, N1) + beta * N1;
  double best = T0;
  int bh = 0, bk = 1;
  for (int k = 2; k <= 16; k *= 2) {
    int64_t Sh = 0;
    for (int h = 1; h <= ntiles && h * k <= max_items; h++) {
      Sh += counts_desc[h - 1];
      const double next = h < ntiles ? (double)counts_desc[h] : 0.0;
      const double l = fmax((2.0 * N1) / (double)k, next);
      const double avg = ((Nt + (double)Sh) + (lambda_ * (double)h) * (double)k) / workers;
      const double est = fmax(avg, l) + beta * l;
      if (est < best) {
        best = est;
        bh = h;
        bk = k;
      }
    }
  }
  if (bh > 0 && best <= (1.0 - eps) * T0) {
    *h_out = bh;
    *k_out = bk;
  }
}

/* Number of OpenMP threads the oracle's parallel loops use (1 without OpenMP). */
int or_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count of the parallel loops that follow (no effect without OpenMP). */
void or_set_num_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
