/* Oracle: per-frame chunking policy. TEST INFRASTRUCTURE ONLY.
 *
 * [LOAD-IMB] section 4.4, Eq. 6 (garbled in extraction; reading below).
 * With tile counts N_1 >= N_2 >= ... and N_total = sum_t N_t, chunking the h
 * heaviest tiles into k chunks each costs an average-workload term
 * (N_total + lambda h k) / K over K concurrent workers; the longest remaining
 * unit is l(h, k) = max(N_1 / k, N_{h+1}); the estimate is
 *   T(h, k) = max((N_total + lambda h k) / K, l) + beta l.
 * The policy searches k in {2, 4, 8, 16} and h = 1..T, keeps the first strict
 * minimum (k ascending, then h ascending), and chunks only if that minimum is at
 * least eps (10%) below the no-chunking estimate T(0) = max(N_total / K, N_1) + beta N_1.
 * Candidates are limited to h k <= max_items (the number of chunk partials a frame
 * can hold).
 * All arithmetic is fp64 in this exact order, so a device copy can match it bit
 * for bit. lambda and beta are not printed on the page: parity for their values
 * is unpinned.
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
    for (int h = 1; h <= ntiles && h * k <= max_items; h++) {
      const double next = h < ntiles ? (double)counts_desc[h] : 0.0;
      const double l = fmax(N1 / (double)k, next);
      const double avg = (Nt + (lambda_ * (double)h) * (double)k) / workers;
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
