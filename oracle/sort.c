/* Oracle: (tile, depth) key order and tile ranges. TEST INFRASTRUCTURE ONLY.
 *
 * Order of the pairs, as [LOAD-IMB] section 2.1 and [3DGS-CUDA] Step 1 (d)
 * define it: (tile id, depth bits, Gaussian id) ascending, where the key packs
 * the tile above the fp32 depth bits (positive depths compare like their bit
 * patterns) and the Gaussian id breaks ties (a reading: the pages leave ties
 * open). The C library qsort over (key, id) is the sorting step.
 */
#include <stdlib.h>
#include <string.h>
#include "oracle.h"

typedef struct {
  uint64_t key;
  int32_t id;
} pair_t;

static int cmp_pair(const void *pa, const void *pb) {
  const pair_t *a = (const pair_t *)pa, *b = (const pair_t *)pb;
  if (a->key != b->key) return a->key < b->key ? -1 : 1;
  if (a->id != b->id) return a->id < b->id ? -1 : 1;
  return 0;
}

void or_sort_pairs(int64_t npairs, const uint64_t *keys, const int32_t *ids,
                   uint64_t *sorted_keys, int32_t *sorted_ids) {
  pair_t *p = (pair_t *)malloc(sizeof(pair_t) * (size_t)(npairs > 0 ? npairs : 1));
  for (int64_t i = 0; i < npairs; i++) {
    p[i].key = keys[i];
    p[i].id = ids[i];
  }
  qsort(p, (size_t)npairs, sizeof(pair_t), cmp_pair);
  for (int64_t i = 0; i < npairs; i++) {
    sorted_keys[i] = p[i].key;
    sorted_ids[i] = p[i].id;
  }
  free(p);
}

/* ranges[2t] = number of pairs with tile < t, ranges[2t+1] = number with tile <= t. */
void or_tile_ranges(int64_t npairs, const uint64_t *sorted_keys, int ntiles, int32_t *ranges) {
  int64_t *cnt = (int64_t *)calloc((size_t)ntiles + 1, sizeof(int64_t));
  for (int64_t i = 0; i < npairs; i++) {
    uint64_t t = sorted_keys[i] >> 32;
    if (t < (uint64_t)ntiles) cnt[t]++;
  }
  int64_t run = 0;
  for (int t = 0; t < ntiles; t++) {
    ranges[2 * t] = (int32_t)run;
    run += cnt[t];
    ranges[2 * t + 1] = (int32_t)run;
  }
  free(cnt);
}
