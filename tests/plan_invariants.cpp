// Host check of the work-item plan shared by both kernels and the host
// mirror (xqa_internal.h): for every tested (blocks per head, workgroups
// per head) the items are non-empty, tile [0, NB) in order, and
// item_of_block inverts item_lo. Exits non-zero on the first violation.
#include <cstdio>
#include <cstdlib>

#include "xqa_internal.h"

static int check(long long nb, int per_head, bool dense) {
  const int P = xqa::items_per_head(nb, per_head);
  auto fail = [&](const char* what, long long v) {
    std::printf("FAIL nb=%lld per_head=%d P=%d: %s (%lld)\n", nb, per_head, P, what, v);
    return 1;
  };
  if (P < 1 || P > per_head) return fail("item count", P);
  if ((long long)P > (nb + xqa::kMinItemBlocks - 1) / xqa::kMinItemBlocks)
    return fail("items shorter than the minimum", P);
  if (xqa::item_lo(0, nb, P) != 0) return fail("first item start", xqa::item_lo(0, nb, P));
  if (xqa::item_lo(P, nb, P) != nb) return fail("last item end", xqa::item_lo(P, nb, P));
  for (int i = 0; i < P; ++i) {
    const long long lo = xqa::item_lo(i, nb, P), hi = xqa::item_lo(i + 1, nb, P);
    if (hi <= lo) return fail("empty item", i);
    if (hi - lo > (nb + P - 1) / P) return fail("item longer than ceil(NB / P)", i);
    if (xqa::item_of_block(lo, nb, P) != i) return fail("item_of_block(first block)", i);
    if (xqa::item_of_block(hi - 1, nb, P) != i) return fail("item_of_block(last block)", i);
    if (dense) {
      for (long long x = lo; x < hi; ++x)
        if (xqa::item_of_block(x, nb, P) != i) return fail("item_of_block(inner block)", x);
    }
  }
  return 0;
}

int main() {
  const int per_heads[] = {1, 2, 3, 4, 6, 7, 8, 64, 127, 128, 256, 2048};
  long long cases = 0;
  for (int ph : per_heads) {
    for (long long nb = 1; nb <= 5000; ++nb, ++cases)
      if (check(nb, ph, true)) return 1;
    // Up to the largest stream: 65536 sequences of 2^24 tokens = 2^35 blocks.
    const long long big[] = {65536, 1000003, 1ll << 30, 34359738367ll, 1ll << 35};
    for (long long nb : big) {
      ++cases;
      if (check(nb, ph, false)) return 1;
    }
  }
  std::printf("OK %lld plans\n", cases);
  return 0;
}
