// Host check of the work-item plan shared by both kernels and the host
// mirror (xqa_internal.h): for every tested (blocks per head, workgroups
// per head) the items are non-empty, tile [0, NB) in order, and
// item_of_block inverts item_lo; then the cost-stream plan the kernels use
// over random batches. Exits non-zero on the first violation.
#include <cstdio>
#include <cstdlib>
#include <vector>

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

// The cost-stream plan over explicit lengths: each item's block range from
// its two cost ends. Checks that the items tile [0, NB) in order, that each
// holds at least one block, that the cost of every item is within one unit
// of C / P, that with short sequences every item's cost range is at least
// kSeqStartCost + 1 units long whenever P > 1, and that without them the
// items are the block plan's.
static int check_costs(const std::vector<int>& lens, int per_head) {
  const int max_tokens = 1 << 24;
  std::vector<long long> nb, cost, off(1, 0), coff(1, 0);
  for (int n : lens) {
    const int blocks = xqa::seq_blocks(xqa::clamp_len(n, max_tokens));
    nb.push_back(blocks);
    off.push_back(off.back() + blocks);
  }
  const long long NB = off.back();
  const int P = xqa::items_per_head(NB, per_head);
  for (long long blocks : nb) {
    // The division-free test is 0 < blocks < floor(NB / P).
    const bool charged = P > 0 && blocks > 0 && blocks < NB / P;
    if (xqa::seq_charged((int)blocks, NB, P) != charged) {
      std::printf("FAIL seq_charged blocks=%lld NB=%lld P=%d\n", blocks, NB, P);
      return 1;
    }
    cost.push_back(xqa::seq_cost((int)blocks, NB, P));
    coff.push_back(coff.back() + cost.back());
  }
  const long long C = coff.back();
  auto fail = [&](const char* what, long long v) {
    std::printf("FAIL cost plan batch=%zu per_head=%d P=%d: %s (%lld)\n", lens.size(), per_head, P,
                what, v);
    return 1;
  };
  auto block_at = [&](long long c) {
    if (c >= C) return NB;
    for (size_t b = 0; b < lens.size(); ++b)
      if (cost[b] > 0 && c >= coff[b] && c < coff[b] + cost[b]) {
        const long long local = c - coff[b] - (cost[b] - nb[b]);
        return off[b] + (local > 0 ? local : 0);
      }
    return -1LL;
  };
  if (NB == 0) return P == 0 ? 0 : fail("items without blocks", P);
  long long prev = 0;
  for (int i = 0; i < P; ++i) {
    const long long clo = xqa::item_lo(i, C, P), chi = xqa::item_lo(i + 1, C, P);
    const long long lo = block_at(clo), hi = block_at(chi);
    if (lo != prev) return fail("items do not tile", i);
    if (hi <= lo) return fail("item without a block", i);
    if (chi - clo < C / P || chi - clo > (C + P - 1) / P) return fail("unbalanced cost", i);
    // With a charged sequence, no item's cost range fits inside a charge.
    if (P > 1 && C > NB && chi - clo < xqa::kSeqStartCost + 1)
      return fail("cost range too short", i);
    // Without short sequences the items are the plain block plan's.
    if (C == NB && (lo != xqa::item_lo(i, NB, P) || hi != xqa::item_lo(i + 1, NB, P)))
      return fail("not the block plan", i);
    prev = hi;
  }
  return prev == NB ? 0 : fail("items end before NB", prev);
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
  // Cost-stream plans over random batches: short, long, empty and mixed lengths.
  unsigned long long x = 12345;
  auto rnd = [&](int m) {
    x = x * 6364136223846793005ULL + 1442695040888963407ULL;
    return (int)((x >> 33) % (unsigned long long)m);
  };
  const int lens_pool[] = {0, 1, 15, 16, 17, 31, 32, 33, 255, 257, 1025, 4097, 65536, 262144};
  for (int t = 0; t < 4000; ++t, ++cases) {
    const int batch = 1 + rnd(t % 3 == 0 ? 8 : 200);
    std::vector<int> lens(batch);
    for (int& n : lens) n = t % 2 ? lens_pool[rnd(14)] : rnd(3000) - 5;
    if (check_costs(lens, per_heads[rnd(12)])) return 1;
  }
  std::printf("OK %lld plans\n", cases);
  return 0;
}
