// Host-side check of the decode plan (decode_plan.h, oscar_internal.h): for
// random batches, the blocks of a launch cover every pair's history pages
// exactly once and its window exactly once, every index a decode block
// derives from its split stays inside the pair, a fused step's evicting
// pair keeps its last page in the split that holds its window (the block
// that appends), the merge side sees the same splits, and the launch order
// is a permutation of the batch.  Exits non-zero on the first violation.
#include "decode_plan.h"

#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

using namespace oscar;

static int fail(const char *what, int it) {
  std::printf("FAIL (case %d): %s\n", it, what);
  return 1;
}

int main(int argc, char **argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 2000;
  std::mt19937 rng(12345);
  for (int it = 0; it < cases; ++it) {
    DecodeBatch b{};
    const int Hkv = 1 << (rng() % 4);
    b.n = 1 + (int)(rng() % 64);
    std::vector<int32_t> ids(b.n);
    std::vector<int> len(b.n);
    for (int e = 0; e < b.n; ++e) {
      // short (window only), page-aligned and ragged lengths
      const int kind = (int)(rng() % 4);
      int L = kind == 0 ? 1 + (int)(rng() % 330) : 321 + (int)(rng() % 70000);
      if (kind == 1) L = kWindow + kPage * (1 + (int)(rng() % 1200));
      len[e] = L;
      ids[e] = 1000 + e;
    }
    const int slots = 1 + (int)(rng() % 1024);
    const int d = rng() % 2 ? 128 : 64, G = (d == 128 && rng() % 2) ? 128 : 64;
    const bool fused = rng() % 2;
    plan_splits(b, ids.data(), len, Hkv, slots, window_units(d, G, fused), fused);
    std::vector<int> seen_row(b.n, 0);
    for (int e = 0; e < b.n; ++e) {
      if (b.row[e] >= b.n || b.seq[e] != ids[b.row[e]] || b.len[e] != len[b.row[e]])
        return fail("launch order is not the batch", it);
      seen_row[b.row[e]]++;
      if (b.nsplit[e] < 1 || b.nsplit[e] > kMaxSplits) return fail("split count out of range", it);
      if (e > 0 && b.nsplit[e] > b.nsplit[e - 1]) return fail("split counts not descending", it);
    }
    for (int e = 0; e < b.n; ++e)
      if (seen_row[e] != 1) return fail("row not a permutation", it);
    // direct output (no merge launch) exactly when no pair is split
    if (b.direct != 0) return fail("a plan starts without direct output", it);
    set_direct(b);
    {
      bool one = true;
      for (int e = 0; e < b.n; ++e) one = one && b.nsplit[e] == 1;
      if ((b.direct != 0) != one) return fail("direct output with a split pair, or not without one", it);
    }
    if (b.hist_blocks != b.layer_prefix[kMaxSplits]) return fail("block count", it);
    std::vector<std::vector<int>> pages(b.n * Hkv), windows(b.n * Hkv, std::vector<int>(1, 0));
    for (int e = 0; e < b.n; ++e)
      for (int kv = 0; kv < Hkv; ++kv) pages[e * Hkv + kv].assign(plan_pages(std::max(0, b.len[e] - kWindow)), 0);
    for (int blk = 0; blk < b.hist_blocks; ++blk) {
      int s, e, kv;
      block_split(b, Hkv, blk, s, e, kv);
      if (e < 0 || e >= b.n || kv < 0 || kv >= Hkv || s >= b.nsplit[e]) return fail("block maps outside", it);
      if (b.layer_prefix[s] + e * Hkv + kv != blk) return fail("block numbering", it);
      const int S = b.nsplit[e], n_hist = b.len[e] - kWindow;
      const int np = plan_pages(std::max(0, n_hist));
      int p0, p1;
      split_range(np, S, s, b.win_units, p0, p1);
      if (p0 < 0 || p1 > np || p0 > p1) return fail("pages out of range", it);
      if (p0 == p1 && s != S - 1) return fail("empty split that holds no window", it);
      const int pf = full_pages_end(n_hist, p0, p1);
      if (pf < p0 || pf > p1) return fail("full-page end outside the split", it);
      if (pf < p1 && (pf != np - 1 || n_hist % kPage == 0)) return fail("partial page is not the last", it);
      for (int q = p0; q < p1; ++q) pages[e * Hkv + kv][q]++;
      if (s == S - 1) windows[e * Hkv + kv][0]++;
      // a fused step's evicting pair keeps its last page in the split that
      // holds the window (the block that appends)
      if (fused && s == S - 1 && b.len[e] - 1 >= kWindow && !(p0 <= np - 1 && np - 1 < p1))
        return fail("fused step: last page outside the window's split", it);
    }
    for (int i = 0; i < b.n * Hkv; ++i) {
      if (windows[i][0] != 1) return fail("window not held by exactly one block", it);
      for (int c : pages[i])
        if (c != 1) return fail("page not covered exactly once", it);
    }
  }
  std::printf("decode plan ok (%d cases)\n", cases);
  return 0;
}
