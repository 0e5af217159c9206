// Host-side decode planning: how one decode launch splits the pairs of its
// batch into blocks.  Shared by the library and its host-side tests.
#pragma once

#include "oscar_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

namespace oscar {

inline int plan_pages(int64_t n_hist) { return (int)((n_hist + kPage - 1) / kPage); }

// Split policy of one decode launch.  A pair's work is its history pages
// plus its window, worth window_units pages (the window's bytes over a page
// block's bytes, times kWindowCost; kStepWindowCost when the launch also
// appends, since the append then runs on the window block's waves after its
// window).  Pieces of at most P units: a pair gets
// S = ceil(U / P) blocks (at most kMaxSplits, and at most U / wu so that
// only the last split can be window-only), and P is the smallest piece size
// for which all blocks fit in R rounds of the device's resident block slots
// (one decode block fills a compute unit): one round when the batch has no
// more pairs than slots, else kExtraRounds more than the pairs need, so that
// long pairs are cut and rounds even out.  Blocks are dispatched largest
// first (more splits, then more pages).
constexpr double kWindowCost = 1.0, kStepWindowCost = 2.4;
constexpr int kExtraRounds = 0;

inline int window_units(int d, int G, bool fused = false) {
  return (int)std::lround((fused ? kStepWindowCost : kWindowCost) * kWindow * 4 * d / block_bytes_for(d, G));
}
// the same for a BF16-history pool (window and pages cost alike per byte)
inline int window_units_bf16(int d) { return (int)std::lround((double)kWindow * 4 * d / bf16_block_bytes(d)); }

// fused: the launch also appends (len is the length after the append); a
// pair whose append evicts into the history keeps its last page in its last
// split, the block that does the append: S <= (np + wu) / (wu + 1).
inline void plan_splits(DecodeBatch &b, const int32_t *seq_ids, const std::vector<int> &len, int Hkv, int slots, int wu,
                        bool fused = false) {
  std::vector<int> np(b.n);
  int64_t total = 0, umax = 1;
  for (int e = 0; e < b.n; ++e) {
    np[e] = plan_pages(std::max(0, len[e] - kWindow));
    total += np[e];
    umax = std::max<int64_t>(umax, np[e] + wu);
  }
  b.total_pages = (int32_t)total;
  b.win_units = wu;
  b.fused = fused ? 1 : 0;
  b.direct = 0;
  for (int e = 0; e < kMaxBatch; ++e) b.new_page[e] = -1;
  auto splits = [&](int e, int64_t P) {
    if (np[e] == 0) return 1; // window only
    const int64_t U = np[e] + wu;
    int64_t S = std::min<int64_t>(kMaxSplits, (U + P - 1) / P);
    if (wu > 0) S = std::min<int64_t>(S, U / wu);
    if (fused && len[e] - 1 >= kWindow) S = std::min<int64_t>(S, U / (wu + 1));
    return (int)std::max<int64_t>(1, S);
  };
  auto blocks = [&](int64_t P) {
    int64_t nb = 0;
    for (int e = 0; e < b.n; ++e) nb += splits(e, P);
    return nb * Hkv;
  };
  const int64_t pairs = (int64_t)b.n * Hkv;
  const int64_t rounds = pairs <= slots ? 1 : (pairs + slots - 1) / slots + kExtraRounds;
  const int64_t budget = rounds * slots;
  int64_t lo = 1, hi = umax; // blocks(umax) = n * Hkv: the fewest possible
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (blocks(mid) <= budget) hi = mid;
    else lo = mid + 1;
  }
  std::vector<int> S(b.n), order(b.n);
  for (int e = 0; e < b.n; ++e) {
    S[e] = splits(e, lo);
    order[e] = e;
  }
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return S[x] != S[y] ? S[x] > S[y] : np[x] > np[y]; });
  for (int i = 0; i < b.n; ++i) {
    const int e = order[i];
    b.seq[i] = seq_ids[e];
    b.len[i] = len[e];
    b.row[i] = (uint16_t)e;
    b.nsplit[i] = (uint8_t)S[e];
  }
  // layer l holds the pairs of the sequences with more than l splits: the
  // first count(S > l) sequences of the launch order
  b.layer_prefix[0] = 0;
  for (int l = 0; l < kMaxSplits; ++l) {
    int cnt = 0;
    while (cnt < b.n && b.nsplit[cnt] > l) ++cnt;
    b.layer_prefix[l + 1] = b.layer_prefix[l] + cnt * Hkv;
  }
  b.hist_blocks = b.layer_prefix[kMaxSplits];
}

// INT2 decode launches whose pairs all have one split write the output rows
// from the decode blocks (no merge launch).
inline void set_direct(DecodeBatch &b) {
  int one = 1;
  for (int e = 0; e < b.n; ++e) one &= b.nsplit[e] == 1;
  b.direct = one;
}

} // namespace oscar
