// The varlen work scheduler of the SegPagedAttention prefill library (host side, g++).
#include "rk_sched.h"

#include <algorithm>

#include "rk_seg.h"

namespace rk {

// Work schedule of one layer (the varlen scheduler).  Items are (seq, kv head, q tile) with cost =
// key tiles visited.  Longest first (LPT) over the whole chip, or, when the long K/V streams do not
// fit the shared cache (below), XCD binning.  Workgroup i of a launch runs on XCD i % kXcd (checked
// on the GPU), and each XCD has its own L2, so items that stream the same K/V should sit on one XCD:
//   1. the items of one (seq, kv head) form a group; a group costlier than 1/(4 kXcd) of the layer is
//      cut into k runs by striding (runs at most a quarter of a bin keep the bins balanced) (item i -> run i % k), so every run spans the group's whole range of
//      item costs (a run of only the longest items would leave its XCD with a few very long items
//      at the end) while all runs still stream the same K/V from the first tile;
//   2. runs go to kXcd bins, costliest first, each to the least loaded bin (LPT);
//   3. each bin runs its items longest first, ties in (seq, kv head, tile) order;
//   4. launch position i takes the next item of bin i % kXcd; a bin that has run dry is padded with
//      an empty item (seq = -1) that the kernel skips.
// When the K/V streams of the GLOBAL heads (the long ones) fit in the 256 MB last-level cache that
// all XCDs share, every XCD finds them there and plain longest-first order over the whole chip
// balances best; XCD binning pays once those streams overflow it (measured: 31 x 32K sequences,
// ~500 MB of global-head K/V, run 3% faster binned; one 128K sequence, 64 MB, 7% slower).
constexpr int64_t kSharedCacheBytes = 256ll << 20;

void schedule_layer(const SchedInput &t, std::vector<Item> &items) {
  items.clear();
  int64_t global_kv_bytes = 0;
  for (int32_t g = 0; g < t.Hkv; ++g)
    if (t.head_class[g] == RK_GLOBAL)
      for (int32_t b = 0; b < t.num_seqs; ++b) global_kv_bytes += (int64_t)t.kv_len[b] * t.D * 2 * t.elem_bytes;
  if (global_kv_bytes <= kSharedCacheBytes) {
    for (int32_t b = 0; b < t.num_seqs; ++b)
      for (int32_t g = 0; g < t.Hkv; ++g) {
        int cls = t.head_class[g];
        // the head's rows: positions class_start .. kv_len - 1, packed rows from q_begin
        const int32_t qs = (cls == RK_GLOBAL ? t.q_begin[b] : t.q_start[b]), row0 = qs - t.q_begin[b], nq = t.kv_len[b] - qs;
        for (int32_t tok0 = 0; tok0 < nq; tok0 += t.T) {
          int32_t tok1 = std::min(nq, tok0 + t.T);
          TileRange r = tile_range(cls, qs + tok0, qs + tok1 - 1, t.sink, t.window);
          items.push_back({b, g, row0 + tok0, r.count()});
        }
      }
    std::stable_sort(items.begin(), items.end(), [](const Item &a, const Item &b) { return a.tiles > b.tiles; });
    return;
  }
  std::vector<std::vector<Item>> runs;
  int64_t total = 0;
  std::vector<Item> grp;
  for (int32_t b = 0; b < t.num_seqs; ++b) {
    for (int32_t g = 0; g < t.Hkv; ++g) {
      int cls = t.head_class[g];
      const int32_t qs = (cls == RK_GLOBAL ? t.q_begin[b] : t.q_start[b]), row0 = qs - t.q_begin[b], nq = t.kv_len[b] - qs;
      grp.clear();
      for (int32_t tok0 = 0; tok0 < nq; tok0 += t.T) {
        int32_t tok1 = std::min(nq, tok0 + t.T);
        TileRange r = tile_range(cls, qs + tok0, qs + tok1 - 1, t.sink, t.window);
        grp.push_back({b, g, row0 + tok0, r.count()});
        total += r.count();
      }
      if (!grp.empty()) runs.push_back(grp);
    }
  }
  if (runs.empty()) return;
  const int64_t cap = std::max<int64_t>(1, (total + 4 * kXcd - 1) / (4 * kXcd));
  std::vector<std::vector<Item>> chunks;
  std::vector<int64_t> chunk_cost;
  for (const auto &r : runs) {
    int64_t c = 0;
    for (const Item &it : r) c += it.tiles;
    const int64_t k = std::min<int64_t>((c + cap - 1) / cap, (int64_t)r.size());
    for (int64_t part = 0; part < k; ++part) {
      std::vector<Item> cur;
      int64_t cc = 0;
      for (size_t i = part; i < r.size(); i += k) {
        cur.push_back(r[i]);
        cc += r[i].tiles;
      }
      chunks.push_back(cur);
      chunk_cost.push_back(cc);
    }
  }
  std::vector<size_t> order(chunks.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return chunk_cost[a] > chunk_cost[b]; });
  std::vector<std::vector<Item>> bins(kXcd);
  std::vector<int64_t> load(kXcd, 0);
  for (size_t ci : order) {
    int x = 0;
    for (int k = 1; k < kXcd; ++k)
      if (load[k] < load[x]) x = k;
    bins[x].insert(bins[x].end(), chunks[ci].begin(), chunks[ci].end());
    load[x] += chunk_cost[ci];
  }
  size_t rounds = 0;
  for (auto &bin : bins) {
    std::stable_sort(bin.begin(), bin.end(), [](const Item &a, const Item &b) { return a.tiles > b.tiles; });
    rounds = std::max(rounds, bin.size());
  }
  items.reserve(rounds * kXcd);
  for (size_t k = 0; k < rounds; ++k)
    for (int x = 0; x < kXcd; ++x) items.push_back(k < bins[x].size() ? bins[x][k] : Item{-1, 0, 0, 0});
  while (!items.empty() && items.back().seq < 0) items.pop_back();  // trailing pads launch nothing
}

}  // namespace rk
