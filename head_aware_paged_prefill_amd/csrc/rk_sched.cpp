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

int64_t mass_units_bound(const SchedInput &t, int32_t keys, int32_t tokens) {
  // any class: key blocks x query chunks from the earliest start (q_begin <= q_start), plus the
  // padding of the XCD bins (they differ by at most kMassRun units)
  int64_t n = 0;
  for (int32_t b = 0; b < t.num_seqs; ++b) {
    const int64_t L = t.kv_len[b], q = L - t.q_begin[b];
    if (q <= 0) continue;
    const int64_t steps = (q + tokens - 1) / tokens;
    n += (int64_t)t.Hkv * ((L + keys - 1) / keys) * ((steps + kMassChunkSteps - 1) / kMassChunkSteps);
  }
  return n + (int64_t)kXcd * kMassRun;
}

void mass_schedule(const SchedInput &t, int32_t keys, int32_t tokens, std::vector<MassUnit> &units) {
  units.clear();
  const int64_t S = kMassChunkSteps;
  // runs of key blocks sharing (seq, kv head, query chunk), at most kMassRun long
  std::vector<std::vector<MassUnit>> runs;
  std::vector<std::vector<int32_t>> by_chunk;  // query chunk -> key blocks that need it
  for (int32_t b = 0; b < t.num_seqs; ++b)
    for (int32_t g = 0; g < t.Hkv; ++g) {
      const int cls = t.head_class[g];
      const int32_t L = t.kv_len[b];
      const int32_t start = cls == RK_GLOBAL ? t.q_begin[b] : t.q_start[b];
      if (L <= start) continue;  // no query: every mass stays zero
      by_chunk.assign((size_t)(((int64_t)L - start + tokens - 1) / tokens / S + 1), {});
      for (int32_t kb = 0; (int64_t)kb * keys < L; ++kb) {
        // query tokens that see a key of the block: from max(j0, start); a LOCAL block past the
        // sink only up to the window after its last key
        const int64_t j0 = (int64_t)kb * keys;
        const int64_t t_first = std::max<int64_t>(j0, start);
        int64_t t_last = L - 1;
        if (cls == RK_LOCAL && j0 >= t.sink) t_last = std::min<int64_t>(t_last, j0 + keys - 1 + t.window - 1);
        if (t_first > t_last) continue;
        const int64_t k0 = (t_first - start) / tokens, k1 = (t_last - start) / tokens;
        for (int64_t qc = k0 / S; qc <= k1 / S; ++qc) by_chunk[qc].push_back(kb);
      }
      for (size_t qc = 0; qc < by_chunk.size(); ++qc)
        for (size_t i = 0; i < by_chunk[qc].size(); i += kMassRun) {
          std::vector<MassUnit> run;
          for (size_t k = i; k < std::min(by_chunk[qc].size(), i + (size_t)kMassRun); ++k)
            run.push_back({b, g, by_chunk[qc][k], (int32_t)qc});
          runs.push_back(run);
        }
    }
  // each run goes to the XCD bin with the fewest units so far, so that bins differ by at most
  // kMassRun units; launch position i takes the next unit of bin i % kXcd
  std::vector<std::vector<MassUnit>> bins(kXcd);
  for (const auto &run : runs) {
    int x = 0;
    for (int y = 1; y < kXcd; ++y)
      if (bins[y].size() < bins[x].size()) x = y;
    bins[x].insert(bins[x].end(), run.begin(), run.end());
  }
  size_t rounds = 0;
  for (const auto &bin : bins) rounds = std::max(rounds, bin.size());
  units.reserve(rounds * kXcd);
  for (size_t k = 0; k < rounds; ++k)
    for (int x = 0; x < kXcd; ++x) units.push_back(k < bins[x].size() ? bins[x][k] : MassUnit{-1, 0, 0, 0});
  while (!units.empty() && units.back().seq < 0) units.pop_back();
}

namespace {
// visible key ranges of the query at position L - 1 of one (kv head, seq); returns their number
int decode_ranges(int cls, int32_t L, int32_t S, int32_t W, int32_t r[4]) {
  if (L <= 0) return 0;
  if (cls == RK_GLOBAL) {
    r[0] = 0, r[1] = L;
    return 1;
  }
  const int32_t s1 = std::min(S, L), w0 = std::max(0, L - W);
  if (s1 >= w0) {
    r[0] = 0, r[1] = L;
    return 1;
  }
  int n = 0;
  if (s1 > 0) r[2 * n] = 0, r[2 * n + 1] = s1, ++n;
  r[2 * n] = w0, r[2 * n + 1] = L, ++n;
  return n;
}
}  // namespace

// A range of n keys cut at multiples of the chunk gives at most n / chunk + 2 items, and keys / chunk
// <= kDecodeTargetItems; a (seq, kv head) has at most two ranges.
int64_t decode_items_bound(const SchedInput &t) { return kDecodeTargetItems + 4 * (int64_t)t.num_seqs * t.Hkv; }

void decode_schedule(const SchedInput &t, std::vector<DecItem> &items, std::vector<int32_t> &comb_off) {
  items.clear();
  comb_off.assign((size_t)t.num_seqs * t.Hkv + 1, 0);
  int64_t keys = 0, ranges = 0;
  int32_t r[4];
  for (int32_t b = 0; b < t.num_seqs; ++b) {
    if (t.kv_len[b] - t.q_begin[b] != 1) continue;  // no query row
    for (int32_t g = 0; g < t.Hkv; ++g) {
      const int n = decode_ranges(t.head_class[g], t.kv_len[b], t.sink, t.window, r);
      ranges += n;
      for (int i = 0; i < n; ++i) keys += r[2 * i + 1] - r[2 * i];
    }
  }
  // a range gives at most len / chunk + 2 items: leave room for them, so that the items fit one
  // round of resident waves where they can
  const int64_t room = std::max<int64_t>(kDecodeTargetItems / 4, kDecodeTargetItems - 2 * ranges);
  int64_t chunk = (keys + room - 1) / room;
  chunk = std::max<int64_t>(kDecodeMinChunk, (chunk + 31) / 32 * 32);
  for (int32_t b = 0; b < t.num_seqs; ++b)
    for (int32_t g = 0; g < t.Hkv; ++g) {
      comb_off[(size_t)b * t.Hkv + g] = (int32_t)items.size();
      if (t.kv_len[b] - t.q_begin[b] != 1) continue;
      const int n = decode_ranges(t.head_class[g], t.kv_len[b], t.sink, t.window, r);
      for (int i = 0; i < n; ++i)
        for (int64_t c = r[2 * i] / chunk; c * chunk < r[2 * i + 1]; ++c)
          items.push_back({b, g, (int32_t)std::max<int64_t>(r[2 * i], c * chunk),
                           (int32_t)std::min<int64_t>(r[2 * i + 1], (c + 1) * chunk)});
    }
  comb_off[(size_t)t.num_seqs * t.Hkv] = (int32_t)items.size();
}

}  // namespace rk
