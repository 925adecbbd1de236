// Host schedulers of the per-key mass pass and of split-KV decode (see rk_sched_ops.h).
#include "rk_sched_ops.h"

#include <algorithm>

#include "rk_seg.h"

namespace rk {

int64_t mass_units_bound(const SchedInput &t, int32_t keys, int32_t tokens, int32_t S) {
  // any class: key blocks x query chunks from the earliest start (q_begin <= q_start), plus the
  // padding of the XCD bins (they differ by at most kMassRun units)
  int64_t n = 0;
  for (int32_t b = 0; b < t.num_seqs; ++b) {
    const int64_t L = t.kv_len[b], q = L - t.q_begin[b];
    if (q <= 0) continue;
    const int64_t steps = (q + tokens - 1) / tokens;
    n += (int64_t)t.Hkv * ((L + keys - 1) / keys) * ((steps + S - 1) / S);
  }
  return n + (int64_t)kXcd * kMassRun;
}

int32_t mass_steps_per_chunk(const SchedInput &t, int32_t keys, int32_t tokens) {
  int32_t S = kMassChunkSteps;
  while (S > kMassMinChunkSteps && mass_units_bound(t, keys, tokens, S) < kMassTargetUnits) S /= 2;
  return S;
}

void mass_schedule(const SchedInput &t, int32_t keys, int32_t tokens, int32_t steps, std::vector<MassUnit> &units) {
  units.clear();
  const int64_t S = steps;
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
// <= kDecodeTargetItems; a (seq, kv head) has at most two ranges and kDecodeWaves - 1 padding items.
int64_t decode_items_bound(const SchedInput &t) {
  return kDecodeTargetItems + (4 + kDecodeWaves - 1) * (int64_t)t.num_seqs * t.Hkv;
}

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
  // a small layer is latency-bound and gains from more, shorter items; a large one needs longer key
  // runs per wave to keep its loads in flight
  const int64_t min_chunk = keys >= kDecodeLargeKeys ? kDecodeMinChunkLarge : kDecodeMinChunk;
  chunk = std::max<int64_t>(min_chunk, (chunk + 31) / 32 * 32);
  for (int32_t b = 0; b < t.num_seqs; ++b)
    for (int32_t g = 0; g < t.Hkv; ++g) {
      comb_off[(size_t)b * t.Hkv + g] = (int32_t)items.size();
      if (t.kv_len[b] - t.q_begin[b] != 1) continue;
      const int n = decode_ranges(t.head_class[g], t.kv_len[b], t.sink, t.window, r);
      for (int i = 0; i < n; ++i)
        for (int64_t c = r[2 * i] / chunk; c * chunk < r[2 * i + 1]; ++c)
          items.push_back({b, g, (int32_t)std::max<int64_t>(r[2 * i], c * chunk),
                           (int32_t)std::min<int64_t>(r[2 * i + 1], (c + 1) * chunk)});
      while (items.size() % kDecodeWaves) items.push_back({b, g, 0, 0});  // workgroup of one (seq, kv head)
    }
  comb_off[(size_t)t.num_seqs * t.Hkv] = (int32_t)items.size();
}

}  // namespace rk
