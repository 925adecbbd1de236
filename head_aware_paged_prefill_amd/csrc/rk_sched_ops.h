// Host schedulers of the library's other kernels: the per-key mass work units and the split-KV
// decode items of one layer.  Pure functions of the call's shape (SchedInput).
#pragma once

#include <stdint.h>

#include <vector>

#include "rk_ops.h"
#include "rk_sched.h"

namespace rk {

// Query steps per work unit of the per-key mass pass for one layer: kMassChunkSteps, halved (down to
// kMassMinChunkSteps) while the class-independent unit bound stays below kMassTargetUnits, so that a
// small call still spreads over the chip instead of running a few long units.  A function of the
// shape only, so the workspace bound and the schedule agree.
int32_t mass_steps_per_chunk(const SchedInput &in, int32_t keys, int32_t tokens);

// Work units of the per-key mass pass: key block kblk (`keys` keys) of (seq, kv head) over query
// chunk qc (`steps` steps of `tokens` tokens on the token grid from the head's class start).
// Only units with a visible pair are listed.  Runs of at most kMassRun units with the same (seq, kv
// head, qc) -- key blocks reading the same query rows -- are placed on one XCD, each run on the XCD
// with the fewest units so far: launch position i runs on XCD i % kXcd; padding has seq = -1.
void mass_schedule(const SchedInput &in, int32_t keys, int32_t tokens, int32_t steps, std::vector<MassUnit> &units);

// An upper bound of mass_schedule's list length that holds for any head classes (head_class unused).
int64_t mass_units_bound(const SchedInput &in, int32_t keys, int32_t tokens, int32_t steps);

// Decode-shaped calls (every sequence has at most one query row, at position kv_len - 1): split-KV
// items over the query's visible key ranges (GLOBAL: [0, L); LOCAL: [0, min(S, L)) and
// [max(0, L - W), L), merged when they touch).  A range is cut at multiples of the key chunk, which
// keeps the layer within kDecodeTargetItems items, two per range reserved for the cuts that do not
// fall on a range boundary (a multiple of 32, at least kDecodeMinChunk keys, or kDecodeMinChunkLarge
// keys in a layer with at least kDecodeLargeKeys visible keys).
// Items come grouped by (seq, kv head) in ascending key order, each group padded with empty items
// (k0 = k1 = 0) to a multiple of kDecodeWaves; comb_off[b * Hkv + g] is the first item of (b, g) and
// comb_off[num_seqs * Hkv] the item count.
void decode_schedule(const SchedInput &in, std::vector<DecItem> &items, std::vector<int32_t> &comb_off);

// An upper bound of decode_schedule's item count for any head classes: kDecodeTargetItems plus four
// cut items and kDecodeWaves - 1 padding items per (seq, kv head).
int64_t decode_items_bound(const SchedInput &in);

}  // namespace rk
