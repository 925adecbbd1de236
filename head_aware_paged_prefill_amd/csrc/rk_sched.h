// The varlen work scheduler: one layer's attention work items and their launch order (host side).
#pragma once

#include <stdint.h>

#include <vector>

#include "rk_internal.h"

namespace rk {

constexpr int kXcd = 8;  // XCDs of an MI355X; workgroup i of a launch runs on XCD i % kXcd

// One layer of one call.  Arrays are host [num_seqs]; head_class is the layer's [Hkv] row.
struct SchedInput {
  int32_t num_seqs, Hkv, T, D, elem_bytes, sink, window;
  const uint8_t *head_class;
  const int32_t *kv_len;
  const int32_t *q_start;  // first query position of the LOCAL heads
  const int32_t *q_begin;  // first query position of the GLOBAL heads (a sequence's first packed row)
};

// Items (seq, kv head, first packed row, key tiles) in launch order; schedule padding has seq = -1.
void schedule_layer(const SchedInput &in, std::vector<Item> &items);

}  // namespace rk
