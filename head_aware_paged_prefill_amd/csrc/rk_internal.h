// Internal structures of the attention path shared by the host core (rk_host.cpp), the scheduler
// (rk_sched.cpp) and the attention kernel (rk_attn.hip); the other kernels add rk_ops.h.
// Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define RK_HD __host__ __device__
#else
#define RK_HD
#endif

namespace rk {

// One attention work item covers kRowsPerItem query rows: G heads of one KV head x T tokens,
// T = kRowsPerItem / G.  Key tiles of kKeyTile tokens are staged through LDS.
constexpr int kRowsPerItem = 256;
constexpr int kKeyTile = 64;
constexpr int kThreads = 256;

struct SeqInfo {
  int32_t q_start;        // position of the sequence's first packed row (the GLOBAL heads' start)
  int32_t kv_len;
  int32_t cu_q;           // first packed query row of the sequence
  int32_t n_q;            // kv_len - q_start
  int32_t q_start_local;  // first query position of the LOCAL heads (>= q_start)
  int32_t kv_off;         // first key of the sequence in per-key outputs (sum of earlier kv_len)
};

struct Item {
  int32_t seq;
  int32_t kv_head;
  int32_t tok0;   // first query index within the sequence's queries
  int32_t tiles;  // key tiles the item visits (its cost)
};

// Everything the attention kernel needs to start one item, in one 32-byte record the host fills
// in launch order: reading it is the only memory round trip before the item's page ids and queries
// (the item record, its sequence, its page-table base and its fallback page were four).
struct ItemCtx {
  int32_t kvh_cls;   // KV head | class << 16; -1 for schedule padding
  int32_t tok0;      // first query index within the sequence's packed rows
  int32_t cu_q;      // first packed row of the sequence
  int32_t q_start;   // position of the sequence's first packed row
  int32_t n_q;       // packed rows of the sequence
  int32_t kv_len;
  int32_t page_off;  // offset of the (KV head, seq) logical page table in page_ids
  int32_t fallback;  // physical page of the item's last query (held, fully written)
};

// Visible key tiles of one item: sink tiles [0, ns) then window tiles [wt0, wt1].  For GLOBAL
// heads ns = 0, wt0 = 0.  The host scheduler and the kernel both use this one definition.
struct TileRange {
  int32_t ns, wt0, wt1;
  RK_HD int32_t count() const { return ns + (wt1 - wt0 + 1); }
  RK_HD int32_t tile(int32_t idx) const { return idx < ns ? idx : wt0 + (idx - ns); }
};

RK_HD inline TileRange tile_range(int cls, int32_t i_min, int32_t i_max, int32_t sink,
                                                int32_t window) {
  TileRange r;
  r.wt1 = i_max / kKeyTile;
  if (cls == 1) {
    r.ns = 0;
    r.wt0 = 0;
  } else {
    int32_t wlo = i_min - window + 1;
    if (wlo < 0) wlo = 0;
    r.wt0 = wlo / kKeyTile;
    int32_t sink_tiles = (sink + kKeyTile - 1) / kKeyTile;
    r.ns = sink_tiles < r.wt0 ? sink_tiles : r.wt0;
  }
  return r;
}

struct AttnParams {
  const void *q;
  void *o;
  float *lse;
  const void *k_pages;
  const void *v_pages;
  const int32_t *page_base;  // [Hkv][num_seqs] offset of each (kv head, seq) logical table in page_ids
  const int32_t *page_ids;   // logical page -> physical page, -1 when not held
  const SeqInfo *seqs;
  const Item *items;
  const ItemCtx *ictx;        // per launch slot (bf16 kernel)
  const uint8_t *head_class;  // [Hkv] of this layer
  int32_t n_items;
  int32_t num_seqs;
  int32_t H;
  int32_t Hkv;
  int32_t G;
  int32_t T;
  int32_t P;
  int32_t log2P;
  int32_t sink;
  int32_t window;
  int32_t total_q;
  float scale_log2;  // softmax scale * log2(e)
};

hipError_t launch_attention(const AttnParams &p, int dtype, int head_dim, hipStream_t stream);

}  // namespace rk
