// Internal structures shared by the host core (rk_host.cpp) and the gfx950 kernels (rk_kernels.hip).
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

// Writes token rows into held pages: the append of new tokens (src = k_new/v_new rows) or the
// import of a reused document (src = [Hkv][n_tok][D] with a head stride, keys rotated by delta).
struct KvWriteParams {
  void *k_pages;
  void *v_pages;
  int32_t sink;    // append: a LOCAL head's slots below its window and above the sink are zeroed
  int32_t window;
  const int32_t *page_base;
  const int32_t *page_ids;
  const SeqInfo *seqs;
  const int32_t *app_items;  // append: [n][2] = (seq, logical page)
  const uint8_t *head_class; // append: [Hkv] classes of the layer
  int32_t n_items;
  int32_t num_seqs;
  int32_t Hkv;
  int32_t P;
  int32_t log2P;
  // append source
  const void *k_src;
  const void *v_src;
  // import source
  int64_t src_head_stride;
  int32_t seq;        // import: the sequence
  int32_t tok_begin;  // import: first token of the range
  int32_t n_tok;      // import: tokens in the range
  int32_t page0;      // import: first logical page overlapping the range
  int64_t delta;
  double rope_base;
  int32_t rope_style;
};

// Per-key attention mass of one layer's call (bf16 pools, G <= 16).  A workgroup of 8 waves owns
// mass_keys_per_unit(G) keys; its per-(head, key) LDS accumulators hold kMassAccFloats floats.  A step
// stages kRowsPerItem query rows: mass_tokens_per_step(G) tokens (a multiple of 16, so that every
// 16-row half of a 32-row MFMA block belongs to one head) of each of the G heads, the rest padding.
constexpr int kMassAccFloats = 4096;
constexpr int mass_keys_per_wave(int G) { return G <= 8 ? 64 : 32; }
constexpr int mass_keys_per_unit(int G) { return 8 * mass_keys_per_wave(G); }
constexpr int mass_tokens_per_step(int G) { return kRowsPerItem / G / 16 * 16; }
struct MassUnit {
  int32_t seq;  // < 0: padding
  int32_t kv_head;
  int32_t kblk;  // key block: keys kblk * mass_keys_per_unit(G) ..
  int32_t qc;    // query chunk: steps qc * kMassChunkSteps .. of the head's token grid
};
struct MassParams {
  const void *q;
  const float *lse;     // [H][total_q], natural log
  float *mass;          // [H][total_kv]
  const void *k_pages;
  const int32_t *page_base;
  const int32_t *page_ids;
  const SeqInfo *seqs;
  const uint8_t *head_class;  // [Hkv] of the layer
  int32_t num_seqs;
  int32_t H;
  int32_t Hkv;
  int32_t G;
  int32_t T;  // mass_tokens_per_step(G)
  int32_t P;
  int32_t log2P;
  int32_t sink;
  int32_t window;
  float scale_log2;
  int32_t total_q;
  int32_t total_kv;
  const MassUnit *units;  // launch order
  int32_t n_units;
};
constexpr int kMassRun = 16;         // units placed together on one XCD
constexpr int kMassChunkSteps = 64;  // steps per query chunk

// Decode (one query row per sequence): split-KV work items, one wave each, over key ranges of the
// query's visible set; the partial (o, lse) of item i go to slot i and are merged per (seq, kv head)
// by the combine kernel.
constexpr int kDecodeTargetItems = 4096;  // items per layer the key chunk aims at (two rounds of 8 waves per CU)
constexpr int kDecodeMinChunk = 256;      // keys
struct DecItem {
  int32_t seq;
  int32_t kv_head;
  int32_t k0, k1;  // key range [k0, k1) of the sequence, all visible to its query
};
struct DecodeParams {
  const void *q;       // [total_q][H][D] bf16
  void *o;             // [total_q][H][D] bf16
  float *lse;          // [H][total_q] or null
  const void *k_pages;
  const void *v_pages;
  const int32_t *page_base;
  const int32_t *page_ids;
  const SeqInfo *seqs;
  const DecItem *items;   // slot order: grouped by (seq, kv head), ranges ascending
  const int32_t *comb_off;  // [num_seqs * Hkv + 1]: first slot of (seq, kv head) = b * Hkv + g
  float *part_o;          // [n_items][G][D] fp32, normalised partial outputs
  float *part_lse;        // [n_items][G] fp32, natural log
  int32_t num_seqs;
  int32_t H;
  int32_t Hkv;
  int32_t G;
  int32_t P;
  int32_t log2P;
  float scale_log2;
  int32_t total_q;
  int32_t n_items;
};

// Page hand-off: copies whole K and V pages between the pool and a packed buffer.
struct PageCopyParams {
  void *k_pages;
  void *v_pages;
  const int32_t *ids;  // physical pages in packed order
  int64_t n;           // pages
  void *buf;           // packed: [n][2][page_bytes]
  int64_t page_bytes;  // page_size * head_dim * element size (a multiple of 16)
};

hipError_t launch_attention(const AttnParams &p, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_page_copy(const PageCopyParams &p, bool pack, hipStream_t stream);
hipError_t launch_decode(const DecodeParams &p, int head_dim, hipStream_t stream);
hipError_t launch_key_mass(const MassParams &p, int head_dim, hipStream_t stream);
hipError_t launch_append(const KvWriteParams &p, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_import(const KvWriteParams &p, int n_pages, int dtype, int head_dim, hipStream_t stream);

}  // namespace rk
