// Internal structures of the library's other kernels (KV writes, per-key mass, decode, page
// hand-off), shared by the host core (rk_host.cpp) and those kernels.  Nothing here is part of the
// public ABI.  The attention kernel's structures are in rk_internal.h.
#pragma once

#include "rk_internal.h"
#include "rk_seg.h"

namespace rk {

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
  // import: cos and sin of delta * base^(-2m/D) for pair m < D/2 (computed in fp64 on the host,
  // rounded to fp32)
  float rope_cos[64];
  float rope_sin[64];
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
  int32_t qc;    // query chunk: steps qc * steps_per_chunk .. of the head's token grid
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
  int32_t steps_per_chunk;  // query steps per unit (the layer's mass_steps_per_chunk)
};
constexpr int kMassRun = 16;         // units placed together on one XCD
constexpr int kMassChunkSteps = 64;      // steps per query chunk, at most
constexpr int kMassMinChunkSteps = 4;    // ... and at least
constexpr int kMassTargetUnits = 2048;   // units per layer below which the chunk is halved

// Decode (one query row per sequence): split-KV work items, one wave each, over key ranges of the
// query's visible set.  kDecodeWaves consecutive items belong to one (seq, kv head) (padding items
// have an empty range) and form one workgroup, which merges their partials in LDS into slot
// item / kDecodeWaves; the combine kernel merges the slots of each (seq, kv head).
constexpr int kDecodeWaves = 4;           // items (waves) per workgroup
constexpr int kDecodeTargetItems = 8192;  // items per layer the key chunk aims at (eight waves per SIMD)
constexpr int kDecodeMinChunk = 128;      // keys
constexpr int kDecodeMinChunkLarge = 192;  // keys, for layers with at least kDecodeLargeKeys visible keys
constexpr int64_t kDecodeLargeKeys = 65536;
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
  const DecItem *items;   // grouped by (seq, kv head), ranges ascending, kDecodeWaves per workgroup
  const int32_t *comb_off;  // [num_seqs * Hkv + 1]: first item of (seq, kv head) = b * Hkv + g
  float *part_o;          // [n_items / kDecodeWaves][G][D] fp32, normalised partial outputs
  float *part_lse;        // [n_items / kDecodeWaves][G] fp32, natural log
  // the new token of each sequence with a query row, [total_q][Hkv][D] bf16, or null when the caller
  // appended it already: then the item that ends at kv_len writes it into its page
  const void *k_src;
  const void *v_src;
  const uint8_t *head_class;  // [Hkv] classes of the layer
  int32_t sink;
  int32_t window;
  int32_t num_seqs;
  int32_t H;
  int32_t Hkv;
  int32_t G;
  int32_t P;
  int32_t log2P;
  float scale_log2;
  int32_t total_q;
  int32_t n_items;  // a multiple of kDecodeWaves
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

hipError_t launch_page_copy(const PageCopyParams &p, bool pack, hipStream_t stream);
hipError_t launch_decode(const DecodeParams &p, int head_dim, hipStream_t stream);
// Size of the per-GPU static partials array of the decode variant that allocates nothing, and its
// device address on the current device (looked up on the first call per device, then cached).
constexpr size_t kDecodeScratchBytes = RK_DECODE_SCRATCH_BYTES;
hipError_t decode_scratch(void **ptr);
hipError_t launch_key_mass(const MassParams &p, int head_dim, hipStream_t stream);
hipError_t launch_append(const KvWriteParams &p, int dtype, int head_dim, hipStream_t stream);
hipError_t launch_import(const KvWriteParams &p, int n_pages, int dtype, int head_dim, hipStream_t stream);

}  // namespace rk
