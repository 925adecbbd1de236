/*
 * rk_seg.h -- C ABI of the SegPagedAttention prefill library for AMD MI355X (gfx950).
 *
 * What the library computes.  The KV cache is kept in pages owned by one
 * (layer, KV head, sequence).  Heads are classified once, offline, as GLOBAL or
 * LOCAL; the class map is an input read by table lookup with no online cost
 * (page "RedKnot - Xiaohongshuが開発した…" (aiboss88.com), section RedKnotの使い方,
 * PROFILE item, and section 主な利点, second item).  GLOBAL heads hold and read
 * every context page; LOCAL heads physically hold only the sink pages and the
 * pages of a recent window (page "为什么长上下文推理这么慢？RedKnot如何用1个百分点的
 * 质量代价换来2–5倍TTFT加速" (bjdmk.com.cn), section 二 ③ SegPagedAttention).
 * Attention runs without any attention mask: visibility is derived from token
 * indices inside the kernel (same page, section 二 ③; aiboss88.com, section 技術原則,
 * fourth item).  Reused document keys are rotated from their offline to their
 * actual position before use (page "RedKnot – 小红书研发并开源的长上下文大模型推理引擎"
 * (shshi.cn), section RedKnot技术原理, 2. 位置无关缓存复用).
 *
 * Visibility (token indices; i = absolute query position, j = key position):
 *   GLOBAL: j <= i.       LOCAL: j <= i and (j < sink or j > i - window).
 * The window holds `window` keys including the query; the sink is the first
 * `sink` absolute positions of the sequence.  Query head h reads KV head
 * h / (num_q_heads / num_kv_heads); the class is per (layer, KV head).
 *
 * Memory layout (all device buffers are caller-owned; the library allocates no
 * device memory):
 *   K pages   [num_pages][page_size][head_dim]   (token-major)
 *   V pages   [num_pages][head_dim][page_size]   (channel-major: each page stores V transposed)
 *   q, o      [total_q][num_q_heads][head_dim]   queries packed by sequence, in sequence order
 *   k_new, v_new [total_q][num_kv_heads][head_dim]  keys/values of the query tokens
 *   lse       [num_q_heads][total_q] fp32, natural log
 * where sequence b contributes kv_len[b] - qb[b] rows for absolute positions
 * qb[b] .. kv_len[b]-1, with qb[b] = q_start_global[b] when the batch gives it and
 * q_start[b] otherwise.  Element type: RK_BF16 (bfloat16) or RK_F32.
 *
 * Head-ragged query ranges (EXECUTE's split: global heads recompute attention and
 * write the online KV cache, local heads reuse theirs; page "RedKnot -
 * Xiaohongshuが開発した…", section 使い方, EXECUTE item): a GLOBAL head computes
 * the rows and writes the keys/values of positions q_start_global[b] ..
 * kv_len[b]-1, a LOCAL head those of q_start[b] .. kv_len[b]-1.  Rows of a
 * LOCAL head below q_start[b] are not written (o and lse keep their contents).
 * Without q_start_global both classes start at q_start[b].
 * Every device pointer must be 16-byte aligned; head_dim is 64 or 128; page_size
 * is a power of two in [8, 256].
 *
 * Cache contents contract: before attention, every slot of a held page whose
 * token is below kv_len must have been written -- by the append inside
 * rk_seg_attn_prefill (tokens from the head's class start on) or by
 * rk_seg_reuse_rerotate (tokens below it).  Slots at or beyond kv_len and pages a head does not hold may
 * contain any bits (NaN included) before the call; the append clears the slots
 * of a sequence's last page past kv_len, and pages a head does not hold are
 * never read.  None of them reaches the output.
 *
 * Errors: every call returns an rk_status; no exception crosses the ABI.  On
 * failure, rk_last_error() returns a thread-local message.  A failed call
 * leaves the pool and tables unchanged.
 *
 * Threads and streams: a pool and its tables are not thread-safe; callers
 * serialise calls on one pool.  Device work is enqueued on the given HIP stream
 * (void * holding a hipStream_t; NULL = the null stream) and is asynchronous;
 * host-side state (free list, tables) changes synchronously.  Pages returned to
 * the free list may be handed out again at once: device work that uses them must
 * be ordered after earlier work on them (same stream, or caller synchronisation).
 */
#ifndef RK_SEG_H
#define RK_SEG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t rk_status;
#define RK_OK 0
#define RK_ERR_INVALID_ARG (-1)
#define RK_ERR_OUT_OF_PAGES (-2)
#define RK_ERR_WORKSPACE_TOO_SMALL (-3)
#define RK_ERR_UNSUPPORTED (-4)
#define RK_ERR_HIP (-5)
#define RK_ERR_STATE (-6)
#define RK_ERR_INTERNAL (-7)

#define RK_LOCAL 0
#define RK_GLOBAL 1

#define RK_BF16 0
#define RK_F32 1

#define RK_ROPE_ROTATE_HALF 0 /* pairs (m, m + D/2) */
#define RK_ROPE_INTERLEAVED 1 /* pairs (2m, 2m + 1) */

typedef struct rk_pool rk_pool;
typedef struct rk_tables rk_tables;

/* Pool description.  k_pages / v_pages: device, caller-owned, layout above, 16-byte aligned.
 * initial_free_order: host, optional (NULL = ascending ids); a permutation of [0, num_pages)
 * giving the free list from its head.  The array is copied. */
typedef struct {
  int32_t num_layers;
  int32_t num_kv_heads;
  int32_t head_dim;  /* 64 or 128 */
  int32_t page_size; /* power of two, 8..256 */
  int32_t dtype;     /* RK_BF16 or RK_F32 */
  int32_t reserved0;
  int64_t num_pages; /* >= 0, < 2^31 */
  void *k_pages;
  void *v_pages;
  const int32_t *initial_free_order;
} rk_pool_desc;

/* One prefill call over layers [layer_begin, layer_end) of a batch of sequences.
 * q_start, kv_len: host [num_seqs], 0 <= q_start[b] <= kv_len[b] < 2^31.
 * q_start_global: host [num_seqs] or NULL; 0 <= q_start_global[b] <= q_start[b]: the first query
 *   position of the GLOBAL heads (head-ragged query ranges, above).  NULL: q_start.
 *   A LOCAL head holds and reads its window relative to q_start either way.
 * head_class: host [num_layers * num_kv_heads], row-major by layer, values RK_LOCAL / RK_GLOBAL.
 * sink >= 0, window >= 1.  num_q_heads must be a positive multiple of the pool's num_kv_heads.
 * All host arrays are copied. */
typedef struct {
  int32_t layer_begin;
  int32_t layer_end;
  int32_t num_seqs;
  int32_t num_q_heads;
  const int32_t *q_start;
  const int32_t *kv_len;
  const uint8_t *head_class;
  int32_t sink;
  int32_t window;
  const int32_t *q_start_global;
} rk_batch_desc;

/* Counters of one built call (host, exact integers). */
typedef struct {
  int64_t pages_held;        /* pages the call holds over all its layers */
  int64_t total_q;           /* packed query rows per layer */
  int64_t visible_pairs;     /* sum over layers, q heads and queries of |visible keys| */
  int64_t visible_pairs_global; /* the part from GLOBAL heads */
  int64_t work_items;        /* attention work items over all layers */
  int64_t key_tiles;         /* key tiles the items visit over all layers */
  int64_t workspace_bytes;   /* device workspace the build uses */
} rk_tables_stats;

/* Byte ledger of the state a tables object holds (rk_seg_pack_ledger): what a hand-off of its pages
 * moves, against the dense per-head layout that keeps every token of every KV head.  Host, exact
 * integers; bytes count K and V. */
typedef struct {
  int64_t pages;          /* held pages */
  int64_t pages_global;   /* of GLOBAL heads */
  int64_t pages_local;    /* of LOCAL heads */
  int64_t packed_bytes;   /* pages * 2 * page_size * head_dim * element size: what rk_seg_pack_pages moves */
  int64_t tokens;         /* tokens the held-token rule keeps (the retained rule after trim), summed
                             over (layer, KV head) */
  int64_t token_bytes;    /* tokens * 2 * head_dim * element size: the token-granular lower bound */
  int64_t dense_tokens;   /* kv_len summed over (layer, KV head): every token of every head */
  int64_t dense_bytes;    /* dense_tokens * 2 * head_dim * element size */
} rk_pack_ledger;

/* -- pool ---------------------------------------------------------------------------------- */

/* Create a pool over caller-owned page storage: the KV pools that BUILDSTATE prepares and
 * SELECTVISIBLESTATE draws a request's pages from (page "RedKnot - Xiaohongshuが開発したオープン
 * ソースの長文テキスト推論高速化エンジン" (aiboss88.com), section RedKnotの使い方, BUILDSTATE item;
 * the pages' separate global and local pools are one physical pool here, a page's owner fixing its
 * class).  Host only: no device work.  desc: every field is read at creation and copied; the page
 * storage stays the caller's and must outlive the pool.
 * Storage assumption: page p of the K array starts at k_pages + p*page_size*head_dim elements,
 * of the V array at v_pages + p*head_dim*page_size elements.  initial_free_order (optional) is a
 * permutation of [0, num_pages): the free list, head first.
 * Errors: RK_ERR_INVALID_ARG (null desc or out, num_layers or num_kv_heads < 1, num_pages outside
 * [0, 2^31), null page arrays with num_pages > 0, page arrays not 16-byte aligned, initial_free_order
 * not a permutation); RK_ERR_UNSUPPORTED (head_dim not 64 / 128, page_size not a power of two in
 * [8, 256], unknown dtype).  *out is untouched on error. */
rk_status rk_seg_pool_create(const rk_pool_desc *desc, rk_pool **out);

/* Destroy a pool.  Fails with RK_ERR_STATE while tables built from it are alive. */
rk_status rk_seg_pool_destroy(rk_pool *pool);

/* Free and used page counts (free + used == num_pages). */
rk_status rk_seg_pool_query(const rk_pool *pool, int64_t *free_pages, int64_t *used_pages);

/* Copy up to cap ids of the free list, head first, into out; *n = its full length. */
rk_status rk_seg_pool_free_list(const rk_pool *pool, int32_t *out, int64_t cap, int64_t *n);

/* -- tables: SELECTVISIBLESTATE (page "RedKnot - Xiaohongshuが開発した…", section 使い方) ---------- */

/* Device workspace bytes rk_seg_build_tables needs for this batch. */
rk_status rk_seg_tables_workspace_bytes(const rk_pool *pool, const rk_batch_desc *batch, size_t *bytes);

/* Resolve head classes, compute every (layer, KV head, seq)'s held token ranges, expand them to
 * pages, allocate the pages (all or nothing), build the dense logical->physical page tables and the
 * balanced work schedule, and upload them into d_workspace on `stream`.
 *   Held tokens: GLOBAL [0, kv_len); LOCAL [0, min(sink, kv_len)) and [max(0, q_start - window + 1),
 *   kv_len), expanded to whole pages; runs that overlap or touch merge into one segment.
 *   Allocation: pages are taken from the free list's head in ascending (layer, KV head, seq,
 *   logical page) order.
 * d_workspace: device, >= rk_seg_tables_workspace_bytes, 256-byte aligned, owned by the caller and
 *   read by later device calls on these tables; it must outlive them.  NULL (with ws_bytes 0) builds
 *   the tables on the host only: export, stats, trim and destroy work, device calls fail.
 * Errors: RK_ERR_INVALID_ARG, RK_ERR_OUT_OF_PAGES (pool unchanged), RK_ERR_WORKSPACE_TOO_SMALL,
 *   RK_ERR_HIP.  The host staging of the upload stays alive until the tables are destroyed. */
rk_status rk_seg_build_tables(rk_pool *pool, const rk_batch_desc *batch, void *d_workspace,
                              size_t ws_bytes, void *stream, rk_tables **out);

/* The next call on the same sequences and layers (decode: one token each; or a further chunk):
 * sequence b gains n_new[b] >= 0 tokens, which become its query rows (q_start = q_start_global =
 * the old kv_len; kv_len += n_new[b]).  The pool's pages keep the state the previous call left:
 * every (layer, KV head, seq) keeps the physical page, and its contents, of each logical page it
 * still holds under the held-token rule of rk_seg_build_tables for the new q_start / kv_len; pages
 * it no longer holds (a LOCAL head's window moving on) go back to the free list first, in ascending
 * (layer, KV head, seq, logical page) order, then the new pages are taken from the head of the free
 * list in the same order.  Works on trimmed and untrimmed tables; the result is untrimmed.  (Page
 * "RedKnot – 小红书研发并开源的长上下文大模型推理引擎" (shshi.cn), section RedKnot核心特点: more
 * concurrent long-context sessions per GPU, i.e. serving over the retained segmented state.)
 * d_workspace: as for rk_seg_build_tables, >= rk_seg_tables_advance_workspace_bytes; it may be the
 *   workspace the tables used before (the previous upload is waited for first).  NULL: host only.
 * n_new: host [num_seqs].
 * Errors: RK_ERR_INVALID_ARG, RK_ERR_OUT_OF_PAGES and RK_ERR_WORKSPACE_TOO_SMALL leave the tables
 *   and the pool unchanged; RK_ERR_HIP on the upload leaves the new page state without a device
 *   view (device calls then fail with RK_ERR_STATE). */
rk_status rk_seg_tables_advance_workspace_bytes(const rk_pool *pool, const rk_tables *tables,
                                                const int32_t *n_new, size_t *bytes);
rk_status rk_seg_tables_advance(rk_pool *pool, rk_tables *tables, const int32_t *n_new,
                                void *d_workspace, size_t ws_bytes, void *stream);

/* Export the held segments and physical page ids of one (layer, KV head, seq), host side.
 * seg_tok_begin / seg_npages: [seg_cap]; page_ids: [page_cap], in logical page order.
 * *n_segs and *n_pages receive the full counts even when larger than the capacities. */
rk_status rk_seg_tables_export(const rk_tables *tables, int32_t layer, int32_t kv_head, int32_t seq,
                               int32_t *seg_tok_begin, int32_t *seg_npages, int32_t seg_cap,
                               int32_t *n_segs, int32_t *page_ids, int32_t page_cap, int32_t *n_pages);

/* Export the attention work schedule of one layer in launch order: items [cap][4] =
 * (seq, kv_head, first query index within the sequence, number of key tiles visited).  Workgroup i
 * of the launch runs on XCD i % 8; entries with seq = -1 are empty slots that keep the next items
 * on their XCD.  Every (seq, kv_head, q tile) appears exactly once. */
rk_status rk_seg_tables_schedule(const rk_tables *tables, int32_t layer, int32_t *items, int64_t cap,
                                 int64_t *n_items, int32_t *tokens_per_item, int32_t *key_tile);

/* Export the per-key mass work units of one layer (rk_seg_key_mass) in launch order: units [cap][4] =
 * (seq, kv_head, key block, query chunk).  Key block k holds keys [k * keys_per_unit, ...) of the
 * sequence; query chunk c holds the query tokens start + [c * steps_per_chunk * tokens_per_step,
 * (c + 1) * steps_per_chunk * tokens_per_step) of the head, where start is the head's first query
 * position.  Exactly the (seq, kv_head, key block, query chunk) with at least one visible (query,
 * key) pair appear, each once.  Workgroup i runs on XCD i % 8; entries with seq = -1 are empty
 * slots.  The list is empty when the group size num_q_heads / num_kv_heads exceeds 16 (the mass
 * pass does not support it).  Any output pointer may be NULL. */
rk_status rk_seg_tables_mass_schedule(const rk_tables *tables, int32_t layer, int32_t *units, int64_t cap,
                                      int64_t *n_units, int32_t *keys_per_unit, int32_t *tokens_per_step,
                                      int32_t *steps_per_chunk);

/* Export the split-KV decode items of one layer (rk_seg_attn_decode), in launch order: items
 * [cap][4] = (seq, kv_head, k0, k1): the keys [k0, k1) of the sequence, all visible to its query
 * (the token at kv_len - 1).  A (seq, kv head)'s visible keys are GLOBAL [0, kv_len) or LOCAL
 * [0, min(sink, kv_len)) and [max(0, kv_len - window), kv_len) (merged when they touch), cut at
 * multiples of one key chunk (a multiple of 32, at least 128).  Items come grouped by (seq, kv head),
 * ascending, each group padded with empty items (k0 = k1 = 0) to a multiple of 4: four consecutive
 * items run as one workgroup, which merges their partials.  comb_off [comb_cap] receives the first
 * item of (seq b, kv head g) at b * num_kv_heads + g and the item count at num_seqs * num_kv_heads.
 * *n_items = 0 when the tables are not decode-shaped (a sequence with more than one query row, or
 * more than 16 q heads per KV head).  Any output pointer may be NULL. */
rk_status rk_seg_tables_decode_schedule(const rk_tables *tables, int32_t layer, int32_t *items, int64_t cap,
                                        int64_t *n_items, int32_t *comb_off, int64_t comb_cap);

rk_status rk_seg_tables_stats(const rk_tables *tables, rk_tables_stats *out);

/* After the call: LOCAL heads keep their sink pages and the pages covering
 * [max(0, kv_len - window + 1), kv_len); every other LOCAL page returns to the free list (pushed on
 * its head in ascending (layer, KV head, seq, logical page) order).  GLOBAL heads keep all pages.
 * Afterwards the tables describe the retained state; device calls on them fail with RK_ERR_STATE. */
rk_status rk_seg_tables_trim(rk_pool *pool, rk_tables *tables);

/* Return every page the tables still hold to the free list (same order rule) and free the tables.
 * Waits for the upload of the tables' host staging to finish. */
rk_status rk_seg_tables_destroy(rk_pool *pool, rk_tables *tables);

/* -- device calls -------------------------------------------------------------------------- */

/* Position-independent reuse (page "RedKnot – 小红书研发并开源的长上下文大模型推理引擎", section
 * RedKnot技术原理, 2. 位置无关缓存复用): import tokens [tok_begin, tok_begin + n_tok) of sequence `seq`
 * into the held pages of every KV head of `layer`, rotating each key by delta = actual - offline
 * position: pair m turns by delta * base^(-2m/D) (angle, cos and sin in fp64, rotation in fp32, one
 * round-to-nearest-even store).  V is copied unchanged.  Tokens a head does not hold are skipped.
 * Tokens at or after a head's class start (q_start_global for GLOBAL heads, q_start for LOCAL heads)
 * are the call's own and are skipped too: the append inside rk_seg_attn_prefill writes them.
 * src_k, src_v: device [num_kv_heads][n_tok][head_dim] with head stride src_head_stride elements
 * (>= n_tok*head_dim, a multiple of 16 bytes); read only.  Requires tok_begin + n_tok <= kv_len[seq].
 * Errors: RK_ERR_INVALID_ARG, RK_ERR_STATE (host-only or trimmed tables), RK_ERR_HIP. */
rk_status rk_seg_reuse_rerotate(rk_pool *pool, const rk_tables *tables, int32_t layer, int32_t seq,
                                int32_t tok_begin, int32_t n_tok, const void *src_k, const void *src_v,
                                int64_t src_head_stride, int64_t delta, double rope_base,
                                int32_t rope_style, void *stream);

/* Write the query tokens' keys and values (k_new, v_new: [total_q][num_kv_heads][head_dim]) into
 * their held pages of `layer` (the online KV cache write of EXECUTE, page "RedKnot -
 * Xiaohongshuが開発した…", section 使い方), and set the slots past kv_len of each sequence's last
 * page to zero.  Attention on these tables requires this call (or the append inside
 * rk_seg_attn_prefill) to have run. */
rk_status rk_seg_append_kv(rk_pool *pool, const rk_tables *tables, int32_t layer, const void *k_new,
                           const void *v_new, void *stream);

/* EXECUTE's attention for one layer: append k_new / v_new (skipped when both are NULL, e.g. after
 * rk_seg_append_kv), then mask-free head-ragged paged prefill attention.
 * For every q head h and query token: o = sum over visible keys j of softmax_j(scale * q.k_j) v_j,
 * lse = log sum exp(scale * q.k_j) over the same keys (fp32, natural log).
 * q, o: [total_q][num_q_heads][head_dim]; lse: [num_q_heads][total_q] or NULL.
 * softmax_scale <= 0 selects 1/sqrt(head_dim).  Accumulation and softmax are fp32; bf16 products
 * run on the matrix cores; o is rounded once to the storage dtype.
 * Errors: RK_ERR_INVALID_ARG, RK_ERR_STATE, RK_ERR_HIP. */
rk_status rk_seg_attn_prefill(rk_pool *pool, const rk_tables *tables, int32_t layer, const void *q,
                              const void *k_new, const void *v_new, void *o, float *lse,
                              float softmax_scale, void *stream);

/* Per-key attention mass of one layer's call: the routing signal of the sparse FFN, whose dense
 * FFN runs only on the top-k tokens by attention score (page "小红书把 KV Cache 按「头」拆了…",
 * section 事件内容, item 2; page "RedKnot – 小红书研发并开源的长上下文大模型推理引擎", section
 * RedKnot技术原理, 3).  For every q head h and key j < kv_len[b] of sequence b:
 *   mass[h][kv_off(b) + j] = sum over the call's queries i of head h (from its class start) of
 *                            exp(scale * q_i.k_j - lse[h][i]) over the visible pairs (i, j),
 * with kv_off(b) = kv_len[0] + ... + kv_len[b-1]; keys no query sees get 0.  Every such entry is
 * written.  q: as given to rk_seg_attn_prefill; lse: [num_q_heads][total_q] fp32, the lse that
 * rk_seg_attn_prefill returned for that q (natural log); mass: device fp32
 * [num_q_heads][sum kv_len], 4-byte aligned.  softmax_scale as for rk_seg_attn_prefill.  The K
 * pages must hold what attention read (run it after rk_seg_attn_prefill, before the tables are
 * trimmed or destroyed).  Requires a bf16 pool and num_q_heads / num_kv_heads <= 16.
 * Errors: RK_ERR_INVALID_ARG, RK_ERR_STATE, RK_ERR_UNSUPPORTED (fp32 pool, more than 16 q heads per
 * KV head, more than 2^31 keys), RK_ERR_HIP. */
rk_status rk_seg_key_mass(rk_pool *pool, const rk_tables *tables, int32_t layer, const void *q,
                          const float *lse, float *mass, float softmax_scale, void *stream);

/* Decode for one layer of decode-shaped tables (every sequence has at most one query row, at
 * position kv_len - 1, e.g. after rk_seg_tables_advance with n_new = 1): append k_new / v_new
 * (leaving the pages as rk_seg_append_kv would; skipped when both are NULL), split-KV attention over
 * the items of rk_seg_tables_decode_schedule, each giving a partial (o_s, lse_s) over its key range,
 * then the combine o = sum_s e^{lse_s - lse} o_s, lse = log sum_s e^{lse_s} into o / lse.  The result
 * is the masked softmax attention of rk_seg_attn_prefill for those rows.  Two kernel launches: the
 * append happens inside the attention kernel, by the item whose range ends at kv_len.
 * k_new, v_new: device [total_q][num_kv_heads][head_dim] bf16, 16-byte aligned, both or neither.
 * q, o: device [total_q][num_q_heads][head_dim] bf16 (total_q = the sequences with a query row);
 * lse: device [num_q_heads][total_q] fp32 or NULL; softmax_scale <= 0 selects 1/sqrt(head_dim).
 * The partials live in the tables' workspace, so decode calls on one tables object are ordered on
 * one stream.
 * Errors: RK_ERR_UNSUPPORTED for fp32 pools or more than 16 q heads per KV head; RK_ERR_STATE for
 *   tables that are not decode-shaped, trimmed or host-only; RK_ERR_INVALID_ARG; RK_ERR_HIP. */
rk_status rk_seg_attn_decode(rk_pool *pool, const rk_tables *tables, int32_t layer, const void *q,
                             const void *k_new, const void *v_new, void *o, float *lse,
                             float softmax_scale, void *stream);

/* rk_seg_attn_decode for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments, kernels and result; the
 * split-KV partials go to a static array of RK_DECODE_SCRATCH_BYTES per GPU (a device global of the
 * library, held until the process ends) instead of the tables' workspace, and the call allocates
 * nothing (device or host).  Its address is looked up once per device, on the first call with that
 * device current.  Every call on one GPU shares that array and leaves its contents behind; each
 * call writes every partial it reads, so nothing has to start at zero.  Calls that overlap in time
 * on one GPU (other streams, other threads) race on the array: order them.
 * The partials take align256(slots * G * head_dim * 4) + slots * G * 4 bytes, slots = the layer's
 * decode items / 4 (rk_seg_tables_decode_schedule), G = num_q_heads / num_kv_heads.
 * Errors: those of rk_seg_attn_decode; RK_ERR_UNSUPPORTED when the partials exceed
 *   RK_DECODE_SCRATCH_BYTES (checked before anything runs). */
#define RK_DECODE_SCRATCH_BYTES (32u << 20)
rk_status rk_seg_attn_decode_noalloc(rk_pool *pool, const rk_tables *tables, int32_t layer, const void *q,
                                     const void *k_new, const void *v_new, void *o, float *lse,
                                     float softmax_scale, void *stream);

/* -- page hand-off (page "小红书把 KV Cache 按「头」拆了…" (zhichai.net), section 事件内容, and page
 *    "RedKnot – 小红书研发并开源的长上下文大模型推理引擎" (shshi.cn), section RedKnot核心特点: the
 *    prefill/decode KV transfer shrinks because only the pages a head keeps are sent) ------------ */

/* Byte ledger of sequence seq (-1: every sequence) of the tables' current state, host only: works on
 * host-only and trimmed tables.  Errors: RK_ERR_INVALID_ARG. */
rk_status rk_seg_pack_ledger(const rk_tables *tables, int32_t seq, rk_pack_ledger *out);

/* Copy the held pages of sequence seq (-1: every sequence, in order) into dst: for each sequence,
 * layer, KV head and held logical page in ascending order, the page's K [page_size][head_dim] then
 * its V [head_dim][page_size] (the pool's own page layout, so that a receiving pool adopts a page
 * with one copy), page_size * head_dim elements each.  dst: device, >= the ledger's packed_bytes,
 * 16-byte aligned, caller-owned.  The tables need a device view: after rk_seg_tables_trim, call
 * rk_seg_tables_advance with n_new = 0 to get one of the retained state.
 * Errors: RK_ERR_INVALID_ARG (dst_bytes too small, bad seq), RK_ERR_STATE (no device view), RK_ERR_HIP. */
rk_status rk_seg_pack_pages(rk_pool *pool, const rk_tables *tables, int32_t seq, void *dst, size_t dst_bytes,
                            void *stream);

/* The inverse on the receiving side: write the packed pages of src into the held pages of sequence seq
 * (-1: every sequence) of these tables, in the same order.  The tables must describe the same state
 * as the sender's (same lengths, classes, sink, window, page size, head dim, layers) -- e.g. built
 * with q_start = kv_len, whose held pages are the retained state -- so that src_bytes equals their
 * ledger's packed_bytes (else RK_ERR_INVALID_ARG).  Other errors as rk_seg_pack_pages. */
rk_status rk_seg_unpack_pages(rk_pool *pool, const rk_tables *tables, int32_t seq, const void *src,
                              size_t src_bytes, void *stream);

/* -- diagnostics --------------------------------------------------------------------------- */

const char *rk_status_string(rk_status s);
const char *rk_last_error(void);
/* Version string of the library build. */
const char *rk_seg_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RK_SEG_H */
