// Host core of the SegPagedAttention prefill library: validation, page pool, per-(layer, KV head,
// seq) page tables, the varlen work schedule, the table upload and the C ABI glue.
//
// Sources (web pages about RedKnot, cited by title and section):
//   "为什么长上下文推理这么慢？RedKnot如何用1个百分点的质量代价换来2–5倍TTFT加速" (bjdmk.com.cn), section
//     二 ③ SegPagedAttention: KV pages per (layer, head, segment); global heads read all context
//     pages, local heads physically keep only sink plus recent-window pages.
//   "RedKnot - Xiaohongshuが開発した…" (aiboss88.com), section RedKnotの使い方: a stable head-class
//     map (PROFILE), global/local KV pools filled by head (BUILDSTATE), per-request choice of which
//     KV to reuse and which ranges to recompute (SELECTVISIBLESTATE), fused execution (EXECUTE).
// The allocator policy, the page-table form and the schedule are this library's own design.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <exception>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "rk_internal.h"
#include "rk_ops.h"
#include "rk_sched.h"
#include "rk_sched_ops.h"
#include "rk_seg.h"

namespace {

thread_local std::string g_err;

rk_status fail(rk_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

rk_status hip_fail(hipError_t e, const char *what) {
  return fail(RK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
using rk::kXcd;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Sum over x in [a, b] of min(cap, max(0, x - shift)), exact.
int64_t sum_clamped(int64_t a, int64_t b, int64_t shift, int64_t cap) {
  if (a > b || cap <= 0) return 0;
  // ramp part: x - shift in (0, cap) -> x in [shift + 1, shift + cap - 1]
  int64_t r0 = std::max(a, shift + 1), r1 = std::min(b, shift + cap - 1);
  int64_t s = 0;
  if (r0 <= r1) s += (r0 + r1 - 2 * shift) * (r1 - r0 + 1) / 2;
  // saturated part: x >= shift + cap
  int64_t c0 = std::max(a, shift + cap);
  if (c0 <= b) s += cap * (b - c0 + 1);
  return s;
}

// Visible (query, key) pairs of one (kv head, seq) per q head: queries at positions [qs, L).
int64_t visible_pairs(int cls, int64_t qs, int64_t L, int64_t S, int64_t W) {
  if (qs >= L) return 0;
  // positions i in [qs, L-1]; x = i + 1 in [qs+1, L]
  if (cls == RK_GLOBAL) return (L * (L + 1) - qs * (qs + 1)) / 2;
  // window part: min(x, W) = x - max(0, x - W)
  int64_t win = (L * (L + 1) - qs * (qs + 1)) / 2 - sum_clamped(qs + 1, L, W, INT64_MAX / 4);
  // sink part left of the window: min(S, max(0, x - W))
  int64_t snk = sum_clamped(qs + 1, L, W, S);
  return win + snk;
}

// Logical pages [p0, p1) of the token range [a, b), empty when a >= b.
struct PageRun {
  int32_t p0, p1;
};

// Held pages of one (layer, kv head, seq): up to two runs, ascending and disjoint.
int held_runs(int cls, int32_t qs, int32_t L, int32_t S, int32_t W, int32_t P, PageRun out[2]) {
  if (L <= 0) return 0;
  if (cls == RK_GLOBAL) {
    out[0] = {0, (int32_t)ceil_div(L, P)};
    return 1;
  }
  int n = 0;
  int32_t sink_end = std::min(S, L);
  PageRun sink{0, 0}, win{0, 0};
  bool has_sink = sink_end > 0, has_win = false;
  if (has_sink) sink = {0, (sink_end - 1) / P + 1};
  int32_t wlo = std::max(0, qs - W + 1);
  if (wlo < L) {
    has_win = true;
    win = {wlo / P, (L - 1) / P + 1};
  }
  if (has_sink && has_win && sink.p1 >= win.p0) {
    out[n++] = {0, std::max(sink.p1, win.p1)};
  } else {
    if (has_sink) out[n++] = sink;
    if (has_win) out[n++] = win;
  }
  return n;
}

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }
int32_t log2i(int32_t x) {
  int32_t r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

struct StagingBuf {
  void *ptr = nullptr;
  size_t bytes = 0;
};

}  // namespace

struct rk_pool {
  rk_pool_desc desc{};
  std::vector<int32_t> free_stack;  // back() is the head of the free list
  int64_t live_tables = 0;
  std::vector<StagingBuf> staging_cache;
};

struct rk_tables {
  rk_pool *pool = nullptr;
  int32_t layer_begin = 0, layer_end = 0, num_seqs = 0, H = 0, Hkv = 0, G = 0, T = 0, P = 0, D = 0;
  int32_t elem_bytes = 2;
  int32_t sink = 0, window = 1;
  // q_start: the LOCAL heads' first query position; q_begin: the GLOBAL heads' (<= q_start), where
  // a sequence's packed rows begin
  std::vector<int32_t> q_start, q_begin, kv_len, cu_q;
  std::vector<uint8_t> head_class;  // [num_layers * Hkv]
  // held pages per key k = ((l - layer_begin) * Hkv + g) * num_seqs + b, logical pages ascending
  std::vector<int64_t> held_off;
  std::vector<int32_t> held_logical, held_phys;
  std::vector<std::vector<rk::Item>> items;     // per layer of the call, in launch order
  std::vector<std::vector<int32_t>> app_items;  // per layer: (seq, logical page) pairs
  std::vector<std::vector<rk::MassUnit>> mass_units;  // per layer: per-key mass work units, launch order
  std::vector<int32_t> mass_steps;                    // per layer: query steps per mass unit
  bool decode_shaped = false;                          // every sequence has at most one query row
  std::vector<std::vector<rk::DecItem>> dec_items;     // per layer: split-KV decode items, slot order
  std::vector<std::vector<int32_t>> dec_comb;          // per layer: first item of (seq, kv head)
  // device view
  void *d_ws = nullptr;
  size_t ws_used = 0;
  struct LayerDev {
    const int32_t *page_base;
    const int32_t *page_ids;
    const uint8_t *head_class;
    const rk::Item *items;
    const rk::ItemCtx *ictx;
    const int32_t *app;
    const rk::MassUnit *mass_units;
    const rk::DecItem *dec_items;
    const int32_t *dec_comb;
  };
  std::vector<LayerDev> dev;
  const rk::SeqInfo *d_seqs = nullptr;
  float *d_part_o = nullptr, *d_part_lse = nullptr;  // decode partials, shared by the layers
  const int32_t *d_pack_ids = nullptr;  // held pages in (seq, layer, kv head, logical page) order
  std::vector<int64_t> pack_off;        // [num_seqs + 1]: first packed page of each sequence
  StagingBuf staging;
  hipEvent_t ev = nullptr;
  bool trimmed = false;
  rk_tables_stats stats{};

  int64_t key(int32_t l, int32_t g, int32_t b) const {
    return ((int64_t)(l - layer_begin) * Hkv + g) * num_seqs + b;
  }
  int32_t n_logical(int32_t b) const { return (int32_t)ceil_div(kv_len[b], P); }
  int32_t class_start(int cls, int32_t b) const { return cls == RK_GLOBAL ? q_begin[b] : q_start[b]; }
};

namespace {

// Device workspace layout of one build.  Offsets are relative to the workspace base.
struct WsLayout {
  size_t seqs = 0;
  std::vector<size_t> page_base, page_ids, head_class, items, ictx, app, mass, dec_items, dec_comb;
  size_t part_o = 0, part_lse = 0;  // decode-shaped calls only
  size_t pack_ids = 0;              // the held pages in hand-off order
  size_t total = 0;
};

// Host schedules computed while sizing the workspace.
struct CallSched {
  std::vector<std::vector<rk::MassUnit>> mass;
  std::vector<int32_t> mass_steps;
  bool decode = false;
  std::vector<std::vector<rk::DecItem>> dec;
  std::vector<std::vector<int32_t>> comb;
};

// first packed position of sequence b: the GLOBAL heads' start
int32_t batch_q_begin(const rk_batch_desc *bd, int32_t b) {
  return bd->q_start_global ? bd->q_start_global[b] : bd->q_start[b];
}

rk_status check_batch(const rk_pool *pool, const rk_batch_desc *bd) {
  if (!pool || !bd) return fail(RK_ERR_INVALID_ARG, "null pool or batch");
  const rk_pool_desc &pd = pool->desc;
  if (bd->layer_begin < 0 || bd->layer_end > pd.num_layers || bd->layer_begin >= bd->layer_end)
    return fail(RK_ERR_INVALID_ARG, "layer range [%d, %d) outside [0, %d)", bd->layer_begin, bd->layer_end,
                pd.num_layers);
  if (bd->num_seqs < 0) return fail(RK_ERR_INVALID_ARG, "num_seqs < 0");
  if (bd->num_q_heads <= 0 || bd->num_q_heads % pd.num_kv_heads != 0)
    return fail(RK_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                bd->num_q_heads, pd.num_kv_heads);
  if (bd->num_q_heads / pd.num_kv_heads > rk::kRowsPerItem)
    return fail(RK_ERR_UNSUPPORTED, "more than %d q heads per KV head", rk::kRowsPerItem);
  if (bd->sink < 0) return fail(RK_ERR_INVALID_ARG, "sink < 0");
  if (bd->window < 1) return fail(RK_ERR_INVALID_ARG, "window < 1");
  if (bd->num_seqs > 0 && (!bd->q_start || !bd->kv_len)) return fail(RK_ERR_INVALID_ARG, "null q_start/kv_len");
  if (!bd->head_class) return fail(RK_ERR_INVALID_ARG, "null head_class");
  int64_t total_q = 0;
  for (int32_t b = 0; b < bd->num_seqs; ++b) {
    if (bd->kv_len[b] < 0 || bd->q_start[b] < 0 || bd->q_start[b] > bd->kv_len[b])
      return fail(RK_ERR_INVALID_ARG, "seq %d: need 0 <= q_start (%d) <= kv_len (%d)", b, bd->q_start[b],
                  bd->kv_len[b]);
    if (bd->q_start_global && (bd->q_start_global[b] < 0 || bd->q_start_global[b] > bd->q_start[b]))
      return fail(RK_ERR_INVALID_ARG, "seq %d: need 0 <= q_start_global (%d) <= q_start (%d)", b,
                  bd->q_start_global[b], bd->q_start[b]);
    total_q += bd->kv_len[b] - batch_q_begin(bd, b);
  }
  if (total_q > INT32_MAX) return fail(RK_ERR_UNSUPPORTED, "more than 2^31 query tokens");
  for (int64_t i = 0; i < (int64_t)pd.num_layers * pd.num_kv_heads; ++i)
    if (bd->head_class[i] > 1) return fail(RK_ERR_INVALID_ARG, "head_class[%lld] = %d", (long long)i, bd->head_class[i]);
  return RK_OK;
}

// The per-key mass units and the decode items of each layer are scheduled here (their counts size the
// workspace, through bounds that do not depend on the head classes, so that one workspace serves
// every layer of a model) and returned in *sched when it is not null.
WsLayout plan_ws(const rk_pool *pool, const rk_batch_desc *bd, CallSched *sched) {
  const rk_pool_desc &pd = pool->desc;
  WsLayout w;
  std::vector<int32_t> q_begin(std::max(1, bd->num_seqs));
  bool decode = true;  // every sequence has at most one query row
  for (int32_t b = 0; b < bd->num_seqs; ++b) {
    q_begin[b] = batch_q_begin(bd, b);
    decode = decode && bd->kv_len[b] - q_begin[b] <= 1;
  }
  const int32_t nl = bd->layer_end - bd->layer_begin;
  const int32_t G = bd->num_q_heads / pd.num_kv_heads;
  const int32_t T = rk::kRowsPerItem / G;
  decode = decode && G <= 16;
  if (sched) {
    sched->mass.assign(nl, {});
    sched->mass_steps.assign(nl, rk::kMassChunkSteps);
    sched->decode = decode;
    sched->dec.assign(decode ? nl : 0, {});
    sched->comb.assign(decode ? nl : 0, {});
  }
  size_t off = 0;
  w.seqs = off;
  off = align_up(off + sizeof(rk::SeqInfo) * std::max(1, bd->num_seqs));
  int64_t n_logical = 0, n_items = 0, n_app = 0;
  for (int32_t b = 0; b < bd->num_seqs; ++b) {
    int32_t L = bd->kv_len[b], qs = q_begin[b];
    n_logical += ceil_div(L, pd.page_size);
    n_items += ceil_div(L - qs, T);
    if (L > qs) n_app += (L - 1) / pd.page_size - qs / pd.page_size + 1;
  }
  int64_t dec_bound = 0;
  for (int32_t l = bd->layer_begin; l < bd->layer_end; ++l) {
    w.page_base.push_back(off);
    off = align_up(off + sizeof(int32_t) * std::max<int64_t>(1, (int64_t)pd.num_kv_heads * bd->num_seqs));
    w.page_ids.push_back(off);
    off = align_up(off + sizeof(int32_t) * std::max<int64_t>(1, n_logical * pd.num_kv_heads));
    w.head_class.push_back(off);
    off = align_up(off + pd.num_kv_heads);
    w.items.push_back(off);
    // the XCD-interleaved schedule pads short bins: at most kXcd slots per real item
    off = align_up(off + sizeof(rk::Item) * std::max<int64_t>(1, n_items * pd.num_kv_heads * kXcd));
    w.ictx.push_back(off);
    off = align_up(off + sizeof(rk::ItemCtx) * std::max<int64_t>(1, n_items * pd.num_kv_heads * kXcd));
    w.app.push_back(off);
    off = align_up(off + 2 * sizeof(int32_t) * std::max<int64_t>(1, n_app));
    rk::SchedInput si{bd->num_seqs, pd.num_kv_heads, T, pd.head_dim, pd.dtype == RK_F32 ? 4 : 2, bd->sink, bd->window,
                      &bd->head_class[(size_t)l * pd.num_kv_heads], bd->kv_len, bd->q_start, q_begin.data()};
    // the mass pass supports G <= 16 (above, no rows of a step fit and it has no units)
    const int32_t mk = rk::mass_keys_per_unit(G), mt = rk::mass_tokens_per_step(G);
    const int32_t ms = G <= 16 ? rk::mass_steps_per_chunk(si, mk, mt) : rk::kMassChunkSteps;
    if (sched && G <= 16) {
      rk::mass_schedule(si, mk, mt, ms, sched->mass[l - bd->layer_begin]);
      sched->mass_steps[l - bd->layer_begin] = ms;
    }
    w.mass.push_back(off);
    off = align_up(off + sizeof(rk::MassUnit) * std::max<int64_t>(1, G <= 16 ? rk::mass_units_bound(si, mk, mt, ms) : 0));
    if (decode) {
      if (sched) rk::decode_schedule(si, sched->dec[l - bd->layer_begin], sched->comb[l - bd->layer_begin]);
      dec_bound = rk::decode_items_bound(si);
      w.dec_items.push_back(off);
      off = align_up(off + sizeof(rk::DecItem) * dec_bound);
      w.dec_comb.push_back(off);
      off = align_up(off + sizeof(int32_t) * ((int64_t)bd->num_seqs * pd.num_kv_heads + 1));
    }
  }
  if (decode) {
    const int64_t slots = ceil_div(dec_bound, rk::kDecodeWaves);  // one partial per workgroup
    w.part_o = off;
    off = align_up(off + sizeof(float) * slots * G * pd.head_dim);
    w.part_lse = off;
    off = align_up(off + sizeof(float) * slots * G);
  }
  w.pack_ids = off;  // at most every logical page of every (layer, kv head, seq)
  off = align_up(off + sizeof(int32_t) * std::max<int64_t>(1, n_logical * pd.num_kv_heads * nl));
  w.total = off;
  return w;
}

void push_free(rk_pool *pool, const std::vector<int32_t> &ids) {
  for (int32_t id : ids) pool->free_stack.push_back(id);
}

StagingBuf take_staging(rk_pool *pool, size_t bytes, hipError_t *err) {
  *err = hipSuccess;
  size_t best = SIZE_MAX;
  size_t bi = 0;
  for (size_t i = 0; i < pool->staging_cache.size(); ++i) {
    size_t b = pool->staging_cache[i].bytes;
    if (b >= bytes && b < best) best = b, bi = i;
  }
  if (best != SIZE_MAX) {
    StagingBuf s = pool->staging_cache[bi];
    pool->staging_cache.erase(pool->staging_cache.begin() + bi);
    return s;
  }
  StagingBuf s;
  s.bytes = std::max<size_t>(bytes, 1 << 16);
  *err = hipHostMalloc(&s.ptr, s.bytes, hipHostMallocDefault);
  if (*err != hipSuccess) s = StagingBuf{};
  return s;
}

rk_status release_device(rk_tables *t) {
  rk_status st = RK_OK;
  if (t->ev) {
    hipError_t e = hipEventSynchronize(t->ev);
    if (e != hipSuccess) st = hip_fail(e, "hipEventSynchronize");
    hipEventDestroy(t->ev);
    t->ev = nullptr;
  }
  if (t->staging.ptr) {
    t->pool->staging_cache.push_back(t->staging);
    t->staging = StagingBuf{};
  }
  return st;
}

// Everything of a call but its physical pages and device view: shape, held logical pages, schedules
// and counters.  No side effects on the pool.
rk_status prepare_tables(rk_pool *pool, const rk_batch_desc *bd, void *d_ws, size_t ws_bytes, WsLayout &ws,
                         std::unique_ptr<rk_tables> &out) {
  rk_status st = check_batch(pool, bd);
  if (st != RK_OK) return st;
  const rk_pool_desc &pd = pool->desc;
  CallSched sched;
  ws = plan_ws(pool, bd, &sched);
  if (d_ws) {
    if ((reinterpret_cast<uintptr_t>(d_ws) & (kAlign - 1)) != 0)
      return fail(RK_ERR_INVALID_ARG, "workspace not 256-byte aligned");
    if (ws_bytes < ws.total)
      return fail(RK_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", ws_bytes, ws.total);
  }

  std::unique_ptr<rk_tables> t(new rk_tables());
  t->pool = pool;
  t->mass_units = std::move(sched.mass);
  t->mass_steps = std::move(sched.mass_steps);
  t->decode_shaped = sched.decode;
  t->dec_items = std::move(sched.dec);
  t->dec_comb = std::move(sched.comb);
  t->layer_begin = bd->layer_begin;
  t->layer_end = bd->layer_end;
  t->num_seqs = bd->num_seqs;
  t->H = bd->num_q_heads;
  t->Hkv = pd.num_kv_heads;
  t->G = t->H / t->Hkv;
  t->T = rk::kRowsPerItem / t->G;
  t->P = pd.page_size;
  t->D = pd.head_dim;
  t->elem_bytes = pd.dtype == RK_F32 ? 4 : 2;
  t->sink = bd->sink;
  t->window = bd->window;
  t->q_start.assign(bd->q_start, bd->q_start + bd->num_seqs);
  t->q_begin.resize(bd->num_seqs);
  for (int32_t b = 0; b < bd->num_seqs; ++b) t->q_begin[b] = batch_q_begin(bd, b);
  t->kv_len.assign(bd->kv_len, bd->kv_len + bd->num_seqs);
  t->cu_q.resize(bd->num_seqs + 1, 0);
  for (int32_t b = 0; b < bd->num_seqs; ++b) t->cu_q[b + 1] = t->cu_q[b] + (t->kv_len[b] - t->q_begin[b]);
  t->head_class.assign(bd->head_class, bd->head_class + (size_t)pd.num_layers * pd.num_kv_heads);

  // held pages of every (layer, kv head, seq), in allocation order
  const int32_t nl = bd->layer_end - bd->layer_begin;
  const int64_t nkeys = (int64_t)nl * t->Hkv * t->num_seqs;
  t->held_off.assign(nkeys + 1, 0);
  std::vector<PageRun> runs(nkeys * 2);
  std::vector<int8_t> nrun(nkeys);
  for (int32_t l = bd->layer_begin; l < bd->layer_end; ++l)
    for (int32_t g = 0; g < t->Hkv; ++g)
      for (int32_t b = 0; b < t->num_seqs; ++b) {
        int64_t k = t->key(l, g, b);
        int cls = t->head_class[(size_t)l * t->Hkv + g];
        nrun[k] = (int8_t)held_runs(cls, t->q_start[b], t->kv_len[b], t->sink, t->window, t->P, &runs[2 * k]);
        int64_t n = 0;
        for (int r = 0; r < nrun[k]; ++r) n += runs[2 * k + r].p1 - runs[2 * k + r].p0;
        t->held_off[k + 1] = t->held_off[k] + n;
      }
  const int64_t need = t->held_off[nkeys];
  t->held_logical.resize(need);
  t->held_phys.assign(need, -1);
  for (int64_t k = 0; k < nkeys; ++k) {
    int64_t o = t->held_off[k];
    for (int r = 0; r < nrun[k]; ++r)
      for (int32_t p = runs[2 * k + r].p0; p < runs[2 * k + r].p1; ++p) t->held_logical[o++] = p;
  }

  // schedules
  t->items.resize(nl);
  t->app_items.resize(nl);
  int64_t key_tiles = 0, n_items = 0;
  for (int32_t l = bd->layer_begin; l < bd->layer_end; ++l) {
    rk::SchedInput si{t->num_seqs, t->Hkv, t->T, t->D, t->elem_bytes, t->sink, t->window,
                      &t->head_class[(size_t)l * t->Hkv], t->kv_len.data(), t->q_start.data(), t->q_begin.data()};
    rk::schedule_layer(si, t->items[l - bd->layer_begin]);
    for (const rk::Item &it : t->items[l - bd->layer_begin]) {
      key_tiles += it.tiles;
      n_items += it.seq >= 0 ? 1 : 0;
    }
    std::vector<int32_t> &app = t->app_items[l - bd->layer_begin];
    for (int32_t b = 0; b < t->num_seqs; ++b) {
      int32_t qs = t->q_begin[b], L = t->kv_len[b];  // pages from the earliest class start
      if (L <= qs) continue;
      for (int32_t p = qs / t->P; p <= (L - 1) / t->P; ++p) {
        app.push_back(b);
        app.push_back(p);
      }
    }
  }

  // counters
  rk_tables_stats &s = t->stats;
  s.pages_held = need;
  s.total_q = t->cu_q[t->num_seqs];
  s.work_items = n_items;
  s.key_tiles = key_tiles;
  s.workspace_bytes = d_ws ? (int64_t)ws.total : 0;
  for (int32_t l = bd->layer_begin; l < bd->layer_end; ++l)
    for (int32_t g = 0; g < t->Hkv; ++g) {
      int cls = t->head_class[(size_t)l * t->Hkv + g];
      for (int32_t b = 0; b < t->num_seqs; ++b) {
        int64_t v = (int64_t)t->G * visible_pairs(cls, t->class_start(cls, b), t->kv_len[b], t->sink, t->window);
        s.visible_pairs += v;
        if (cls == RK_GLOBAL) s.visible_pairs_global += v;
      }
    }
  out = std::move(t);
  return RK_OK;
}

// Pinned staging and the upload event of t's device view (before the pool is touched, so that a
// failure leaves it unchanged).
rk_status acquire_staging(rk_pool *pool, rk_tables *t, const WsLayout &ws) {
  hipError_t e;
  t->staging = take_staging(pool, ws.total, &e);
  if (e != hipSuccess) return hip_fail(e, "hipHostMalloc (table staging)");
  e = hipEventCreateWithFlags(&t->ev, hipEventDisableTiming);
  if (e != hipSuccess) {
    pool->staging_cache.push_back(t->staging);
    t->staging = StagingBuf{};
    t->ev = nullptr;
    return hip_fail(e, "hipEventCreate");
  }
  return RK_OK;
}

// Writes t's device view (pages assigned) into its staging and uploads it into d_ws on the stream.
// Only the bytes written here travel: the regions are sized by bounds (the item lists for the
// XCD-padded schedule, the mass units for any head classes), and every byte a kernel reads lies in a
// written span.  Spans closer than kUploadGap are sent as one copy.
hipError_t fill_and_upload(rk_tables *t, const WsLayout &ws, void *d_ws, void *stream) {
  constexpr size_t kUploadGap = 256 << 10;
  char *h = static_cast<char *>(t->staging.ptr);
  std::vector<std::pair<size_t, size_t>> spans;  // (offset, bytes) written
  auto wrote = [&](size_t off, size_t bytes) {
    if (bytes) spans.emplace_back(off, bytes);
  };
  rk::SeqInfo *seqs = reinterpret_cast<rk::SeqInfo *>(h + ws.seqs);
  wrote(ws.seqs, sizeof(rk::SeqInfo) * t->num_seqs);
  int64_t kv_off = 0;  // per-key outputs need it below 2^31 (checked where they are computed)
  for (int32_t b = 0; b < t->num_seqs; ++b) {
    seqs[b] = {t->q_begin[b], t->kv_len[b], t->cu_q[b], t->kv_len[b] - t->q_begin[b], t->q_start[b],
               (int32_t)std::min<int64_t>(kv_off, INT32_MAX)};
    kv_off += t->kv_len[b];
  }
  char *dbase = static_cast<char *>(d_ws);
  t->d_seqs = reinterpret_cast<const rk::SeqInfo *>(dbase + ws.seqs);
  const int32_t nl = t->layer_end - t->layer_begin;
  t->dev.resize(nl);
  for (int32_t l = t->layer_begin; l < t->layer_end; ++l) {
    const int32_t li = l - t->layer_begin;
    int32_t *pbase = reinterpret_cast<int32_t *>(h + ws.page_base[li]);
    int32_t *pids = reinterpret_cast<int32_t *>(h + ws.page_ids[li]);
    int32_t off = 0;
    for (int32_t g = 0; g < t->Hkv; ++g)
      for (int32_t b = 0; b < t->num_seqs; ++b) {
        pbase[g * t->num_seqs + b] = off;
        int32_t nlog = t->n_logical(b);
        std::fill(pids + off, pids + off + nlog, -1);
        int64_t k = t->key(l, g, b);
        for (int64_t i = t->held_off[k]; i < t->held_off[k + 1]; ++i) pids[off + t->held_logical[i]] = t->held_phys[i];
        off += nlog;
      }
    wrote(ws.page_base[li], sizeof(int32_t) * t->Hkv * t->num_seqs);
    wrote(ws.page_ids[li], sizeof(int32_t) * off);
    std::memcpy(h + ws.head_class[li], &t->head_class[(size_t)l * t->Hkv], t->Hkv);
    wrote(ws.head_class[li], t->Hkv);
    std::memcpy(h + ws.items[li], t->items[li].data(), sizeof(rk::Item) * t->items[li].size());
    wrote(ws.items[li], sizeof(rk::Item) * t->items[li].size());
    wrote(ws.ictx[li], sizeof(rk::ItemCtx) * t->items[li].size());
    {
      rk::ItemCtx *ctx = reinterpret_cast<rk::ItemCtx *>(h + ws.ictx[li]);
      const uint8_t *cls = &t->head_class[(size_t)l * t->Hkv];
      const int32_t lg = log2i(t->P);
      for (size_t i = 0; i < t->items[li].size(); ++i) {
        const rk::Item &it = t->items[li][i];
        if (it.seq < 0) {
          ctx[i] = {-1, 0, 0, 0, 0, 0, 0, 0};
          continue;
        }
        const int32_t b = it.seq, g = it.kv_head;
        const int32_t qb = t->q_begin[b], L = t->kv_len[b], nq = L - qb;
        const int32_t i_max = qb + std::min(it.tok0 + t->T, nq) - 1;
        const int32_t po = pbase[g * t->num_seqs + b];
        ctx[i] = {g | ((int32_t)cls[g] << 16), it.tok0, t->cu_q[b], qb, nq, L, po, pids[po + (i_max >> lg)]};
      }
    }
    std::memcpy(h + ws.app[li], t->app_items[li].data(), sizeof(int32_t) * t->app_items[li].size());
    wrote(ws.app[li], sizeof(int32_t) * t->app_items[li].size());
    std::memcpy(h + ws.mass[li], t->mass_units[li].data(), sizeof(rk::MassUnit) * t->mass_units[li].size());
    wrote(ws.mass[li], sizeof(rk::MassUnit) * t->mass_units[li].size());
    const rk::DecItem *dec_items = nullptr;
    const int32_t *dec_comb = nullptr;
    if (t->decode_shaped) {
      std::memcpy(h + ws.dec_items[li], t->dec_items[li].data(), sizeof(rk::DecItem) * t->dec_items[li].size());
      std::memcpy(h + ws.dec_comb[li], t->dec_comb[li].data(), sizeof(int32_t) * t->dec_comb[li].size());
      wrote(ws.dec_items[li], sizeof(rk::DecItem) * t->dec_items[li].size());
      wrote(ws.dec_comb[li], sizeof(int32_t) * t->dec_comb[li].size());
      dec_items = reinterpret_cast<const rk::DecItem *>(dbase + ws.dec_items[li]);
      dec_comb = reinterpret_cast<const int32_t *>(dbase + ws.dec_comb[li]);
    }
    t->dev[li] = {reinterpret_cast<const int32_t *>(dbase + ws.page_base[li]),
                  reinterpret_cast<const int32_t *>(dbase + ws.page_ids[li]),
                  reinterpret_cast<const uint8_t *>(dbase + ws.head_class[li]),
                  reinterpret_cast<const rk::Item *>(dbase + ws.items[li]),
                  reinterpret_cast<const rk::ItemCtx *>(dbase + ws.ictx[li]),
                  reinterpret_cast<const int32_t *>(dbase + ws.app[li]),
                  reinterpret_cast<const rk::MassUnit *>(dbase + ws.mass[li]),
                  dec_items,
                  dec_comb};
  }
  {
    int32_t *ids = reinterpret_cast<int32_t *>(h + ws.pack_ids);
    t->pack_off.assign(t->num_seqs + 1, 0);
    int64_t n = 0;
    for (int32_t b = 0; b < t->num_seqs; ++b) {
      t->pack_off[b] = n;
      for (int32_t l = t->layer_begin; l < t->layer_end; ++l)
        for (int32_t g = 0; g < t->Hkv; ++g) {
          const int64_t k = t->key(l, g, b);
          for (int64_t i = t->held_off[k]; i < t->held_off[k + 1]; ++i) ids[n++] = t->held_phys[i];
        }
    }
    t->pack_off[t->num_seqs] = n;
    t->d_pack_ids = reinterpret_cast<const int32_t *>(dbase + ws.pack_ids);
    wrote(ws.pack_ids, sizeof(int32_t) * n);
  }
  t->d_part_o = t->decode_shaped ? reinterpret_cast<float *>(dbase + ws.part_o) : nullptr;
  t->d_part_lse = t->decode_shaped ? reinterpret_cast<float *>(dbase + ws.part_lse) : nullptr;
  hipStream_t sm = static_cast<hipStream_t>(stream);
  std::sort(spans.begin(), spans.end());
  hipError_t e = hipSuccess;
  for (size_t i = 0; i < spans.size() && e == hipSuccess;) {
    const size_t a = spans[i].first;
    size_t z = a + spans[i].second;
    for (++i; i < spans.size() && spans[i].first <= z + kUploadGap; ++i) z = std::max(z, spans[i].first + spans[i].second);
    e = hipMemcpyAsync(dbase + a, h + a, z - a, hipMemcpyHostToDevice, sm);
  }
  if (e == hipSuccess) e = hipEventRecord(t->ev, sm);
  if (e == hipSuccess) {
    t->d_ws = d_ws;
    t->ws_used = ws.total;
  }
  return e;
}

rk_status build_tables_impl(rk_pool *pool, const rk_batch_desc *bd, void *d_ws, size_t ws_bytes, void *stream,
                            rk_tables **out) {
  if (!out) return fail(RK_ERR_INVALID_ARG, "null out");
  WsLayout ws;
  std::unique_ptr<rk_tables> t;
  rk_status st = prepare_tables(pool, bd, d_ws, ws_bytes, ws, t);
  if (st != RK_OK) return st;
  const int64_t need = (int64_t)t->held_phys.size();
  if (need > (int64_t)pool->free_stack.size())
    return fail(RK_ERR_OUT_OF_PAGES, "call holds %lld pages, %zu free", (long long)need, pool->free_stack.size());
  if (d_ws) {
    st = acquire_staging(pool, t.get(), ws);
    if (st != RK_OK) return st;
  }
  // allocate: pop from the head of the free list in (layer, kv head, seq, logical page) order
  for (int64_t i = 0; i < need; ++i) {
    t->held_phys[i] = pool->free_stack.back();
    pool->free_stack.pop_back();
  }
  if (d_ws) {
    hipError_t e = fill_and_upload(t.get(), ws, d_ws, stream);
    if (e != hipSuccess) {
      // undo the allocation so that the pool is unchanged
      for (int64_t i = need - 1; i >= 0; --i) pool->free_stack.push_back(t->held_phys[i]);
      hipStreamSynchronize(static_cast<hipStream_t>(stream));
      release_device(t.get());
      return hip_fail(e, "table upload");
    }
  }
  pool->live_tables++;
  *out = t.release();
  return RK_OK;
}

// The call after t's on the same sequences: sequence b gains n_new[b] tokens, which are its queries
// (q_start = q_start_global = the old kv_len).  Pages that stay held keep their physical page and
// contents; pages no longer held are freed first (in (layer, kv head, seq, logical page) order),
// then the new pages are taken from the head of the free list in the same order.
rk_status advance_desc(const rk_tables *t, const int32_t *n_new, std::vector<int32_t> &qs, std::vector<int32_t> &kv,
                       rk_batch_desc &nb) {
  if (t->num_seqs > 0 && !n_new) return fail(RK_ERR_INVALID_ARG, "null n_new");
  qs.resize(std::max(1, t->num_seqs));
  kv.resize(std::max(1, t->num_seqs));
  for (int32_t b = 0; b < t->num_seqs; ++b) {
    if (n_new[b] < 0 || (int64_t)t->kv_len[b] + n_new[b] > INT32_MAX)
      return fail(RK_ERR_INVALID_ARG, "seq %d: n_new %d out of range", b, n_new[b]);
    qs[b] = t->kv_len[b];
    kv[b] = t->kv_len[b] + n_new[b];
  }
  nb = rk_batch_desc{};
  nb.layer_begin = t->layer_begin;
  nb.layer_end = t->layer_end;
  nb.num_seqs = t->num_seqs;
  nb.num_q_heads = t->H;
  nb.q_start = qs.data();
  nb.kv_len = kv.data();
  nb.head_class = t->head_class.data();
  nb.sink = t->sink;
  nb.window = t->window;
  nb.q_start_global = nullptr;
  return RK_OK;
}

rk_status advance_impl(rk_pool *pool, rk_tables *t, const int32_t *n_new, void *d_ws, size_t ws_bytes, void *stream) {
  std::vector<int32_t> qs, kv;
  rk_batch_desc nb;
  rk_status st = advance_desc(t, n_new, qs, kv, nb);
  if (st != RK_OK) return st;
  WsLayout ws;
  std::unique_ptr<rk_tables> nt;
  st = prepare_tables(pool, &nb, d_ws, ws_bytes, ws, nt);
  if (st != RK_OK) return st;
  // pages per key: kept (same logical page), freed (old only), new (new only)
  std::vector<int32_t> freed;
  std::vector<int64_t> fresh;  // indices into nt->held_phys
  const int64_t nkeys = (int64_t)t->held_off.size() - 1;
  for (int64_t k = 0; k < nkeys; ++k) {
    int64_t i = t->held_off[k], i1 = t->held_off[k + 1];
    int64_t j = nt->held_off[k], j1 = nt->held_off[k + 1];
    while (i < i1 || j < j1) {
      if (j == j1 || (i < i1 && t->held_logical[i] < nt->held_logical[j])) {
        freed.push_back(t->held_phys[i++]);
      } else if (i == i1 || nt->held_logical[j] < t->held_logical[i]) {
        fresh.push_back(j++);
      } else {
        nt->held_phys[j++] = t->held_phys[i++];
      }
    }
  }
  if ((int64_t)fresh.size() > (int64_t)(pool->free_stack.size() + freed.size()))
    return fail(RK_ERR_OUT_OF_PAGES, "advance needs %zu new pages, %zu free after releasing %zu", fresh.size(),
                pool->free_stack.size() + freed.size(), freed.size());
  st = release_device(t);  // the previous upload has landed; its staging goes back to the pool
  if (st != RK_OK) return st;
  if (d_ws) {
    st = acquire_staging(pool, nt.get(), ws);
    if (st != RK_OK) return st;
  }
  // from here on the pool changes
  push_free(pool, freed);
  for (int64_t j : fresh) {
    nt->held_phys[j] = pool->free_stack.back();
    pool->free_stack.pop_back();
  }
  hipError_t e = hipSuccess;
  if (d_ws) e = fill_and_upload(nt.get(), ws, d_ws, stream);
  // t becomes the new call (same handle); its old staging and event were released above
  nt->pool = pool;
  if (!d_ws || e != hipSuccess) nt->d_ws = nullptr;
  *t = std::move(*nt);
  if (e != hipSuccess) return hip_fail(e, "table upload (the tables keep their pages, without a device view)");
  return RK_OK;
}

rk_status check_device_tables(const rk_pool *pool, const rk_tables *t, int32_t layer) {
  if (!pool || !t) return fail(RK_ERR_INVALID_ARG, "null pool or tables");
  if (t->pool != pool) return fail(RK_ERR_INVALID_ARG, "tables belong to another pool");
  if (!t->d_ws) return fail(RK_ERR_STATE, "tables were built on the host only (no workspace)");
  if (t->trimmed) return fail(RK_ERR_STATE, "tables were trimmed; they describe the retained state only");
  if (layer < t->layer_begin || layer >= t->layer_end)
    return fail(RK_ERR_INVALID_ARG, "layer %d outside the call's range [%d, %d)", layer, t->layer_begin,
                t->layer_end);
  return RK_OK;
}

rk::KvWriteParams kv_params(const rk_pool *pool, const rk_tables *t, int32_t layer) {
  rk::KvWriteParams p{};
  const rk_tables::LayerDev &d = t->dev[layer - t->layer_begin];
  p.k_pages = pool->desc.k_pages;
  p.v_pages = pool->desc.v_pages;
  p.sink = t->sink;
  p.window = t->window;
  p.page_base = d.page_base;
  p.page_ids = d.page_ids;
  p.seqs = t->d_seqs;
  p.head_class = d.head_class;
  p.num_seqs = t->num_seqs;
  p.Hkv = t->Hkv;
  p.P = t->P;
  p.log2P = log2i(t->P);
  return p;
}

rk_status append_impl(rk_pool *pool, const rk_tables *t, int32_t layer, const void *k_new, const void *v_new,
                      void *stream) {
  if (!k_new || !v_new) return fail(RK_ERR_INVALID_ARG, "null k_new / v_new");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(RK_ERR_INVALID_ARG, "k_new / v_new not 16-byte aligned");
  rk::KvWriteParams p = kv_params(pool, t, layer);
  p.app_items = t->dev[layer - t->layer_begin].app;
  p.n_items = (int32_t)(t->app_items[layer - t->layer_begin].size() / 2);
  p.k_src = k_new;
  p.v_src = v_new;
  if (p.n_items == 0) return RK_OK;
  hipError_t e = rk::launch_append(p, pool->desc.dtype, pool->desc.head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append kernel launch");
  return RK_OK;
}

// Decode of one layer; static_partials: the split-KV partials go to the per-GPU static array instead
// of the tables' workspace, and nothing is allocated.
rk_status decode_impl(rk_pool *pool, const rk_tables *t, int32_t layer, const void *q, const void *k_new,
                      const void *v_new, void *o, float *lse, float softmax_scale, void *stream,
                      bool static_partials) {
  rk_status st = check_device_tables(pool, t, layer);
  if (st != RK_OK) return st;
  if (pool->desc.dtype != RK_BF16) return fail(RK_ERR_UNSUPPORTED, "decode needs a bf16 pool");
  if (t->G > 16) return fail(RK_ERR_UNSUPPORTED, "decode supports at most 16 q heads per KV head");
  if (!t->decode_shaped)
    return fail(RK_ERR_STATE, "decode needs tables whose sequences have at most one query row each");
  const int64_t total_q = t->cu_q[t->num_seqs];
  if (total_q == 0) return RK_OK;
  if (!q || !o || !aligned16(q) || !aligned16(o)) return fail(RK_ERR_INVALID_ARG, "q / o null or not 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(RK_ERR_INVALID_ARG, "lse not 4-byte aligned");
  if (!(softmax_scale <= 0.0f) && !std::isfinite(softmax_scale)) return fail(RK_ERR_INVALID_ARG, "softmax_scale not finite");
  const int32_t li = layer - t->layer_begin;
  float *part_o = t->d_part_o, *part_lse = t->d_part_lse;
  if (static_partials) {  // checked before anything runs: a rejected call leaves the pool as it was
    const int64_t slots = (int64_t)t->dec_items[li].size() / rk::kDecodeWaves;
    const size_t o_bytes = align_up(sizeof(float) * slots * t->G * pool->desc.head_dim);
    const size_t need = o_bytes + sizeof(float) * slots * t->G;
    if (need > rk::kDecodeScratchBytes)
      return fail(RK_ERR_UNSUPPORTED, "decode partials need %zu bytes, the static scratch holds %zu", need,
                  rk::kDecodeScratchBytes);
    void *base = nullptr;
    hipError_t e = rk::decode_scratch(&base);
    if (e != hipSuccess) return hip_fail(e, "static scratch address");
    part_o = static_cast<float *>(base);
    part_lse = reinterpret_cast<float *>(static_cast<char *>(base) + o_bytes);
  }
  // both NULL: the caller appended the tokens already (rk_seg_append_kv); one NULL is an error.
  // Otherwise the decode kernel appends them itself (the item that ends at kv_len writes its token).
  if (k_new || v_new) {
    if (!k_new || !v_new) return fail(RK_ERR_INVALID_ARG, "null k_new / v_new");
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(RK_ERR_INVALID_ARG, "k_new / v_new not 16-byte aligned");
  }
  const rk_tables::LayerDev &d = t->dev[li];
  rk::DecodeParams p{};
  p.q = q;
  p.o = o;
  p.lse = lse;
  p.k_pages = pool->desc.k_pages;
  p.v_pages = pool->desc.v_pages;
  p.page_base = d.page_base;
  p.page_ids = d.page_ids;
  p.seqs = t->d_seqs;
  p.items = d.dec_items;
  p.comb_off = d.dec_comb;
  p.part_o = part_o;
  p.part_lse = part_lse;
  p.k_src = k_new;
  p.v_src = v_new;
  p.head_class = d.head_class;
  p.sink = t->sink;
  p.window = t->window;
  p.num_seqs = t->num_seqs;
  p.H = t->H;
  p.Hkv = t->Hkv;
  p.G = t->G;
  p.P = t->P;
  p.log2P = log2i(t->P);
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)pool->desc.head_dim);
  p.scale_log2 = scale * 1.4426950408889634f;
  p.total_q = (int32_t)total_q;
  p.n_items = (int32_t)t->dec_items[li].size();
  hipError_t e = rk::launch_decode(p, pool->desc.head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  return RK_OK;
}

}  // namespace

#define RK_GUARD_BEGIN try {
#define RK_GUARD_END                                                     \
  }                                                                      \
  catch (const std::bad_alloc &) {                                       \
    return fail(RK_ERR_INTERNAL, "host out of memory");                  \
  }                                                                      \
  catch (const std::exception &ex) {                                     \
    return fail(RK_ERR_INTERNAL, "internal error: %s", ex.what());       \
  }                                                                      \
  catch (...) {                                                          \
    return fail(RK_ERR_INTERNAL, "internal error");                      \
  }

extern "C" {

const char *rk_status_string(rk_status s) {
  switch (s) {
    case RK_OK: return "RK_OK";
    case RK_ERR_INVALID_ARG: return "RK_ERR_INVALID_ARG";
    case RK_ERR_OUT_OF_PAGES: return "RK_ERR_OUT_OF_PAGES";
    case RK_ERR_WORKSPACE_TOO_SMALL: return "RK_ERR_WORKSPACE_TOO_SMALL";
    case RK_ERR_UNSUPPORTED: return "RK_ERR_UNSUPPORTED";
    case RK_ERR_HIP: return "RK_ERR_HIP";
    case RK_ERR_STATE: return "RK_ERR_STATE";
    case RK_ERR_INTERNAL: return "RK_ERR_INTERNAL";
    default: return "RK_ERR_UNKNOWN";
  }
}

const char *rk_last_error(void) { return g_err.c_str(); }

const char *rk_seg_version(void) { return "rk_seg 0.1 gfx950"; }

rk_status rk_seg_pool_create(const rk_pool_desc *desc, rk_pool **out) {
  RK_GUARD_BEGIN
  if (!desc || !out) return fail(RK_ERR_INVALID_ARG, "null desc or out");
  const rk_pool_desc &d = *desc;
  if (d.num_layers < 1 || d.num_kv_heads < 1) return fail(RK_ERR_INVALID_ARG, "num_layers / num_kv_heads < 1");
  if (d.head_dim != 64 && d.head_dim != 128) return fail(RK_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", d.head_dim);
  if (!is_pow2(d.page_size) || d.page_size < 8 || d.page_size > 256)
    return fail(RK_ERR_UNSUPPORTED, "page_size %d (power of two in [8, 256])", d.page_size);
  if (d.dtype != RK_BF16 && d.dtype != RK_F32) return fail(RK_ERR_UNSUPPORTED, "dtype %d", d.dtype);
  if (d.num_pages < 0 || d.num_pages > INT32_MAX) return fail(RK_ERR_INVALID_ARG, "num_pages %lld", (long long)d.num_pages);
  if (d.num_pages > 0 && (!d.k_pages || !d.v_pages)) return fail(RK_ERR_INVALID_ARG, "null page storage");
  if (!aligned16(d.k_pages) || !aligned16(d.v_pages)) return fail(RK_ERR_INVALID_ARG, "page storage not 16-byte aligned");
  std::unique_ptr<rk_pool> p(new rk_pool());
  p->desc = d;
  p->desc.initial_free_order = nullptr;
  const int32_t n = (int32_t)d.num_pages;
  p->free_stack.resize(n);
  if (d.initial_free_order) {
    std::vector<uint8_t> seen(n, 0);
    for (int32_t i = 0; i < n; ++i) {
      int32_t id = d.initial_free_order[i];
      if (id < 0 || id >= n || seen[id]) return fail(RK_ERR_INVALID_ARG, "initial_free_order is not a permutation");
      seen[id] = 1;
      p->free_stack[n - 1 - i] = id;
    }
  } else {
    for (int32_t i = 0; i < n; ++i) p->free_stack[n - 1 - i] = i;
  }
  *out = p.release();
  return RK_OK;
  RK_GUARD_END
}

rk_status rk_seg_pool_destroy(rk_pool *pool) {
  RK_GUARD_BEGIN
  if (!pool) return fail(RK_ERR_INVALID_ARG, "null pool");
  if (pool->live_tables > 0) return fail(RK_ERR_STATE, "%lld tables still alive", (long long)pool->live_tables);
  for (StagingBuf &s : pool->staging_cache) hipHostFree(s.ptr);
  delete pool;
  return RK_OK;
  RK_GUARD_END
}

rk_status rk_seg_pool_query(const rk_pool *pool, int64_t *free_pages, int64_t *used_pages) {
  if (!pool) return fail(RK_ERR_INVALID_ARG, "null pool");
  if (free_pages) *free_pages = (int64_t)pool->free_stack.size();
  if (used_pages) *used_pages = pool->desc.num_pages - (int64_t)pool->free_stack.size();
  return RK_OK;
}

rk_status rk_seg_pool_free_list(const rk_pool *pool, int32_t *out, int64_t cap, int64_t *n) {
  if (!pool) return fail(RK_ERR_INVALID_ARG, "null pool");
  const int64_t sz = (int64_t)pool->free_stack.size();
  if (n) *n = sz;
  if (out)
    for (int64_t i = 0; i < std::min(cap, sz); ++i) out[i] = pool->free_stack[sz - 1 - i];
  return RK_OK;
}

rk_status rk_seg_tables_workspace_bytes(const rk_pool *pool, const rk_batch_desc *batch, size_t *bytes) {
  RK_GUARD_BEGIN
  if (!bytes) return fail(RK_ERR_INVALID_ARG, "null bytes");
  rk_status st = check_batch(pool, batch);
  if (st != RK_OK) return st;
  *bytes = plan_ws(pool, batch, nullptr).total;
  return RK_OK;
  RK_GUARD_END
}

rk_status rk_seg_build_tables(rk_pool *pool, const rk_batch_desc *batch, void *d_workspace, size_t ws_bytes,
                              void *stream, rk_tables **out) {
  RK_GUARD_BEGIN
  return build_tables_impl(pool, batch, d_workspace, ws_bytes, stream, out);
  RK_GUARD_END
}

rk_status rk_seg_tables_advance_workspace_bytes(const rk_pool *pool, const rk_tables *t, const int32_t *n_new,
                                                size_t *bytes) {
  RK_GUARD_BEGIN
  if (!pool || !t || t->pool != pool || !bytes) return fail(RK_ERR_INVALID_ARG, "null or foreign argument");
  std::vector<int32_t> qs, kv;
  rk_batch_desc nb;
  rk_status st = advance_desc(t, n_new, qs, kv, nb);
  if (st != RK_OK) return st;
  st = check_batch(pool, &nb);
  if (st != RK_OK) return st;
  *bytes = plan_ws(pool, &nb, nullptr).total;
  return RK_OK;
  RK_GUARD_END
}

rk_status rk_seg_tables_advance(rk_pool *pool, rk_tables *t, const int32_t *n_new, void *d_workspace, size_t ws_bytes,
                                void *stream) {
  RK_GUARD_BEGIN
  if (!pool || !t || t->pool != pool) return fail(RK_ERR_INVALID_ARG, "null or foreign tables");
  return advance_impl(pool, t, n_new, d_workspace, ws_bytes, stream);
  RK_GUARD_END
}

rk_status rk_seg_tables_export(const rk_tables *t, int32_t layer, int32_t kv_head, int32_t seq, int32_t *seg_tok_begin,
                               int32_t *seg_npages, int32_t seg_cap, int32_t *n_segs, int32_t *page_ids,
                               int32_t page_cap, int32_t *n_pages) {
  if (!t) return fail(RK_ERR_INVALID_ARG, "null tables");
  if (layer < t->layer_begin || layer >= t->layer_end || kv_head < 0 || kv_head >= t->Hkv || seq < 0 ||
      seq >= t->num_seqs)
    return fail(RK_ERR_INVALID_ARG, "(layer %d, kv head %d, seq %d) outside the tables", layer, kv_head, seq);
  int64_t k = t->key(layer, kv_head, seq);
  int64_t a = t->held_off[k], b = t->held_off[k + 1];
  int32_t ns = 0;
  for (int64_t i = a; i < b; ++i) {
    bool starts = (i == a) || (t->held_logical[i] != t->held_logical[i - 1] + 1);
    if (starts) {
      if (ns < seg_cap) {
        if (seg_tok_begin) seg_tok_begin[ns] = t->held_logical[i] * t->P;
        if (seg_npages) seg_npages[ns] = 0;
      }
      ++ns;
    }
    if (ns - 1 < seg_cap && seg_npages) seg_npages[ns - 1] += 1;
    if (page_ids && i - a < page_cap) page_ids[i - a] = t->held_phys[i];
  }
  if (n_segs) *n_segs = ns;
  if (n_pages) *n_pages = (int32_t)(b - a);
  return RK_OK;
}

rk_status rk_seg_tables_schedule(const rk_tables *t, int32_t layer, int32_t *items, int64_t cap, int64_t *n_items,
                                 int32_t *tokens_per_item, int32_t *key_tile) {
  if (!t) return fail(RK_ERR_INVALID_ARG, "null tables");
  if (layer < t->layer_begin || layer >= t->layer_end) return fail(RK_ERR_INVALID_ARG, "layer outside the tables");
  const std::vector<rk::Item> &v = t->items[layer - t->layer_begin];
  if (n_items) *n_items = (int64_t)v.size();
  if (tokens_per_item) *tokens_per_item = t->T;
  if (key_tile) *key_tile = rk::kKeyTile;
  if (items)
    for (int64_t i = 0; i < std::min<int64_t>(cap, (int64_t)v.size()); ++i) {
      items[4 * i + 0] = v[i].seq;
      items[4 * i + 1] = v[i].kv_head;
      items[4 * i + 2] = v[i].tok0;
      items[4 * i + 3] = v[i].tiles;
    }
  return RK_OK;
}

rk_status rk_seg_tables_mass_schedule(const rk_tables *t, int32_t layer, int32_t *units, int64_t cap,
                                      int64_t *n_units, int32_t *keys_per_unit, int32_t *tokens_per_step,
                                      int32_t *steps_per_chunk) {
  if (!t) return fail(RK_ERR_INVALID_ARG, "null tables");
  if (layer < t->layer_begin || layer >= t->layer_end) return fail(RK_ERR_INVALID_ARG, "layer outside the tables");
  const std::vector<rk::MassUnit> &v = t->mass_units[layer - t->layer_begin];
  if (n_units) *n_units = (int64_t)v.size();
  if (keys_per_unit) *keys_per_unit = rk::mass_keys_per_unit(t->G);
  if (steps_per_chunk) *steps_per_chunk = t->mass_steps[layer - t->layer_begin];
  if (tokens_per_step) *tokens_per_step = rk::mass_tokens_per_step(t->G);
  if (units)
    for (int64_t i = 0; i < std::min<int64_t>(cap, (int64_t)v.size()); ++i) {
      units[4 * i + 0] = v[i].seq;
      units[4 * i + 1] = v[i].kv_head;
      units[4 * i + 2] = v[i].kblk;
      units[4 * i + 3] = v[i].qc;
    }
  return RK_OK;
}

rk_status rk_seg_tables_decode_schedule(const rk_tables *t, int32_t layer, int32_t *items, int64_t cap,
                                        int64_t *n_items, int32_t *comb_off, int64_t comb_cap) {
  if (!t) return fail(RK_ERR_INVALID_ARG, "null tables");
  if (layer < t->layer_begin || layer >= t->layer_end) return fail(RK_ERR_INVALID_ARG, "layer outside the tables");
  if (!t->decode_shaped) {
    if (n_items) *n_items = 0;
    return RK_OK;
  }
  const std::vector<rk::DecItem> &v = t->dec_items[layer - t->layer_begin];
  const std::vector<int32_t> &c = t->dec_comb[layer - t->layer_begin];
  if (n_items) *n_items = (int64_t)v.size();
  if (items)
    for (int64_t i = 0; i < std::min<int64_t>(cap, (int64_t)v.size()); ++i) {
      items[4 * i + 0] = v[i].seq;
      items[4 * i + 1] = v[i].kv_head;
      items[4 * i + 2] = v[i].k0;
      items[4 * i + 3] = v[i].k1;
    }
  if (comb_off)
    for (int64_t i = 0; i < std::min<int64_t>(comb_cap, (int64_t)c.size()); ++i) comb_off[i] = c[i];
  return RK_OK;
}

rk_status rk_seg_tables_stats(const rk_tables *t, rk_tables_stats *out) {
  if (!t || !out) return fail(RK_ERR_INVALID_ARG, "null tables or out");
  *out = t->stats;
  return RK_OK;
}

rk_status rk_seg_tables_trim(rk_pool *pool, rk_tables *t) {
  RK_GUARD_BEGIN
  if (!pool || !t || t->pool != pool) return fail(RK_ERR_INVALID_ARG, "null or foreign tables");
  std::vector<int64_t> off(t->held_off.size(), 0);
  std::vector<int32_t> lg, ph, freed;
  lg.reserve(t->held_logical.size());
  ph.reserve(t->held_phys.size());
  const int64_t nkeys = (int64_t)t->held_off.size() - 1;
  for (int32_t l = t->layer_begin; l < t->layer_end; ++l)
    for (int32_t g = 0; g < t->Hkv; ++g)
      for (int32_t b = 0; b < t->num_seqs; ++b) {
        int64_t k = t->key(l, g, b);
        int cls = t->head_class[(size_t)l * t->Hkv + g];
        PageRun keep[2];
        // retained state: what a query at position kv_len would see
        int nk = cls == RK_GLOBAL ? held_runs(cls, 0, t->kv_len[b], t->sink, t->window, t->P, keep)
                                  : held_runs(cls, t->kv_len[b], t->kv_len[b], t->sink, t->window, t->P, keep);
        for (int64_t i = t->held_off[k]; i < t->held_off[k + 1]; ++i) {
          int32_t p = t->held_logical[i];
          bool kept = false;
          for (int r = 0; r < nk; ++r) kept |= (p >= keep[r].p0 && p < keep[r].p1);
          if (kept) {
            lg.push_back(p);
            ph.push_back(t->held_phys[i]);
          } else {
            freed.push_back(t->held_phys[i]);
          }
        }
        off[k + 1] = (int64_t)lg.size();
      }
  (void)nkeys;
  push_free(pool, freed);
  t->held_off.swap(off);
  t->held_logical.swap(lg);
  t->held_phys.swap(ph);
  t->trimmed = true;
  t->stats.pages_held = (int64_t)t->held_phys.size();
  return RK_OK;
  RK_GUARD_END
}

rk_status rk_seg_tables_destroy(rk_pool *pool, rk_tables *t) {
  RK_GUARD_BEGIN
  if (!pool || !t || t->pool != pool) return fail(RK_ERR_INVALID_ARG, "null or foreign tables");
  rk_status st = release_device(t);
  push_free(pool, t->held_phys);
  pool->live_tables--;
  delete t;
  return st;
  RK_GUARD_END
}

rk_status rk_seg_reuse_rerotate(rk_pool *pool, const rk_tables *t, int32_t layer, int32_t seq, int32_t tok_begin,
                                int32_t n_tok, const void *src_k, const void *src_v, int64_t src_head_stride,
                                int64_t delta, double rope_base, int32_t rope_style, void *stream) {
  RK_GUARD_BEGIN
  rk_status st = check_device_tables(pool, t, layer);
  if (st != RK_OK) return st;
  if (seq < 0 || seq >= t->num_seqs) return fail(RK_ERR_INVALID_ARG, "seq %d outside [0, %d)", seq, t->num_seqs);
  if (tok_begin < 0 || n_tok < 0 || (int64_t)tok_begin + n_tok > t->kv_len[seq])
    return fail(RK_ERR_INVALID_ARG, "token range [%d, %d + %d) outside [0, kv_len %d)", tok_begin, tok_begin, n_tok,
                t->kv_len[seq]);
  if (n_tok == 0) return RK_OK;
  if (!src_k || !src_v || !aligned16(src_k) || !aligned16(src_v))
    return fail(RK_ERR_INVALID_ARG, "src_k / src_v null or not 16-byte aligned");
  const int32_t D = pool->desc.head_dim;
  if (src_head_stride < (int64_t)n_tok * D) return fail(RK_ERR_INVALID_ARG, "src_head_stride < n_tok * head_dim");
  const int64_t elem = pool->desc.dtype == RK_F32 ? 4 : 2;
  if ((src_head_stride * elem) % 16)
    return fail(RK_ERR_INVALID_ARG, "src_head_stride %lld elements is not a multiple of 16 bytes",
                (long long)src_head_stride);
  if (!(rope_base > 1.0) || !std::isfinite(rope_base)) return fail(RK_ERR_INVALID_ARG, "rope_base must be > 1");
  if (rope_style != RK_ROPE_ROTATE_HALF && rope_style != RK_ROPE_INTERLEAVED)
    return fail(RK_ERR_INVALID_ARG, "rope_style %d", rope_style);
  rk::KvWriteParams p = kv_params(pool, t, layer);
  p.k_src = src_k;
  p.v_src = src_v;
  p.src_head_stride = src_head_stride;
  p.seq = seq;
  p.tok_begin = tok_begin;
  p.n_tok = n_tok;
  p.page0 = tok_begin / t->P;
  p.delta = delta;
  p.rope_base = rope_base;
  p.rope_style = rope_style;
  for (int m = 0; m < D / 2; ++m) {  // the angle, its cos and sin in fp64, rounded to fp32
    const double a = (double)delta * std::pow(rope_base, -2.0 * (double)m / (double)D);
    p.rope_cos[m] = (float)std::cos(a);
    p.rope_sin[m] = (float)std::sin(a);
  }
  // Launch over the logical pages some head imports: pages it holds in [tok_begin, its class start) of the
  // document's range (a reused document below every LOCAL window and above the sink imports nothing, and
  // under the split a GLOBAL head imports nothing).
  int32_t lo = INT32_MAX, hi = -1;
  for (int32_t g = 0; g < t->Hkv; ++g) {
    const bool global = t->head_class[(size_t)layer * t->Hkv + g] == RK_GLOBAL;
    const int32_t end = std::min(tok_begin + n_tok, global ? t->q_begin[seq] : t->q_start[seq]);
    if (end <= tok_begin) continue;
    const int64_t k = t->key(layer, g, seq);
    const auto h0 = t->held_logical.begin() + t->held_off[k], h1 = t->held_logical.begin() + t->held_off[k + 1];
    const auto first = std::lower_bound(h0, h1, tok_begin / t->P);
    const auto last = std::upper_bound(first, h1, (end - 1) / t->P);
    if (first == last) continue;
    lo = std::min(lo, *first);
    hi = std::max(hi, *(last - 1));
  }
  if (hi < 0) return RK_OK;
  p.page0 = lo;
  const int n_pages = hi - lo + 1;
  hipError_t e = rk::launch_import(p, n_pages, pool->desc.dtype, D, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "re-rotate kernel launch");
  return RK_OK;
  RK_GUARD_END
}

rk_status rk_seg_append_kv(rk_pool *pool, const rk_tables *t, int32_t layer, const void *k_new, const void *v_new,
                           void *stream) {
  RK_GUARD_BEGIN
  rk_status st = check_device_tables(pool, t, layer);
  if (st != RK_OK) return st;
  return append_impl(pool, t, layer, k_new, v_new, stream);
  RK_GUARD_END
}

rk_status rk_seg_attn_prefill(rk_pool *pool, const rk_tables *t, int32_t layer, const void *q, const void *k_new,
                              const void *v_new, void *o, float *lse, float softmax_scale, void *stream) {
  RK_GUARD_BEGIN
  rk_status st = check_device_tables(pool, t, layer);
  if (st != RK_OK) return st;
  const int64_t total_q = t->cu_q[t->num_seqs];
  if (total_q > 0) {
    if (!q || !o || !aligned16(q) || !aligned16(o)) return fail(RK_ERR_INVALID_ARG, "q / o null or not 16-byte aligned");
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(RK_ERR_INVALID_ARG, "lse not 4-byte aligned");
  }
  if ((k_new == nullptr) != (v_new == nullptr)) return fail(RK_ERR_INVALID_ARG, "k_new and v_new must both be set or both NULL");
  if (!(softmax_scale <= 0.0f) && !std::isfinite(softmax_scale)) return fail(RK_ERR_INVALID_ARG, "softmax_scale not finite");
  if (k_new) {
    st = append_impl(pool, t, layer, k_new, v_new, stream);
    if (st != RK_OK) return st;
  }
  const int32_t li = layer - t->layer_begin;
  if (t->items[li].empty()) return RK_OK;
  const rk_tables::LayerDev &d = t->dev[li];
  rk::AttnParams p{};
  p.q = q;
  p.o = o;
  p.lse = lse;
  p.k_pages = pool->desc.k_pages;
  p.v_pages = pool->desc.v_pages;
  p.page_base = d.page_base;
  p.page_ids = d.page_ids;
  p.seqs = t->d_seqs;
  p.items = d.items;
  p.ictx = d.ictx;
  p.head_class = d.head_class;
  p.n_items = (int32_t)t->items[li].size();
  p.num_seqs = t->num_seqs;
  p.H = t->H;
  p.Hkv = t->Hkv;
  p.G = t->G;
  p.T = t->T;
  p.P = t->P;
  p.log2P = log2i(t->P);
  p.sink = t->sink;
  p.window = t->window;
  p.total_q = (int32_t)total_q;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)pool->desc.head_dim);
  p.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = rk::launch_attention(p, pool->desc.dtype, pool->desc.head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention kernel launch");
  return RK_OK;
  RK_GUARD_END
}

rk_status rk_seg_key_mass(rk_pool *pool, const rk_tables *t, int32_t layer, const void *q, const float *lse,
                          float *mass, float softmax_scale, void *stream) {
  RK_GUARD_BEGIN
  rk_status st = check_device_tables(pool, t, layer);
  if (st != RK_OK) return st;
  if (pool->desc.dtype != RK_BF16) return fail(RK_ERR_UNSUPPORTED, "per-key mass needs a bf16 pool");
  if (t->G > 16) return fail(RK_ERR_UNSUPPORTED, "per-key mass supports at most 16 q heads per KV head");
  const int64_t total_q = t->cu_q[t->num_seqs];
  int64_t total_kv = 0;
  for (int32_t b = 0; b < t->num_seqs; ++b) total_kv += t->kv_len[b];
  if (total_kv > INT32_MAX) return fail(RK_ERR_UNSUPPORTED, "more than 2^31 keys in the call");
  if (total_kv == 0) return RK_OK;
  if (!mass || (reinterpret_cast<uintptr_t>(mass) & 3u)) return fail(RK_ERR_INVALID_ARG, "mass null or not 4-byte aligned");
  if (total_q > 0 && (!q || !aligned16(q) || !lse || (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return fail(RK_ERR_INVALID_ARG, "q / lse null or misaligned");
  if (!(softmax_scale <= 0.0f) && !std::isfinite(softmax_scale)) return fail(RK_ERR_INVALID_ARG, "softmax_scale not finite");
  const rk_tables::LayerDev &d = t->dev[layer - t->layer_begin];
  rk::MassParams p{};
  p.q = q;
  p.lse = lse;
  p.mass = mass;
  p.k_pages = pool->desc.k_pages;
  p.page_base = d.page_base;
  p.page_ids = d.page_ids;
  p.seqs = t->d_seqs;
  p.head_class = d.head_class;
  p.num_seqs = t->num_seqs;
  p.H = t->H;
  p.Hkv = t->Hkv;
  p.G = t->G;
  p.T = rk::mass_tokens_per_step(t->G);
  p.P = t->P;
  p.log2P = log2i(t->P);
  p.sink = t->sink;
  p.window = t->window;
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / std::sqrt((float)pool->desc.head_dim);
  p.scale_log2 = scale * 1.4426950408889634f;
  p.total_q = (int32_t)total_q;
  p.total_kv = (int32_t)total_kv;
  const std::vector<rk::MassUnit> &units = t->mass_units[layer - t->layer_begin];
  if (units.size() > (size_t)INT32_MAX) return fail(RK_ERR_UNSUPPORTED, "per-key mass: too many work units");
  p.units = d.mass_units;
  p.n_units = (int32_t)units.size();
  p.steps_per_chunk = t->mass_steps[layer - t->layer_begin];
  hipError_t e = rk::launch_key_mass(p, pool->desc.head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "key mass kernel launch");
  return RK_OK;
  RK_GUARD_END
}

rk_status rk_seg_pack_ledger(const rk_tables *t, int32_t seq, rk_pack_ledger *out) {
  RK_GUARD_BEGIN
  if (!t || !out) return fail(RK_ERR_INVALID_ARG, "null tables or out");
  if (seq < -1 || seq >= t->num_seqs) return fail(RK_ERR_INVALID_ARG, "seq %d outside [-1, %d)", seq, t->num_seqs);
  rk_pack_ledger L{};
  const int64_t tok_bytes = 2LL * t->D * t->elem_bytes;
  for (int32_t b = (seq < 0 ? 0 : seq); b < (seq < 0 ? t->num_seqs : seq + 1); ++b)
    for (int32_t l = t->layer_begin; l < t->layer_end; ++l)
      for (int32_t g = 0; g < t->Hkv; ++g) {
        const int64_t k = t->key(l, g, b);
        const int cls = t->head_class[(size_t)l * t->Hkv + g];
        const int64_t np = t->held_off[k + 1] - t->held_off[k];
        L.pages += np;
        (cls == RK_GLOBAL ? L.pages_global : L.pages_local) += np;
        const int64_t Lb = t->kv_len[b];
        L.dense_tokens += Lb;
        // held tokens by the rule of the current state: the retained rule once trimmed
        const int64_t qs = t->trimmed ? Lb : t->q_start[b];
        int64_t n = Lb;
        if (cls == RK_LOCAL && Lb > 0) {
          const int64_t s1 = std::min<int64_t>(t->sink, Lb), w0 = std::max<int64_t>(0, qs - t->window + 1);
          n = s1 + (Lb - std::max(w0, s1));
          if (w0 >= Lb) n = s1;
        }
        L.tokens += n;
      }
  L.packed_bytes = L.pages * 2LL * t->P * t->D * t->elem_bytes;
  L.token_bytes = L.tokens * tok_bytes;
  L.dense_bytes = L.dense_tokens * tok_bytes;
  *out = L;
  return RK_OK;
  RK_GUARD_END
}

namespace {
rk_status page_copy_impl(rk_pool *pool, const rk_tables *t, int32_t seq, void *buf, size_t buf_bytes, bool pack,
                         void *stream) {
  if (!pool || !t || t->pool != pool) return fail(RK_ERR_INVALID_ARG, "null or foreign tables");
  if (!t->d_ws) return fail(RK_ERR_STATE, "tables were built on the host only (no workspace)");
  if (t->trimmed) return fail(RK_ERR_STATE, "trimmed tables have no device view; advance them by 0 tokens first");
  if (seq < -1 || seq >= t->num_seqs) return fail(RK_ERR_INVALID_ARG, "seq %d outside [-1, %d)", seq, t->num_seqs);
  const int64_t p0 = t->pack_off[seq < 0 ? 0 : seq], p1 = t->pack_off[seq < 0 ? t->num_seqs : seq + 1];
  const int64_t page_bytes = (int64_t)t->P * t->D * t->elem_bytes;
  const size_t need = (size_t)((p1 - p0) * 2 * page_bytes);
  if (pack ? buf_bytes < need : buf_bytes != need)
    return fail(RK_ERR_INVALID_ARG, "packed buffer has %zu bytes, the held pages take %zu", buf_bytes, need);
  if (p1 == p0) return RK_OK;
  if (!buf || !aligned16(buf)) return fail(RK_ERR_INVALID_ARG, "buffer null or not 16-byte aligned");
  rk::PageCopyParams p{};
  p.k_pages = pool->desc.k_pages;
  p.v_pages = pool->desc.v_pages;
  p.ids = t->d_pack_ids + p0;
  p.n = p1 - p0;
  p.buf = buf;
  p.page_bytes = page_bytes;
  hipError_t e = rk::launch_page_copy(p, pack, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "page copy launch");
  return RK_OK;
}
}  // namespace

rk_status rk_seg_pack_pages(rk_pool *pool, const rk_tables *t, int32_t seq, void *dst, size_t dst_bytes, void *stream) {
  RK_GUARD_BEGIN
  return page_copy_impl(pool, t, seq, dst, dst_bytes, true, stream);
  RK_GUARD_END
}

rk_status rk_seg_unpack_pages(rk_pool *pool, const rk_tables *t, int32_t seq, const void *src, size_t src_bytes,
                              void *stream) {
  RK_GUARD_BEGIN
  return page_copy_impl(pool, t, seq, const_cast<void *>(src), src_bytes, false, stream);
  RK_GUARD_END
}

rk_status rk_seg_attn_decode(rk_pool *pool, const rk_tables *t, int32_t layer, const void *q, const void *k_new,
                             const void *v_new, void *o, float *lse, float softmax_scale, void *stream) {
  RK_GUARD_BEGIN
  return decode_impl(pool, t, layer, q, k_new, v_new, o, lse, softmax_scale, stream, false);
  RK_GUARD_END
}

rk_status rk_seg_attn_decode_noalloc(rk_pool *pool, const rk_tables *t, int32_t layer, const void *q,
                                     const void *k_new, const void *v_new, void *o, float *lse, float softmax_scale,
                                     void *stream) {
  RK_GUARD_BEGIN
  return decode_impl(pool, t, layer, q, k_new, v_new, o, lse, softmax_scale, stream, true);
  RK_GUARD_END
}

}  // extern "C"
