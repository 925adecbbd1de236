// gfx950 (CDNA4) kernels of decode over the segmented pool: one query row per sequence, after the
// prefill call whose state the pool keeps (page "RedKnot – 小红书研发并开源的长上下文大模型推理引擎"
// (shshi.cn), section RedKnot核心特点: sessions per GPU at long context; page "小红书把 KV Cache 按
// 「头」拆了…" (zhichai.net), section 事件内容: GLOBAL heads read every context page, LOCAL heads only
// their sink and recent-window pages).
//
//  * decode_bf16<D>: one wave per split-KV item (seq, kv head, key range), kDecodeWaves waves per
//    workgroup on consecutive items of one (seq, kv head).  The G <= 16 query rows of the KV head are
//    the N = 16 columns of v_mfma_f32_16x16x32_bf16: S^T = K Q^T with keys as M, then O^T += V^T P^T
//    with channels as M, so P never leaves registers (the two 16-key halves of a 32-key tile give each
//    lane the 8 keys its B operand needs, in the order the V loads follow).  K and V come straight
//    from the pages into registers (16- and 8-byte loads off a scalar page base), one 32-key tile
//    ahead.  Online softmax in fp32.  The waves merge their (max, sum, unnormalised o) in LDS, and the
//    workgroup writes one normalised partial output and lse.
//  * decode_combine<D>: merges the partials of each query row: lse = log sum_s e^{lse_s},
//    o = sum_s e^{lse_s - lse} o_s (the split-KV combine), one workgroup per row.
//  * The new token (position kv_len - 1) of each sequence: when the caller passes it, the one item of a
//    (seq, kv head) whose range ends at kv_len writes it into its page, with the slot clearing of the
//    append kernel, and computes with it from registers; no wave reads a slot this launch writes.
// Decode reads every visible K/V byte once, so it is bound by HBM bandwidth, not by the MFMAs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "rk_device.h"
#include "rk_ops.h"
#include "rk_seg.h"

// Split-KV partials of the decode variant that allocates nothing: one array per GPU, a device global
// of the code object, shared by every such call on that GPU and holding the last call's contents.
// Host code never passes its name to a kernel (there it is a host-side stand-in): it passes the
// address that hipGetSymbolAddress returned for the device.
static __device__ __align__(256) float scratch[rk::kDecodeScratchBytes / sizeof(float)];

namespace rk {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(4))) const int32_t ConstI32;  // read-only for the kernel's lifetime

// max / sum over the four 16-lane groups (lanes c16, c16 + 16, c16 + 32, c16 + 48), with lane swaps
// (no LDS traffic)
__device__ __forceinline__ float groups_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float groups_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct DecTile {
  bf16x8 k[2][D / 32];  // A operand of S^T: keys kt + 16 h + (lane % 16), channels 32 ks + 8 (lane / 16) ..
  u32x2 va[D / 16];     // V^T rows 16 dt + lane % 16, keys kt + 4 (lane / 16) .. + 3
  u32x2 vb[D / 16];     // the same, keys kt + 16 + 4 (lane / 16) .. + 3
};

// The append of one (seq, kv head)'s new token at position j into page pg, by one wave: K row j and V
// column j, then the clearing the append kernel does, so that every slot attention may load is finite:
// the slots past kv_len = j + 1, and on a LOCAL head the slots of the page below its window and above
// the sink.  The V chunk (8 slots) holding j is read, merged and written back; it holds earlier tokens.
template <int D>
__device__ void write_new_token(const DecodeParams &p, int pg, int j, int g, const bf16_t *kr, const bf16_t *vr,
                                int lane) {
  const int P = p.P, lp = j >> p.log2P, s = j & (P - 1);
  bf16_t *kp = static_cast<bf16_t *>(const_cast<void *>(p.k_pages)) + (int64_t)pg * P * D;
  bf16_t *vp = static_cast<bf16_t *>(const_cast<void *>(p.v_pages)) + (int64_t)pg * D * P;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // K rows [s, P): row s from the source, the rest zero (16 bytes per lane and step)
  for (int c = lane; c < (P - s) * (D / 8); c += 64) {
    const int r = s + c / (D / 8), ch = c % (D / 8);
    *reinterpret_cast<u32x4 *>(kp + (int64_t)r * D + 8 * ch) =
        r == s ? *reinterpret_cast<const u32x4 *>(kr + 8 * ch) : zero;
  }
  // V channel rows, chunks of 8 slots from the one holding s: slot s from the source, later slots zero
  const int cs = s >> 3, nch = P / 8 - cs;
  for (int c = lane; c < D * nch; c += 64) {
    const int d = c / nch, k = cs + c % nch;
    bf16x8 *dst = reinterpret_cast<bf16x8 *>(vp + (int64_t)d * P + 8 * k);
    bf16x8 w = {};
    if (k == cs) {
      const bf16x8 old = *dst;
      const bf16_t v = vr[d];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = 8 * k + i < s ? old[i] : (8 * k + i == s ? v : bf16_t(0.f));
    }
    *dst = w;
  }
  // a LOCAL head: slots [max(page start, sink), kv_len - window) of the page
  if (p.head_class[g] != RK_GLOBAL) {
    const int z0 = max(lp * P, p.sink) - lp * P, z1 = min(j + 1 - p.window, j) - lp * P;
    for (int c = lane; c < max(0, z1 - z0) * D; c += 64) {
      const int r = z0 + c / D, d = c % D;
      kp[(int64_t)r * D + d] = bf16_t(0.f);
      vp[(int64_t)d * P + r] = bf16_t(0.f);
    }
  }
}

// SMALLP: 8-key pages, where a 16-key half of a tile spans two pages (each lane picks its page)
template <int D, bool SMALLP>
__global__ void __launch_bounds__(64 * kDecodeWaves) __attribute__((amdgpu_waves_per_eu(2))) decode_bf16(DecodeParams p) {
  constexpr int KS = D / 32;  // 32-channel steps of QK
  constexpr int DT = D / 16;  // 16-channel tiles of PV
  constexpr int NW = kDecodeWaves;
  // per wave: unnormalised O^T columns (query rows); a row is padded by one 16-byte chunk so that the
  // sixteen rows a store instruction writes (lanes c16) start in different banks
  __shared__ f32x4 sm_o[NW][16][D / 4 + 1];
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, c16 = lane & 15, q4 = lane >> 4;
  const DecItem it = p.items[blockIdx.x * NW + wave];
  const int b = it.seq, g = it.kv_head, k0 = it.k0, k1 = it.k1;
  const SeqInfo si = p.seqs[b];
  const int L = si.kv_len, P = p.P, G = p.G;
  // the page table through the constant address space: the kernel never writes it, and so its
  // uniform lookups compile to scalar loads (a vector load here would make the tile loop wait on
  // vmcnt(0), i.e. on the next tile's prefetch, before every tile)
  const ConstI32 *pt = (const ConstI32 *)(p.page_ids + p.page_base[g * p.num_seqs + b]);
  // a key past kv_len or on a page the head does not hold reads the page of k0 (held) and is masked
  const int pg0 = pt[k0 >> p.log2P];
  auto page_of = [&](int key) {  // uniform: a scalar load of the page table
    const int pg = pt[min(key, L - 1) >> p.log2P];
    return key < L && pg >= 0 ? pg : pg0;
  };
  // page ids of a tile's two 16-key halves (with 8-key pages: of its four 8-key quarters), looked up
  // two tiles before its loads are issued
  struct Pages {
    int a, b, a1, b1;
  };
  auto pages_of = [&](int kt) {
    if constexpr (SMALLP) return Pages{page_of(kt), page_of(kt + 16), page_of(kt + 8), page_of(kt + 24)};
    else return Pages{page_of(kt), page_of(kt + 16), 0, 0};
  };

  // Q as the B operand of S^T: lane holds channels 32 ks + 8 q4 .. + 7 of row c16 (q head g G + c16)
  bf16x8 qf[KS];
  {
    const bool ok = c16 < G;
    const bf16_t *qrow = static_cast<const bf16_t *>(p.q) + ((int64_t)si.cu_q * p.H + g * G + (ok ? c16 : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 z = {};
      qf[ks] = ok ? *reinterpret_cast<const bf16x8 *>(qrow + 32 * ks + 8 * q4) : z;
    }
  }

  // the call's new token, when this item owns it: kn (K channels 32 ks + 8 q4 .. + 7) and vn (V channel
  // 16 dt + c16) patch its key in the last tile; the page gets the row and the append's clearing
  const int jn = L - 1;
  const bool own_new = p.k_src != nullptr && k1 == L && k1 > k0;  // uniform
  bf16x8 kn[KS];
  bf16_t vn[DT];
  if (own_new) {
    const int64_t row = ((int64_t)si.cu_q * p.Hkv + g) * D;
    const bf16_t *kr = static_cast<const bf16_t *>(p.k_src) + row;
    const bf16_t *vr = static_cast<const bf16_t *>(p.v_src) + row;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kn[ks] = *reinterpret_cast<const bf16x8 *>(kr + 32 * ks + 8 * q4);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vn[dt] = vr[16 * dt + c16];
    write_new_token<D>(p, pt[jn >> p.log2P], jn, g, kr, vr, lane);
  }

  const char *kbytes = static_cast<const char *>(p.k_pages);
  const char *vbytes = static_cast<const char *>(p.v_pages);
  const uint32_t k_lane = (uint32_t)((c16 * D + 8 * q4) * 2);  // bytes within a 16-key block of a K page
  const uint32_t v_lane = (uint32_t)((c16 * P + 4 * q4) * 2);  // bytes within a 16-channel block of a V page
  auto load = [&](int kt, Pages pg, DecTile<D> &T) {  // pg: uniform; a == b when P >= 32
    if constexpr (SMALLP) {
      // K row c16 of a half: key 16 h + c16, page a / a1 (b / b1) by c16 < 8; V run 4 q4 .. + 3: page
      // by q4 < 2, slot (4 q4) % 8.  Per-lane 64-bit addresses.
      const int64_t ra = c16 < 8 ? pg.a : pg.a1, rb = c16 < 8 ? pg.b : pg.b1;
      const char *ka = kbytes + ((ra * 8 + (c16 & 7)) * D + 8 * q4) * 2;
      const char *kb = kbytes + ((rb * 8 + (c16 & 7)) * D + 8 * q4) * 2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        T.k[0][ks] = *reinterpret_cast<const bf16x8 *>(ka + 64 * ks);
        T.k[1][ks] = *reinterpret_cast<const bf16x8 *>(kb + 64 * ks);
      }
      const int64_t qa = q4 < 2 ? pg.a : pg.a1, qb = q4 < 2 ? pg.b : pg.b1;
      const char *va = vbytes + (qa * D * 8 + c16 * 8 + ((4 * q4) & 7)) * 2;
      const char *vb = vbytes + (qb * D * 8 + c16 * 8 + ((4 * q4) & 7)) * 2;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        T.va[dt] = *reinterpret_cast<const u32x2 *>(va + dt * 16 * 8 * 2);
        T.vb[dt] = *reinterpret_cast<const u32x2 *>(vb + dt * 16 * 8 * 2);
      }
      return;
    }
    const int sa = kt & (P - 1), sb = (kt + 16) & (P - 1);
    const char *ka = kbytes + ((int64_t)pg.a * P + sa) * D * 2;
    const char *kb = kbytes + ((int64_t)pg.b * P + sb) * D * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      T.k[0][ks] = *reinterpret_cast<const bf16x8 *>(ka + 64 * ks + opaque(k_lane));
      T.k[1][ks] = *reinterpret_cast<const bf16x8 *>(kb + 64 * ks + opaque(k_lane));
    }
    const char *va = vbytes + ((int64_t)pg.a * D * P + sa) * 2;
    const char *vb = vbytes + ((int64_t)pg.b * D * P + sb) * 2;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int64_t row = (int64_t)dt * 16 * P * 2;  // uniform: the dt-th 16-channel block
      T.va[dt] = *reinterpret_cast<const u32x2 *>(va + row + opaque(v_lane));
      T.vb[dt] = *reinterpret_cast<const u32x2 *>(vb + row + opaque(v_lane));
    }
  };

  const float c2 = p.scale_log2;
  float m = -INFINITY, l = 0.f;  // running max (log2 units) and this lane's part of the row sum
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the owner's last tile: key jn from registers, keys past it zero in V (their slots may hold anything
  // in this launch; a masked key weighs 0, and 0 times a non-finite value would not be 0)
  auto patch = [&](int kt, DecTile<D> &T) {
    const bool krow = c16 == (jn & 15);  // the lane holding K row jn (in half (jn - kt) / 16)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {  // static indices only: the tile stays in registers
      const bool mine = krow && hh == ((jn - kt) >> 4);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) T.k[hh][ks] = mine ? kn[ks] : T.k[hh][ks];
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x4 r = __builtin_bit_cast(bf16x4, hh ? T.vb[dt] : T.va[dt]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kt + 16 * hh + 4 * q4 + i;
          r[i] = key == jn ? vn[dt] : (key > jn ? bf16_t(0.f) : r[i]);
        }
        if (hh) T.vb[dt] = __builtin_bit_cast(u32x2, r);
        else T.va[dt] = __builtin_bit_cast(u32x2, r);
      }
  };

  auto compute = [&](int kt, DecTile<D> &T) {
    if (own_new && kt == (jn & ~31)) patch(kt, T);
    f32x4 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(T.k[h][ks], qf[ks], s[h], 0, 0, 0);
    }
    // lane holds keys kt + 16 h + 4 q4 + i of row c16; keys outside [k0, k1) are masked (the mask
    // depends on the key only, and every tile holds an unmasked key)
    float x[8];
    float mt = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kt + 16 * h + 4 * q4 + i;
        const float v = (key >= k0 && key < k1) ? s[h][i] * c2 : -INFINITY;
        x[4 * h + i] = v;
        mt = fmaxf(mt, v);
      }
    mt = groups_max(mt);
    const float mn = fmaxf(m, mt);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    f32x8 pw;
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pw[e] = fast_exp2(x[e] - mn);
      ps += pw[e];
    }
    l = l * alpha + ps;
    const bf16x8 pb = __builtin_convertvector(pw, bf16x8);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] *= alpha;
      const u32x4 a = {T.va[dt][0], T.va[dt][1], T.vb[dt][0], T.vb[dt][1]};
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pb, o[dt], 0, 0, 0);
    }
  };

  // tile t + 1's loads are issued before tile t is computed; page ids are looked up two tiles before
  // their loads.  The steady-state loop issues both of its loads on every pass (tiles t + 1 and
  // t + 2 exist), so every path into a tile's first use has the same loads outstanding and the
  // compiler's wait counts leave the next tile in flight; the last one or two tiles are peeled.
  const int t0 = k0 & ~31;
  const int ntiles = k1 > k0 ? ((k1 - 1 - t0) >> 5) + 1 : 0;  // a padding item has no keys
  if (ntiles > 0) {
    DecTile<D> buf[2];
    Pages pn = pages_of(t0), pn2 = pages_of(t0 + 32);
    load(t0, pn, buf[0]);
    pn = pn2;
    pn2 = pages_of(t0 + 64);
    int t = 0;
    for (; t + 2 < ntiles; t += 2) {
      load(t0 + 32 * (t + 1), pn, buf[1]);
      pn = pn2;
      pn2 = pages_of(t0 + 32 * (t + 3));
      compute(t0 + 32 * t, buf[0]);
      load(t0 + 32 * (t + 2), pn, buf[0]);
      pn = pn2;
      pn2 = pages_of(t0 + 32 * (t + 4));
      compute(t0 + 32 * (t + 1), buf[1]);
    }
    if (t + 1 < ntiles) {
      load(t0 + 32 * (t + 1), pn, buf[1]);
      compute(t0 + 32 * t, buf[0]);
      compute(t0 + 32 * (t + 1), buf[1]);
    } else {
      compute(t0 + 32 * t, buf[0]);
    }
  }

  // row sum over the four lane groups; the wave's (max, sum, unnormalised o) of each query row to LDS
  // (a padding item: max -inf, sum 0, o 0)
  l = groups_sum(l);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) sm_o[wave][c16][4 * dt + q4] = o[dt];
  if (q4 == 0) {
    sm_m[wave][c16] = m;
    sm_l[wave][c16] = l;
  }
  __syncthreads();
  // merge: thread (row r, channel quarter-group cq) combines the waves' parts of row r
  constexpr int CPT = D / 64;  // f32x4 chunks per thread: 16 rows x 16 threads cover [16][D / 4]
  const int r = threadIdx.x >> 4, cq = threadIdx.x & 15;
  if (r < G) {
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm_m[w][r]);
    float a[NW], tot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      a[w] = sm_m[w][r] == -INFINITY ? 0.f : fast_exp2(sm_m[w][r] - mx);
      tot += a[w] * sm_l[w][r];
    }
    const float inv = 1.0f / tot;
    float *po = p.part_o + ((int64_t)blockIdx.x * G + r) * D;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c4 = cq + 16 * j;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w) acc += a[w] * sm_o[w][r][c4];
      *reinterpret_cast<f32x4 *>(po + 4 * c4) = acc * inv;
    }
    if (cq == 0) p.part_lse[(int64_t)blockIdx.x * G + r] = (mx + __log2f(tot)) * 0.6931471805599453f;
  }
}

// One workgroup per query row (seq, q head): lse = log sum_s e^{lse_s} and o = sum_s e^{lse_s - lse} o_s
// over the row's partials s, in one pass.  The partials are spread over NG groups of D / 4 threads
// (each thread four channels); a group keeps a running (max m, weight sum w = sum e^{lse_s - m}, acc =
// sum e^{lse_s - m} o_s), rescaled when m grows, with U partial loads in flight per thread (the combine
// of a long GLOBAL head is latency-bound otherwise).  The groups are merged through LDS at the end.
template <int D>
__global__ void __launch_bounds__(256) decode_combine(DecodeParams p) {
  constexpr int TPG = D / 4;         // threads per group: one 16-byte chunk of a partial each
  constexpr int NG = 256 / TPG;      // groups
  constexpr int U = 8;               // partials in flight per thread
  __shared__ float sm_m[NG], sm_w[NG];
  __shared__ f32x4 part[NG][TPG];
  const int tid = threadIdx.x;
  const int G = p.G;
  const int bg = blockIdx.x / G, r = blockIdx.x - bg * G;
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  // the row's partial slots: one per workgroup of kDecodeWaves items
  const int s0 = p.comb_off[bg] / kDecodeWaves, s1 = p.comb_off[bg + 1] / kDecodeWaves;
  if (s0 == s1) return;  // the sequence has no query row
  const SeqInfo si = p.seqs[b];
  const int grp = tid / TPG, d4 = tid - grp * TPG;
  float m = -INFINITY, w = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = s0 + grp; s < s1; s += NG * U) {
    f32x4 v[U];
    float l[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int su = min(s + NG * u, s1 - 1);  // past the row's last partial: reloaded, weight 0
      v[u] = *reinterpret_cast<const f32x4 *>(p.part_o + ((int64_t)su * G + r) * D + 4 * d4);
      l[u] = s + NG * u < s1 ? p.part_lse[(int64_t)su * G + r] : -INFINITY;
    }
    float mu = m;
#pragma unroll
    for (int u = 0; u < U; ++u) mu = fmaxf(mu, l[u]);
    const float sc = m == -INFINITY ? 0.f : expf(m - mu);  // mu is finite: the first pass has a partial
    acc *= sc;
    w *= sc;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float e = l[u] == -INFINITY ? 0.f : expf(l[u] - mu);
      acc += e * v[u];
      w += e;
    }
    m = mu;
  }
  if (d4 == 0) {
    sm_m[grp] = m;
    sm_w[grp] = w;
  }
  part[grp][d4] = acc;
  __syncthreads();
  if (grp == 0) {
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NG; ++j) mx = fmaxf(mx, sm_m[j]);
    float tot = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const float e = sm_m[j] == -INFINITY ? 0.f : expf(sm_m[j] - mx);  // a group with no partial: 0
      tot += e * sm_w[j];
      o += e * part[j][d4];
    }
    o *= 1.0f / tot;
    const int64_t row = (int64_t)si.cu_q * p.H + g * G + r;
    *reinterpret_cast<bf16x4 *>(static_cast<bf16_t *>(p.o) + row * D + 4 * d4) = __builtin_convertvector(o, bf16x4);
    if (d4 == 0 && p.lse) p.lse[(int64_t)(g * G + r) * p.total_q + si.cu_q] = mx + logf(tot);
  }
}

}  // namespace

hipError_t decode_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // once per device, with that device current
    void *a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams &p, int head_dim, hipStream_t stream) {
  if (p.n_items <= 0) return hipSuccess;
  if (p.n_items % kDecodeWaves) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.n_items / kDecodeWaves)), comb((unsigned)(p.num_seqs * p.Hkv * p.G));
  const dim3 block(64 * kDecodeWaves);
  if (head_dim == 128) {
    if (p.P < 16) hipLaunchKernelGGL((decode_bf16<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((decode_bf16<128, false>), grid, block, 0, stream, p);
    hipLaunchKernelGGL(decode_combine<128>, comb, dim3(256), 0, stream, p);
  } else {
    if (p.P < 16) hipLaunchKernelGGL((decode_bf16<64, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((decode_bf16<64, false>), grid, block, 0, stream, p);
    hipLaunchKernelGGL(decode_combine<64>, comb, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace rk
