// gfx950 (CDNA4) kernels of the SegPagedAttention prefill library.
//
//  * attn_bf16<D>: mask-free head-ragged paged prefill attention.  Global heads attend over every
//    context page, local heads over their sink and recent-window pages (page "为什么长上下文推理这么
//    慢？RedKnot如何用1个百分点的质量代价换来2–5倍TTFT加速" (bjdmk.com.cn), section 二 ③); no mask
//    tensor exists anywhere: visibility comes from token indices (page "RedKnot - Xiaohongshuが開発
//    した…" (aiboss88.com), section 技術原則, fourth item).
//  * attn_f32<D>: the same computation for fp32 storage, on the vector ALUs.
//  * kv_write<...>: writes token rows into held pages, either the new tokens of the call (the online
//    KV write of EXECUTE, aiboss88.com section 使い方) or a reused document whose keys are rotated from
//    their offline to their actual position (page "RedKnot – 小红书研发并开源的长上下文大模型推理引擎"
//    (shshi.cn), section RedKnot技术原理, 2. 位置无关缓存复用).
//
// Design of attn_bf16 (one work item = 256 query rows = G heads x T tokens of one KV head; 4 waves;
// each wave owns 64 rows as two 32-column blocks):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: keys are the M dimension, queries the N dimension, so
//    each lane holds one query column and 16 keys per 32x32 block; a row max is 15 in-lane max ops
//    plus one swap between the two half-waves.
//  * K rows are written to LDS in a permuted order (bits 2 and 3 of the key index swapped) so that
//    the S^T accumulator register i of lane half h holds key 16*(i/8) + 8*h + i%8: the eight
//    probabilities a lane needs as the B operand of the PV product (O^T = V^T P^T) for 16-key chunk
//    c are exactly its registers 8c..8c+7, converted to bf16 in place -- no shuffles.
//  * V pages are stored channel-major ([D][P]) so the A operand of PV (8 consecutive keys of one
//    channel) is one 16-byte LDS read.  LDS rows are padded by 16 bytes to spread 16-byte reads
//    over all banks.
//  * K/V tiles of 64 keys are double-buffered in LDS; the next tile's global loads are issued
//    before the current tile's MFMA work and written to LDS after it (one barrier per tile).
//  * Online softmax in fp32 with exp2; the running max is only raised when a new score exceeds
//    it by more than 2^8 in the exp2 domain, so the O rescale (64 VALU ops per block) is rare.
//    Skipping it is exact: weights up to 2^8 are represented the same way in fp32 and bf16.
//  * Per-wave tile classes from indices: skip (no key visible to any row of the wave), full (every
//    key visible to every row: no per-element work) or edge (per-element index compare).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rk_internal.h"
#include "rk_seg.h"

namespace rk {
namespace {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BN = kKeyTile;
constexpr float kNegBig = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;  // log2 of the largest un-normalised weight allowed

__device__ __forceinline__ int swap_bits23(int j) { return (j & ~0xC) | ((j & 4) << 1) | ((j & 8) >> 1); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Keep the first n (0..8) bf16 elements of a 16-byte chunk, zero the rest.
__device__ __forceinline__ u32x4 keep_first_bf16(u32x4 v, int n) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t x = v[w];
    if (2 * w + 1 >= n) x &= 0x0000FFFFu;
    if (2 * w >= n) x = 0u;
    v[w] = x;
  }
  return v;
}

__device__ __forceinline__ bool visible(int cls, int i, int j, int sink, int window) {
  return j <= i && (cls == RK_GLOBAL || j < sink || j > i - window);
}

// ------------------------------------------------------------------------------------------------
// bf16 attention
// ------------------------------------------------------------------------------------------------

#ifndef RK_ATTN_NB
#define RK_ATTN_NB 1
#endif

// LDS image of one 64-key tile, filled by direct global->LDS 16-byte loads (lane l of a load
// writes bytes [16 l, 16 l + 16) of a 1 KB block, so every block is dense: rows cannot be padded
// and bank conflicts are avoided by choosing, per lane, which 16-byte chunk of the row it fetches).
//  K: 64 rows of D channels in MFMA row order (key index with bits 2 and 3 swapped); chunk c of
//     row r sits in slot c ^ kswz(r).
//  V: per page-in-tile block [D][Pt] (Pt = min(P, 64)); chunk c of channel row d sits in slot
//     c ^ vswz(d).
// Both swizzles make 16 consecutive lanes reading 16 consecutive rows at one chunk index touch 16
// distinct 16-byte slots of every 256-byte bank window.
template <int D>
struct AttnBf16Smem {
  bf16_t k[2][BN * D];  // double buffer: the next tile loads while this one is used
  bf16_t v[2][D * BN];
};

template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
__device__ __forceinline__ int vswz(int d, int Pt) {
  return (d / (128 / Pt)) & (Pt / 8 - 1);
}

// max / sum of a value over the two half-waves (lanes l and l ^ 32)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void load_lds16(const void *gsrc, void *lds_block) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)gsrc,
                                   (__attribute__((address_space(3))) void *)lds_block, 16, 0, 0);
}

// NB = 32-query column blocks per wave.  Every 16-byte K or V fragment read from LDS feeds NB
// MFMAs, so LDS read traffic per flop falls as 1/NB; registers grow with NB (NB = 2 runs one wave
// per SIMD).
template <int D, int NB>
__global__ void __launch_bounds__(kRowsPerItem / NB * 2, 1) attn_bf16(AttnParams p) {
  constexpr int NWAVES = kRowsPerItem / (32 * NB);
  constexpr int NC = D / 16;                 // 16-channel chunks of the QK product
  constexpr int ND = D / 32;                 // 32-channel blocks of O^T
  constexpr int UNITS = BN * D * 2 / 1024;   // 1 KB load blocks per tile, for K and for V each
  constexpr int NU = UNITS / NWAVES;         // per wave
  constexpr int KROWS_U = 512 / D;           // K rows per block
  static_assert(NU >= 1 && UNITS % NWAVES == 0, "tile does not split over the waves");
  __shared__ __attribute__((aligned(1024))) AttnBf16Smem<D> sm;

  const int tid = threadIdx.x;
  // the wave index is uniform: keep it (and everything derived from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, m = lane & 31;
  const Item it = p.items[blockIdx.x];
  if (it.seq < 0) return;  // schedule padding: keeps the next items on their XCD
  const SeqInfo si = p.seqs[it.seq];
  const int g = it.kv_head;
  const int cls = p.head_class[g];
  const int tok_end = min(it.tok0 + p.T, si.n_q);
  const int L = si.kv_len;
  const int i_max = si.q_start + tok_end - 1;
  const TileRange tr = tile_range(cls, si.q_start + it.tok0, i_max, p.sink, p.window);
  const int ntiles = tr.count();
  const int32_t *__restrict__ pt = p.page_ids + p.page_base[g * p.num_seqs + it.seq];
  const bf16_t *__restrict__ kpg = static_cast<const bf16_t *>(p.k_pages);
  const bf16_t *__restrict__ vpg = static_cast<const bf16_t *>(p.v_pages);
  const int P = p.P, log2P = p.log2P;
  const int Pt = P < BN ? P : BN;
  const int n_logical = (L + P - 1) >> log2P;
  const int64_t page_elems = (int64_t)P * D;
  // Pages a tile touches but the head does not hold (or past the sequence's last page) are read
  // from this page instead: the page of the item's last query, held and fully written (the append
  // clears its slots past kv_len).  Its keys are masked out, so only finiteness matters.
  const int pg_fallback = pt[i_max >> log2P];

  // ---- the NB query rows (columns of S^T) this lane owns
  int pos[NB], tq[NB], hq[NB], win_lo[NB];
  bool valid[NB];
  int vmin = INT32_MAX, vmax = -1;
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int r = wave * 32 * NB + 32 * n + m;
    const int hh = r / p.T;
    tq[n] = it.tok0 + (r - hh * p.T);
    valid[n] = hh < p.G && tq[n] < tok_end;
    pos[n] = valid[n] ? si.q_start + tq[n] : -1;
    hq[n] = g * p.G + hh;
    win_lo[n] = cls == RK_GLOBAL ? 0 : pos[n] - p.window + 1;  // first window key of the row
    vmin = min(vmin, valid[n] ? pos[n] : INT32_MAX);
    vmax = max(vmax, pos[n]);
  }
  // wave-uniform query range: scalar registers, so tile classes are scalar branches
  const int wmin = __builtin_amdgcn_readfirstlane(wave_min(vmin));
  const int wmax = __builtin_amdgcn_readfirstlane(wave_max(vmax));

  bf16x8 qf[NB][NC];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const bf16_t *qrow = static_cast<const bf16_t *>(p.q) + ((int64_t)(si.cu_q + tq[n]) * p.H + hq[n]) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 z = {};
      qf[n][c] = valid[n] ? *reinterpret_cast<const bf16x8 *>(qrow + 16 * c + 8 * hl) : z;
    }
  }

  // ---- tile-invariant geometry of this wave's 1 KB load blocks (block b = wave * NU + u)
  int k_key0[NU], k_loff[NU];      // K: first key of the block (uniform); lane's element offset in its page
  int v_pi[NU], v_loff[NU];        // V: page-in-tile (uniform); lane's element offset in its page
  // a D = 64 K block spans 8 keys; with 8-key pages its two 4-key halves come from two pages
  const bool k_split = D == 64 && P < 16;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int b = wave * NU + u;
    // K: LDS rows b*KROWS_U + lane/(D/8), slot lane % (D/8)
    const int row = b * KROWS_U + lane / (D / 8);
    const int slot = lane % (D / 8);
    const int key = swap_bits23(row);
    const int chunk = slot ^ kswz<D>(row);
    k_key0[u] = swap_bits23(b * KROWS_U) & ~(KROWS_U - 1);
    // pages of up to 64 keys: the tile starts on a page boundary; larger pages: + tile offset per tile
    k_loff[u] = (P <= BN ? (key & (P - 1)) : key) * D + chunk * 8;
    // V: block b of the [page][D][Pt] image
    const int upp = D * Pt * 2 / 1024;  // blocks per page-in-tile image (>= 1 for Pt >= 8 with D >= 64)
    const int pi = b / upp;
    const int rows_u = 512 / Pt;        // channel rows per block
    const int d = (b % upp) * rows_u + lane / (Pt / 8);
    const int cl = lane % (Pt / 8);
    const int cg = cl ^ vswz(d, Pt);
    v_pi[u] = pi;
    v_loff[u] = d * P + cg * 8;         // + (j0 & (P - 1)) when P > 64
  }
  // V^T read offsets (elements) for the four (kb, cc) key chunks of a 64-key tile, channel row m
  int v_rd[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int k8 = 2 * q4 + hl;  // 8-key chunk 4kb + 2cc + hl
    const int cpr = Pt / 8;
    v_rd[q4] = (k8 / cpr) * D * Pt + m * Pt + (((k8 % cpr) ^ vswz(m, Pt)) << 3);
  }
  // K read offsets (elements) for the NC channel chunks, rows m (+32 for the second key block)
  int k_rd[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) k_rd[c] = m * D + (((2 * c + hl) ^ kswz<D>(m)) << 3);

  // Page ids of a tile: one vector load per wave (lane i < 64 / P holds the id of the tile's i-th
  // page), issued a tile ahead and read back with readlane, so the lookup latency stays off the
  // critical path and no scalar load shares the LDS wait counter with the operand reads.
  const int npt = P < BN ? BN / P : 1;
  auto load_ids = [&](int tile) -> int {
    const int lp = ((tile * BN) >> log2P) + lane;
    int v = -1;
    if (lane < npt && lp < n_logical) v = pt[lp];
    return v;
  };
  auto fix = [&](int pg) { return pg >= 0 ? pg : pg_fallback; };
  auto issue_tile = [&](int tile, int buf, int ids) {
    const int j0 = tile * BN;
    int pgk[NU], pgv[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      pgk[u] = fix(__builtin_amdgcn_readlane(ids, P < BN ? (k_key0[u] >> log2P) : 0));
      pgv[u] = fix(__builtin_amdgcn_readlane(ids, v_pi[u]));
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int b = wave * NU + u;
      int pk_ = pgk[u];
      if (k_split) pk_ = fix(__shfl(ids, swap_bits23(b * KROWS_U + lane / (D / 8)) >> log2P));  // lane's own page
      const int ko = P > BN ? (j0 & (P - 1)) * D : 0;
      load_lds16(kpg + (int64_t)pk_ * page_elems + k_loff[u] + ko, &sm.k[buf][b * 512]);
      const int vo = P > BN ? (j0 & (P - 1)) : 0;
      load_lds16(vpg + (int64_t)pgv[u] * page_elems + v_loff[u] + vo, &sm.v[buf][b * 512]);
    }
  };

  f32x16 oacc[NB][ND];
  float mrun[NB], lsum[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
#pragma unroll
    for (int db = 0; db < ND; ++db) oacc[n][db] = f32x16{};
    mrun[n] = kNegBig;
    lsum[n] = 0.f;
  }
  const float c2 = p.scale_log2;

  // Loads retire in issue order.  Order per step: data of the next tile, then the page ids of the
  // tile after it; at the end of the step the next tile's data must be in LDS and only the id load
  // (when one was issued) may still be in flight.
  constexpr int WAIT_ALL = 0x0f70;      // vmcnt(0)
  constexpr int WAIT_BUT_ONE = 0x0f71;  // vmcnt(1)
  int ids = load_ids(tr.tile(0));
  issue_tile(tr.tile(0), 0, ids);
  bool ids_pending = ntiles > 1;
  if (ids_pending) ids = load_ids(tr.tile(1));
  if (ids_pending) __builtin_amdgcn_s_waitcnt(WAIT_BUT_ONE);
  else __builtin_amdgcn_s_waitcnt(WAIT_ALL);
  __syncthreads();

  int buf = 0;
  for (int idx = 0; idx < ntiles; ++idx) {
    const bool more = idx + 1 < ntiles;
    ids_pending = false;
    if (more) {
      issue_tile(tr.tile(idx + 1), buf ^ 1, ids);
      ids_pending = idx + 2 < ntiles;
      if (ids_pending) ids = load_ids(tr.tile(idx + 2));
    }
    const int j0 = tr.tile(idx) * BN;
    const bool skip = wmax < 0 || j0 > wmax ||
                      (cls == RK_LOCAL && j0 >= p.sink && j0 + BN - 1 <= wmin - p.window);
    const bool full = j0 + BN - 1 <= wmin &&
                      (cls == RK_GLOBAL || j0 + BN <= p.sink || j0 > wmax - p.window);
    if (!skip) {
      const bf16_t *Kb = sm.k[buf];
      const bf16_t *Vb = sm.v[buf];
      // S^T for the tile's 64 keys (two 32-key blocks) x this wave's NB x 32 queries
      f32x16 s[NB][2];
#pragma unroll
      for (int n = 0; n < NB; ++n) s[n][0] = s[n][1] = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Kb + k_rd[c] + 32 * kb * D);
#pragma unroll
          for (int n = 0; n < NB; ++n) s[n][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[n][c], s[n][kb], 0, 0, 0);
        }
      bf16x8 pk[NB][2][2];
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        if (!full) {
          // key of register i of block kb: jb + 16 * (i / 8) + i % 8, jb = j0 + 32 kb + 8 hl
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const int jb = j0 + 32 * kb + 8 * hl;
            const int hi = pos[n] - jb;     // visible: off <= hi
            const int lo = win_lo[n] - jb;  // local: off >= lo, or off < sk
            const int sk = p.sink - jb;
            if (cls == RK_GLOBAL) {
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int off = 16 * (i >> 3) + (i & 7);
                s[n][kb][i] = off <= hi ? s[n][kb][i] : -INFINITY;
              }
            } else {
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int off = 16 * (i >> 3) + (i & 7);
                s[n][kb][i] = (off <= hi && (off >= lo || off < sk)) ? s[n][kb][i] : -INFINITY;
              }
            }
          }
        }
        float mt = s[n][0][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[n][0][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[n][1][i]);
        mt = halves_max(mt);
        const float mts = mt * c2;
        if (__any(mts > mrun[n] + kRescaleSlack)) {
          const float mnew = fmaxf(mrun[n], mts);
          const float alpha = fast_exp2(mrun[n] - mnew);
#pragma unroll
          for (int db = 0; db < ND; ++db) oacc[n][db] *= alpha;
          lsum[n] *= alpha;
          mrun[n] = mnew;
        }
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x8 e0, e1;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            e0[i] = fast_exp2(fmaf(s[n][kb][i], c2, -mrun[n]));
            e1[i] = fast_exp2(fmaf(s[n][kb][i + 8], c2, -mrun[n]));
            ps += e0[i] + e1[i];
          }
          pk[n][kb][0] = __builtin_convertvector(e0, bf16x8);
          pk[n][kb][1] = __builtin_convertvector(e1, bf16x8);
        }
        lsum[n] += ps;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int db = 0; db < ND; ++db) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Vb + v_rd[2 * kb + cc] + 32 * db * Pt);
#pragma unroll
            for (int n = 0; n < NB; ++n)
              oacc[n][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[n][kb][cc], oacc[n][db], 0, 0, 0);
          }
    }
    if (ids_pending) __builtin_amdgcn_s_waitcnt(WAIT_BUT_ONE);
    else __builtin_amdgcn_s_waitcnt(WAIT_ALL);
    __syncthreads();
    buf ^= 1;
  }

  // ---- epilogue: O^T accumulator (lane column = query, 16 channels per 32-channel block)
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const float lt = halves_sum(lsum[n]);
    if (!valid[n]) continue;
    const float inv = 1.0f / lt;
    bf16_t *orow = static_cast<bf16_t *>(p.o) + ((int64_t)(si.cu_q + tq[n]) * p.H + hq[n]) * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 w = {oacc[n][db][4 * a4 + 0] * inv, oacc[n][db][4 * a4 + 1] * inv, oacc[n][db][4 * a4 + 2] * inv,
                   oacc[n][db][4 * a4 + 3] * inv};
        *reinterpret_cast<bf16x4 *>(orow + 32 * db + 8 * a4 + 4 * hl) = __builtin_convertvector(w, bf16x4);
      }
    if (p.lse && hl == 0)
      p.lse[(int64_t)hq[n] * p.total_q + si.cu_q + tq[n]] = (mrun[n] + log2f(lt)) * 0.69314718055994531f;
  }
}

// ------------------------------------------------------------------------------------------------
// bf16 attention, ping-pong: two groups of four waves (one wave of each group per SIMD) run the same
// per-half-tile work shifted by half a tile, so that while one wave of a SIMD runs its softmax on
// the vector ALUs the other keeps the matrix cores busy.  With both groups in step (one barrier per
// tile), the two waves of a SIMD would run their MFMA phases together and then their softmax phases
// together.
//   group A, tile t:  QK(h0) | softmax(h0) | QK(h1) + PV(h0) | softmax(h1) | PV(h1)
//   group B, tile t:  softmax(t-1, h1) | PV(t-1, h1) + QK(h0) | softmax(h0) | QK(h1) + PV(h0)
// (h0, h1 = keys 0-31 and 32-63 of the tile).  Group B finishes a tile's second half in the next
// iteration, so tiles stay in LDS for one iteration longer: four stages.
// ------------------------------------------------------------------------------------------------

template <int D>
struct AttnPPSmem {
  static constexpr int NSTAGE = 4;
  bf16_t k[NSTAGE][BN * D];
  bf16_t v[NSTAGE][D * BN];
};

#ifndef RK_PP_GROUP_SHIFT
#define RK_PP_GROUP_SHIFT 2  // group = wave >> 2: waves w and w + 4 share a SIMD
#endif

template <int D>
__global__ void __launch_bounds__(512, 1) attn_bf16_pp(AttnParams p) {
  constexpr int NWAVES = 8;
  constexpr int NC = D / 16;
  constexpr int ND = D / 32;
  constexpr int UNITS = BN * D * 2 / 1024;
  constexpr int NU = UNITS / NWAVES;
  constexpr int KROWS_U = 512 / D;
  static_assert(NU >= 1 && UNITS % NWAVES == 0, "tile does not split over the waves");
  __shared__ __attribute__((aligned(1024))) AttnPPSmem<D> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = RK_PP_GROUP_SHIFT == 2 ? (wave >> 2) : (wave & 1);
  const int lane = tid & 63, hl = lane >> 5, m = lane & 31;
  const Item it = p.items[blockIdx.x];
  if (it.seq < 0) return;  // schedule padding: keeps the next items on their XCD
  const SeqInfo si = p.seqs[it.seq];
  const int g = it.kv_head;
  const int cls = p.head_class[g];
  const int tok_end = min(it.tok0 + p.T, si.n_q);
  const int L = si.kv_len;
  const int i_max = si.q_start + tok_end - 1;
  const TileRange tr = tile_range(cls, si.q_start + it.tok0, i_max, p.sink, p.window);
  const int ntiles = tr.count();
  const int32_t *__restrict__ pt = p.page_ids + p.page_base[g * p.num_seqs + it.seq];
  const bf16_t *__restrict__ kpg = static_cast<const bf16_t *>(p.k_pages);
  const bf16_t *__restrict__ vpg = static_cast<const bf16_t *>(p.v_pages);
  const int P = p.P, log2P = p.log2P;
  const int Pt = P < BN ? P : BN;
  const int n_logical = (L + P - 1) >> log2P;
  const int64_t page_elems = (int64_t)P * D;
  const int pg_fallback = pt[i_max >> log2P];

  // ---- the query row (column of S^T) this lane owns
  const int r = wave * 32 + m;
  const int hh = r / p.T;
  const int tq = it.tok0 + (r - hh * p.T);
  const bool valid = hh < p.G && tq < tok_end;
  const int pos = valid ? si.q_start + tq : -1;
  const int hq = g * p.G + hh;
  const int win_lo = cls == RK_GLOBAL ? 0 : pos - p.window + 1;
  const int wmin = __builtin_amdgcn_readfirstlane(wave_min(valid ? pos : INT32_MAX));
  const int wmax = __builtin_amdgcn_readfirstlane(wave_max(pos));

  bf16x8 qf[NC];
  {
    const bf16_t *qrow = static_cast<const bf16_t *>(p.q) + ((int64_t)(si.cu_q + tq) * p.H + hq) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 z = {};
      qf[c] = valid ? *reinterpret_cast<const bf16x8 *>(qrow + 16 * c + 8 * hl) : z;
    }
  }

  // ---- tile-invariant geometry of this wave's 1 KB load blocks (same image as attn_bf16)
  int k_key0[NU], k_loff[NU], v_pi[NU], v_loff[NU];
  const bool k_split = D == 64 && P < 16;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int b = wave * NU + u;
    const int row = b * KROWS_U + lane / (D / 8);
    const int slot = lane % (D / 8);
    const int key = swap_bits23(row);
    const int chunk = slot ^ kswz<D>(row);
    k_key0[u] = swap_bits23(b * KROWS_U) & ~(KROWS_U - 1);
    k_loff[u] = (P <= BN ? (key & (P - 1)) : key) * D + chunk * 8;
    const int upp = D * Pt * 2 / 1024;
    const int rows_u = 512 / Pt;
    const int d = (b % upp) * rows_u + lane / (Pt / 8);
    const int cg = (lane % (Pt / 8)) ^ vswz(d, Pt);
    v_pi[u] = b / upp;
    v_loff[u] = d * P + cg * 8;
  }
  int v_rd[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int k8 = 2 * q4 + hl;
    const int cpr = Pt / 8;
    v_rd[q4] = (k8 / cpr) * D * Pt + m * Pt + (((k8 % cpr) ^ vswz(m, Pt)) << 3);
  }
  int k_rd[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) k_rd[c] = m * D + (((2 * c + hl) ^ kswz<D>(m)) << 3);

  auto page_of = [&](int lp) -> int {
    const int pg = lp < n_logical ? pt[lp] : -1;
    return pg >= 0 ? pg : pg_fallback;
  };
  auto issue_tile = [&](int tile, int buf) {
    const int j0 = tile * BN;
    int pgk[NU], pgv[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      pgk[u] = page_of((j0 + k_key0[u]) >> log2P);
      pgv[u] = page_of((j0 >> log2P) + v_pi[u]);
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int b = wave * NU + u;
      int pk_ = pgk[u];
      if (k_split) pk_ = page_of((j0 + swap_bits23(b * KROWS_U + lane / (D / 8))) >> log2P);
      const int ko = P > BN ? (j0 & (P - 1)) * D : 0;
      load_lds16(kpg + (int64_t)pk_ * page_elems + k_loff[u] + ko, &sm.k[buf][b * 512]);
      const int vo = P > BN ? (j0 & (P - 1)) : 0;
      load_lds16(vpg + (int64_t)pgv[u] * page_elems + v_loff[u] + vo, &sm.v[buf][b * 512]);
    }
  };

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = f32x16{};
  float mrun = kNegBig, lsum = 0.f;
  const float c2 = p.scale_log2;

  // per-tile classes for this wave
  auto tile_skip = [&](int j0) {
    return wmax < 0 || j0 > wmax || (cls == RK_LOCAL && j0 >= p.sink && j0 + BN - 1 <= wmin - p.window);
  };
  auto tile_full = [&](int j0) {
    return j0 + BN - 1 <= wmin && (cls == RK_GLOBAL || j0 + BN <= p.sink || j0 > wmax - p.window);
  };
  // S^T of one 32-key half (kb) of the tile in stage `buf`
  auto qk_half = [&](int buf, int kb, f32x16 &s) {
    const bf16_t *Kb = sm.k[buf] + 32 * kb * D;
    s = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Kb + k_rd[c]);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s, 0, 0, 0);
    }
  };
  // mask, online-softmax update and bf16 pack of one half; pk[cc] = keys 16 cc .. 16 cc + 15 of the half
  auto soft_half = [&](int j0, bool full, int kb, f32x16 &s, bf16x8 (&pk)[2]) {
    if (!full) {
      const int jb = j0 + 32 * kb + 8 * hl;
      const int hi = pos - jb, lo = win_lo - jb, sk = p.sink - jb;
      if (cls == RK_GLOBAL) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 16 * (i >> 3) + (i & 7);
          s[i] = off <= hi ? s[i] : -INFINITY;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = 16 * (i >> 3) + (i & 7);
          s[i] = (off <= hi && (off >= lo || off < sk)) ? s[i] : -INFINITY;
        }
      }
    }
    float mt = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[i]);
    mt = halves_max(mt);
    const float mts = mt * c2;
    if (__any(mts > mrun + kRescaleSlack)) {
      const float mnew = fmaxf(mrun, mts);
      const float alpha = fast_exp2(mrun - mnew);
#pragma unroll
      for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
      lsum *= alpha;
      mrun = mnew;
    }
    f32x8 e0, e1;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e0[i] = fast_exp2(fmaf(s[i], c2, -mrun));
      e1[i] = fast_exp2(fmaf(s[i + 8], c2, -mrun));
      ps += e0[i] + e1[i];
    }
    lsum += ps;
    pk[0] = __builtin_convertvector(e0, bf16x8);
    pk[1] = __builtin_convertvector(e1, bf16x8);
  };
  auto pv_half = [&](int buf, int kb, const bf16x8 (&pk)[2]) {
    const bf16_t *Vb = sm.v[buf];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Vb + v_rd[2 * kb + cc] + 32 * db * Pt);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[cc], oacc[db], 0, 0, 0);
      }
  };

  issue_tile(tr.tile(0), 0);
  if (ntiles > 1) issue_tile(tr.tile(1), 1);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();

  // The two groups run separate loops (same number of barriers) so that each loop's registers are
  // allocated on their own.
  if (group == 0) {
    for (int idx = 0; idx < ntiles; ++idx) {
      const int buf = idx & 3;
      if (idx + 2 < ntiles) issue_tile(tr.tile(idx + 2), (idx + 2) & 3);
      const int j0 = tr.tile(idx) * BN;
      if (!tile_skip(j0)) {
        const bool full = tile_full(j0);
        f32x16 s0, s1;
        bf16x8 pk0[2], pk1[2];
        // phase boundaries are scheduling barriers: the order of MFMA and softmax phases is the point
        qk_half(buf, 0, s0);
        __builtin_amdgcn_sched_barrier(0);
        soft_half(j0, full, 0, s0, pk0);
        __builtin_amdgcn_sched_barrier(0);
        qk_half(buf, 1, s1);
        pv_half(buf, 0, pk0);
        __builtin_amdgcn_sched_barrier(0);
        soft_half(j0, full, 1, s1, pk1);
        __builtin_amdgcn_sched_barrier(0);
        pv_half(buf, 1, pk1);
      }
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
    }
  } else {
    f32x16 s0, s1;  // s1: second half of the previous tile, finished in the next iteration
    int j0_prev = 0;
    bool skip_prev = true, full_prev = true;
    for (int idx = 0; idx < ntiles; ++idx) {
      const int buf = idx & 3;
      if (idx + 2 < ntiles) issue_tile(tr.tile(idx + 2), (idx + 2) & 3);
      const int j0 = tr.tile(idx) * BN;
      const bool skip = tile_skip(j0), full = tile_full(j0);
      bf16x8 pk0[2], pk1[2];
      if (!skip_prev) soft_half(j0_prev, full_prev, 1, s1, pk1);
      __builtin_amdgcn_sched_barrier(0);
      if (!skip) qk_half(buf, 0, s0);
      if (!skip_prev) pv_half((idx - 1) & 3, 1, pk1);
      __builtin_amdgcn_sched_barrier(0);
      if (!skip) {
        soft_half(j0, full, 0, s0, pk0);
        __builtin_amdgcn_sched_barrier(0);
        qk_half(buf, 1, s1);
        pv_half(buf, 0, pk0);
      }
      j0_prev = j0;
      skip_prev = skip;
      full_prev = full;
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
    }
    if (!skip_prev) {
      bf16x8 pk1[2];
      soft_half(j0_prev, full_prev, 1, s1, pk1);
      pv_half((ntiles - 1) & 3, 1, pk1);
    }
  }

  const float lt = halves_sum(lsum);
  if (!valid) return;
  const float inv = 1.0f / lt;
  bf16_t *orow = static_cast<bf16_t *>(p.o) + ((int64_t)(si.cu_q + tq) * p.H + hq) * D;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      f32x4 w = {oacc[db][4 * a4 + 0] * inv, oacc[db][4 * a4 + 1] * inv, oacc[db][4 * a4 + 2] * inv,
                 oacc[db][4 * a4 + 3] * inv};
      *reinterpret_cast<bf16x4 *>(orow + 32 * db + 8 * a4 + 4 * hl) = __builtin_convertvector(w, bf16x4);
    }
  if (p.lse && hl == 0)
    p.lse[(int64_t)hq * p.total_q + si.cu_q + tq] = (mrun + log2f(lt)) * 0.69314718055994531f;
}

// ------------------------------------------------------------------------------------------------
// fp32 attention (vector ALUs): two lanes per query row, each holding half of the channels.
// ------------------------------------------------------------------------------------------------

constexpr int kF32Threads = 512;

template <int D>
__global__ void __launch_bounds__(kF32Threads, 1) attn_f32(AttnParams p) {
  constexpr int DH = D / 2;
  constexpr int VPF = BN + 1;
  __shared__ __attribute__((aligned(16))) float sk[BN * D];
  __shared__ float sv[D * VPF];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, half = lane >> 5;
  const int r = wave * 32 + (lane & 31);
  const Item it = p.items[blockIdx.x];
  if (it.seq < 0) return;  // schedule padding: keeps the next items on their XCD
  const SeqInfo si = p.seqs[it.seq];
  const int g = it.kv_head;
  const int cls = p.head_class[g];
  const int tok_end = min(it.tok0 + p.T, si.n_q);
  const int L = si.kv_len;
  const TileRange tr = tile_range(cls, si.q_start + it.tok0, si.q_start + tok_end - 1, p.sink, p.window);
  const int ntiles = tr.count();
  const int32_t *pt = p.page_ids + p.page_base[g * p.num_seqs + it.seq];
  const float *kpg = static_cast<const float *>(p.k_pages);
  const float *vpg = static_cast<const float *>(p.v_pages);
  const int P = p.P, log2P = p.log2P;

  const int hh = r / p.T;
  const int t = it.tok0 + (r - hh * p.T);
  const bool valid = hh < p.G && t < tok_end;
  const int pos = valid ? si.q_start + t : -1;
  const int hq = g * p.G + hh;
  const float *qrow = static_cast<const float *>(p.q) + ((int64_t)(si.cu_q + t) * p.H + hq) * D + half * DH;

  float qv[DH], acc[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d) {
    qv[d] = valid ? qrow[d] : 0.f;
    acc[d] = 0.f;
  }
  float mrun = kNegBig, lsum = 0.f;
  const float c2 = p.scale_log2;

  for (int idx = 0; idx < ntiles; ++idx) {
    const int j0 = tr.tile(idx) * BN;
    __syncthreads();
    for (int c = tid; c < BN * D / 4; c += kF32Threads) {
      const int row = c / (D / 4), col = c - row * (D / 4);
      const int j = j0 + row;
      f32x4 val = {0.f, 0.f, 0.f, 0.f};
      if (j < L) {
        const int pg = pt[j >> log2P];
        if (pg >= 0) val = *reinterpret_cast<const f32x4 *>(kpg + ((int64_t)pg * P + (j & (P - 1))) * D + col * 4);
      }
      *reinterpret_cast<f32x4 *>(&sk[row * D + col * 4]) = val;
    }
    for (int c = tid; c < BN * D; c += kF32Threads) {
      const int d = c / BN, kk = c - d * BN;
      const int j = j0 + kk;
      float val = 0.f;
      if (j < L) {
        const int pg = pt[j >> log2P];
        if (pg >= 0) val = vpg[(int64_t)pg * D * P + (int64_t)d * P + (j & (P - 1))];
      }
      sv[d * VPF + kk] = val;
    }
    __syncthreads();
    for (int k0 = 0; k0 < BN; k0 += 16) {
      float sc[16];
      float mt = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const float *kr = &sk[(k0 + kk) * D + half * DH];
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < DH; ++d) s = fmaf(qv[d], kr[d], s);
        s += __shfl_xor(s, 32);
        if (!visible(cls, pos, j0 + k0 + kk, p.sink, p.window)) s = -INFINITY;
        sc[kk] = s;
        mt = fmaxf(mt, s);
      }
      const float mts = mt * c2;
      if (mts > mrun + kRescaleSlack) {
        const float alpha = fast_exp2(mrun - mts);
#pragma unroll
        for (int d = 0; d < DH; ++d) acc[d] *= alpha;
        lsum *= alpha;
        mrun = mts;
      }
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        const float e = fast_exp2(fmaf(sc[kk], c2, -mrun));
        lsum += e;
#pragma unroll
        for (int d = 0; d < DH; ++d) acc[d] = fmaf(e, sv[(half * DH + d) * VPF + k0 + kk], acc[d]);
      }
    }
  }
  if (!valid) return;
  const float inv = 1.0f / lsum;
  float *orow = static_cast<float *>(p.o) + ((int64_t)(si.cu_q + t) * p.H + hq) * D + half * DH;
#pragma unroll
  for (int d = 0; d < DH; ++d) orow[d] = acc[d] * inv;
  if (p.lse && half == 0) p.lse[(int64_t)hq * p.total_q + si.cu_q + t] = (mrun + log2f(lsum)) * 0.69314718055994531f;
}

// ------------------------------------------------------------------------------------------------
// page writers
// ------------------------------------------------------------------------------------------------

template <typename T>
struct Vec16;
template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
};

template <typename T>
__device__ __forceinline__ float to_f(T x) {
  return static_cast<float>(x);
}
template <typename T>
__device__ __forceinline__ T from_f(float x) {
  return static_cast<T>(x);
}

constexpr int kTokBlock = 64;  // tokens staged per LDS pass of the V transpose

// One workgroup writes the tokens of one logical page of one KV head.  K rows go to the page as is
// (import: rotated by delta first); V rows are transposed through LDS into the channel-major page.
template <typename T, int D, bool IMPORT>
__global__ void __launch_bounds__(256) kv_write(KvWriteParams p) {
  constexpr int VEC = Vec16<T>::N;
  constexpr int VPITCH = D + 1;
  __shared__ T sv[kTokBlock * VPITCH];
  __shared__ float cs[D / 2], sn[D / 2];

  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int P = p.P;
  int seq, lp, t_lo, t_hi;
  SeqInfo si{};
  if (IMPORT) {
    seq = p.seq;
    lp = p.page0 + blockIdx.x;
    t_lo = max(lp * P, p.tok_begin);
    t_hi = min(lp * P + P, p.tok_begin + p.n_tok);
  } else {
    seq = p.app_items[2 * blockIdx.x];
    lp = p.app_items[2 * blockIdx.x + 1];
    si = p.seqs[seq];
    t_lo = max(lp * P, si.q_start);
    t_hi = min(lp * P + P, si.kv_len);
  }
  const int pg = p.page_ids[p.page_base[g * p.num_seqs + seq] + lp];
  if (pg < 0 || t_hi <= t_lo) return;  // import: this head does not hold the page
  const int n = t_hi - t_lo;
  const int s0 = t_lo - lp * P;
  const T *ksrc = static_cast<const T *>(p.k_src);
  const T *vsrc = static_cast<const T *>(p.v_src);
  auto src_row = [&](const T *base, int t) -> const T * {
    if (IMPORT) return base + (int64_t)g * p.src_head_stride + (int64_t)(t - p.tok_begin) * D;
    return base + ((int64_t)(si.cu_q + t - si.q_start) * p.Hkv + g) * D;
  };
  T *kdst = static_cast<T *>(p.k_pages) + ((int64_t)pg * P + s0) * D;
  T *vdst = static_cast<T *>(p.v_pages) + (int64_t)pg * D * P;

  if (IMPORT) {
    for (int mm = tid; mm < D / 2; mm += blockDim.x) {
      const double th = pow(p.rope_base, -2.0 * (double)mm / (double)D);
      const double a = (double)p.delta * th;
      cs[mm] = (float)cos(a);
      sn[mm] = (float)sin(a);
    }
    __syncthreads();
  }

  // K
  if (!IMPORT) {
    for (int c = tid; c < n * (D / VEC); c += blockDim.x) {
      const int tk = c / (D / VEC), ch = c - tk * (D / VEC);
      *reinterpret_cast<u32x4 *>(kdst + (int64_t)tk * D + ch * VEC) =
          *reinterpret_cast<const u32x4 *>(src_row(ksrc, t_lo + tk) + ch * VEC);
    }
  } else {
    for (int c = tid; c < n * (D / 2); c += blockDim.x) {
      const int tk = c / (D / 2), mm = c - tk * (D / 2);
      const int ia = p.rope_style == RK_ROPE_ROTATE_HALF ? mm : 2 * mm;
      const int ib = p.rope_style == RK_ROPE_ROTATE_HALF ? mm + D / 2 : 2 * mm + 1;
      const T *s = src_row(ksrc, t_lo + tk);
      const float xa = to_f(s[ia]), xb = to_f(s[ib]);
      const float ya = xa * cs[mm] - xb * sn[mm];
      const float yb = xb * cs[mm] + xa * sn[mm];
      kdst[(int64_t)tk * D + ia] = from_f<T>(ya);
      kdst[(int64_t)tk * D + ib] = from_f<T>(yb);
    }
  }

  // Append into the sequence's last page also clears the slots past kv_len (K rows and V columns),
  // so that every slot of a held page that attention may load holds a finite value.
  if (!IMPORT && t_hi == si.kv_len && t_hi < lp * P + P) {
    const int z0 = t_hi - lp * P;  // first unused slot
    T *kz = static_cast<T *>(p.k_pages) + (int64_t)pg * P * D;
    for (int c = tid; c < (P - z0) * D; c += blockDim.x) kz[(int64_t)z0 * D + c] = from_f<T>(0.f);
    for (int c = tid; c < (P - z0) * D; c += blockDim.x) {
      const int d = c / (P - z0), sl = z0 + c % (P - z0);
      vdst[(int64_t)d * P + sl] = from_f<T>(0.f);
    }
  }

  // V: transpose [tokens][D] -> page [D][P] through LDS, kTokBlock tokens at a time
  for (int tb = 0; tb < n; tb += kTokBlock) {
    const int nb = min(kTokBlock, n - tb);
    __syncthreads();
    for (int c = tid; c < nb * D; c += blockDim.x) {
      const int tk = c / D, d = c - tk * D;
      sv[tk * VPITCH + d] = src_row(vsrc, t_lo + tb + tk)[d];
    }
    __syncthreads();
    const int sa = s0 + tb;  // first slot of this block
    for (int c = tid; c < nb * D; c += blockDim.x) {
      const int d = c / nb, tk = c - d * nb;
      vdst[(int64_t)d * P + sa + tk] = sv[tk * VPITCH + d];
    }
  }
}

}  // namespace

hipError_t launch_attention(const AttnParams &p, int dtype, int head_dim, hipStream_t stream) {
  if (p.n_items <= 0) return hipSuccess;
  dim3 grid(p.n_items);
  if (dtype == RK_BF16) {
#ifdef RK_ATTN_PINGPONG
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_bf16_pp<128>, grid, dim3(512), 0, stream, p);
    else
      hipLaunchKernelGGL(attn_bf16_pp<64>, grid, dim3(512), 0, stream, p);
#else
    constexpr int NT = kRowsPerItem / RK_ATTN_NB * 2;
    if (head_dim == 128)
      hipLaunchKernelGGL((attn_bf16<128, RK_ATTN_NB>), grid, dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL((attn_bf16<64, RK_ATTN_NB>), grid, dim3(NT), 0, stream, p);
#endif
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_f32<128>, grid, dim3(kF32Threads), 0, stream, p);
    else
      hipLaunchKernelGGL(attn_f32<64>, grid, dim3(kF32Threads), 0, stream, p);
  }
  return hipGetLastError();
}

template <bool IMPORT>
static hipError_t launch_kv(const KvWriteParams &p, int n_blocks, int dtype, int head_dim, hipStream_t stream) {
  if (n_blocks <= 0 || p.Hkv <= 0) return hipSuccess;
  dim3 grid(n_blocks, p.Hkv);
  if (dtype == RK_BF16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((kv_write<bf16_t, 128, IMPORT>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((kv_write<bf16_t, 64, IMPORT>), grid, dim3(256), 0, stream, p);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((kv_write<float, 128, IMPORT>), grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((kv_write<float, 64, IMPORT>), grid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_append(const KvWriteParams &p, int dtype, int head_dim, hipStream_t stream) {
  return launch_kv<false>(p, p.n_items, dtype, head_dim, stream);
}

hipError_t launch_import(const KvWriteParams &p, int n_pages, int dtype, int head_dim, hipStream_t stream) {
  return launch_kv<true>(p, n_pages, dtype, head_dim, stream);
}

}  // namespace rk
