// gfx950 (CDNA4) attention kernels of the SegPagedAttention prefill library.
//
//  * attn_bf16<D>: mask-free head-ragged paged prefill attention.  Global heads attend over every
//    context page, local heads over their sink and recent-window pages (page "为什么长上下文推理这么
//    慢？RedKnot如何用1个百分点的质量代价换来2–5倍TTFT加速" (bjdmk.com.cn), section 二 ③); no mask
//    tensor exists anywhere: visibility comes from token indices (page "RedKnot - Xiaohongshuが開発
//    した…" (aiboss88.com), section 技術原則, fourth item).
//  * attn_f32<D>: the same computation for fp32 storage, on the vector ALUs.
//
// Design of attn_bf16 (one work item = 256 query rows = G heads x T tokens of one KV head; eight
// waves of 32 rows, two per SIMD):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: keys are the M dimension, queries the N dimension, so
//    each lane holds one query column and 16 keys per 32x32 block; a row max is in-lane max3 ops
//    plus one v_permlane32_swap between the two half-waves.
//  * K rows sit in LDS in a permuted order (bits 2 and 3 of the key index swapped) so that the S^T
//    accumulator register i of lane half h holds key 16*(i/8) + 8*h + i%8: the eight probabilities
//    a lane needs as the B operand of the PV product (O^T = V^T P^T) for 16-key chunk c are
//    exactly its registers 8c..8c+7, converted to bf16 in place -- no shuffles.
//  * V pages are stored channel-major ([D][P]) so the A operand of PV (8 consecutive keys of one
//    channel) is one 16-byte LDS read.
//  * Tiles reach LDS by direct 16-byte buffer->LDS loads (a descriptor on the page's scalar address,
//    32-bit lane offset), one 1 KB block per instruction; XOR swizzles of the 16-byte chunks keep the
//    operand reads free of bank conflicts.  The buffer form matters: with the global form in flight
//    the compiler makes every LDS operand read wait for all outstanding ones.
//  * Operand reads run one MFMA group ahead of their products (K chunk c + 1 during chunk c, V of
//    the first PV group during the softmax), held in place by sched_barrier(0).
//  * Two 64-key tiles per step, double-buffered: the next step's loads are issued before this
//    step's MFMA work; one barrier per step.  The buffer index is a compile-time constant (the step
//    loop is unrolled by two), so operand addresses are lane registers plus immediate offsets.
//  * Online softmax in fp32 with exp2; the running max is only raised when a new score exceeds
//    it by more than 2^8 in the exp2 domain, so the O rescale (64 VALU ops per block) is rare.
//    Skipping it is exact: weights up to 2^8 are represented the same way in fp32 and bf16.
//  * Per-wave tile classes from indices: skip (no key visible to any row of the wave), full (every
//    key visible to every row: no per-element work) or edge (per-element index compare).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rk_device.h"
#include "rk_internal.h"
#include "rk_seg.h"

namespace rk {
namespace {

constexpr int BN = kKeyTile;
constexpr float kNegBig = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;  // log2 of the largest un-normalised weight allowed

// ------------------------------------------------------------------------------------------------
// bf16 attention
// ------------------------------------------------------------------------------------------------

#ifndef RK_TILES_PER_STEP
#define RK_TILES_PER_STEP 2  // key tiles staged per LDS buffer and barrier step
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
template <int D, int TPS>
struct AttnBf16Smem {
  bf16_t k[2][TPS][BN * D];  // double buffer: the next step's tiles load while these are used
  bf16_t v[2][TPS][D * BN];
};

__device__ __forceinline__ int vswz(int d, int Pt) {
  return (d / (128 / Pt)) & (Pt / 8 - 1);
}

// One work item = 256 query rows; eight waves of 32 rows (one query column of S^T per lane).
// Each step stages TPS key tiles of 64 keys (K and V) in one of two LDS buffers while the other
// buffer's tiles are used: the loads of step s + 1 are issued before the compute of step s and one
// barrier closes the step.  Per tile: S^T = K Q^T (16 MFMAs), the online softmax, O^T += V^T P^T
// (16 MFMAs).
// SMALLP: 8-key pages, where one 1 KB load block spans two pages.
template <int D, bool SMALLP>
__global__ void __launch_bounds__(2 * kRowsPerItem, 1) attn_bf16(AttnParams p) {
  constexpr int NC = D / 16;                 // 16-channel chunks of the QK product
  constexpr int ND = D / 32;                 // 32-channel blocks of O^T
  constexpr int UNITS = BN * D * 2 / 1024;   // 1 KB load blocks per tile, for K and for V each
  constexpr int NU = UNITS / 8;              // per wave
  constexpr int KROWS_U = 512 / D;           // K rows per block
  constexpr int TPS = RK_TILES_PER_STEP;
  static_assert(NU >= 1 && UNITS % 8 == 0, "tile does not split over the waves");
  __shared__ __attribute__((aligned(1024))) AttnBf16Smem<D, TPS> sm;

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
  const int ntiles = tr.count();  // >= 1
  const int nsteps = (ntiles + TPS - 1) / TPS;
  const int32_t *__restrict__ pt = p.page_ids + p.page_base[g * p.num_seqs + it.seq];
  const bf16_t *__restrict__ kpg = static_cast<const bf16_t *>(p.k_pages);
  const bf16_t *__restrict__ vpg = static_cast<const bf16_t *>(p.v_pages);
  const int P = p.P, log2P = p.log2P;
  const int Pt = P < BN ? P : BN;
  const int n_logical = (L + P - 1) >> log2P;
  const int64_t page_elems = (int64_t)P * D;
  const uint32_t page_bytes = (uint32_t)page_elems * 2;
  // Pages a tile touches but the head does not hold (or past the sequence's last page) are read
  // from this page instead: the page of the item's last query, held and fully written (the append
  // clears its slots past kv_len).  Its keys are masked out, so only finiteness matters.
  const int pg_fallback = pt[i_max >> log2P];

  // ---- the query row (column of S^T) this lane owns
  const int r = wave * 32 + m;
  const int hh = r / p.T;
  const int tq = it.tok0 + (r - hh * p.T);
  const bool valid = hh < p.G && tq < tok_end;
  const int pos = valid ? si.q_start + tq : -1;
  const int hq = g * p.G + hh;
  const int win_lo = cls == RK_GLOBAL ? 0 : pos - p.window + 1;  // first window key of the row
  // wave-uniform query range: scalar registers, so tile classes are scalar branches
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

  // ---- tile-invariant geometry of this wave's 1 KB load blocks (block b = wave * NU + u)
  int k_key0[NU], v_pi[NU];         // K: first key of the block (uniform); V: page-in-tile
  uint32_t k_loff[NU], v_loff[NU];  // lane's byte offset in its page (unsigned 32-bit: the load
                                    // takes a scalar page address plus a lane offset)
  // a D = 64 K block spans 8 keys; with 8-key pages its two 4-key halves come from two pages
  constexpr bool k_split = D == 64 && SMALLP;
  constexpr bool v_split = SMALLP;
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
    k_loff[u] = ((P <= BN ? (key & (P - 1)) : key) * D + chunk * 8) * 2;
    // V: block b of the [D / 32][page-in-tile][32][Pt] image; the lane fills elements e .. e + 7
    const int e = 512 * b + 8 * lane;
    const int r2 = e % (32 * BN), r3 = r2 % (32 * Pt);
    const int d = 32 * (e / (32 * BN)) + r3 / Pt;
    const int cg = ((r3 % Pt) >> 3) ^ vswz(d, Pt);
    // page-in-tile: uniform over the block, except with 8-key pages (lanes 32-63 take the next page)
    v_pi[u] = v_split ? r2 / (32 * Pt) : ((512 * b) % (32 * BN)) / (32 * Pt);
    v_loff[u] = (d * P + cg * 8) * 2;   // + (j0 & (P - 1)) keys when P > 64
  }
  // V^T read offsets (elements) for the four (kb, cc) key chunks of a 64-key tile, channel row m of
  // the first 32-channel block; block db is 32 * BN elements further (vswz(m + 32 db) = vswz(m))
  int v_rd[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int k8 = 2 * q4 + hl;  // 8-key chunk 4kb + 2cc + hl
    const int cpr = Pt / 8;
    v_rd[q4] = (k8 / cpr) * 32 * Pt + m * Pt + (((k8 % cpr) ^ vswz(m, Pt)) << 3);
  }
  // K read offsets (elements) for the NC channel chunks, rows m (+32 for the second key block)
  int k_rd[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) k_rd[c] = m * D + (((2 * c + hl) ^ kswz<D>(m)) << 3);

  // Page ids of a step's tiles: one vector load per wave (lane x * npt + i holds the id of page i
  // of the step's x-th tile), issued a step ahead and read back with readlane, so the lookup latency
  // stays off the critical path and no scalar load shares the LDS wait counter with operand reads.
  const int npt = P < BN ? BN / P : 1;
  auto load_ids = [&](int step) -> int {
    const int x = lane / npt, i = lane - x * npt;
    const int t = step * TPS + x;
    int v = -1;
    if (x < TPS && t < ntiles) {
      const int lp = ((tr.tile(t) * BN) >> log2P) + i;
      if (lp < n_logical) v = pt[lp];
    }
    return v;
  };
  auto fix = [&](int pg) { return pg >= 0 ? pg : pg_fallback; };
  // loads of the step's x-th tile (key tile `tile`) into slot x of buffer buf
  auto issue_tile = [&](int tile, int buf, int x, int ids) {
    const int j0 = tile * BN;
    const int lane0 = x * npt;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int b = wave * NU + u;
      const int ko = P > BN ? (j0 & (P - 1)) * D : 0;
      if constexpr (k_split) {
        const int pg = fix(__shfl(ids, lane0 + (swap_bits23(b * KROWS_U + lane / (D / 8)) >> log2P)));
        load_lds16(reinterpret_cast<const char *>(kpg + (int64_t)pg * page_elems + ko) + k_loff[u], &sm.k[buf][x][b * 512]);
      } else {
        const int pg = fix(__builtin_amdgcn_readlane(ids, lane0 + (P < BN ? (k_key0[u] >> log2P) : 0)));
        const char *page = reinterpret_cast<const char *>(kpg + (int64_t)pg * page_elems + ko);  // uniform
        load_lds16_buf(page, k_loff[u], page_bytes, &sm.k[buf][x][b * 512]);
      }
      const int vo = P > BN ? (j0 & (P - 1)) : 0;
      if constexpr (v_split) {
        const int pg = fix(__shfl(ids, lane0 + v_pi[u]));
        load_lds16(reinterpret_cast<const char *>(vpg + (int64_t)pg * page_elems + vo) + v_loff[u], &sm.v[buf][x][b * 512]);
      } else {
        const int pg = fix(__builtin_amdgcn_readlane(ids, lane0 + v_pi[u]));
        const char *page = reinterpret_cast<const char *>(vpg + (int64_t)pg * page_elems + vo);  // uniform
        load_lds16_buf(page, v_loff[u], page_bytes, &sm.v[buf][x][b * 512]);
      }
    }
  };
  auto issue_step = [&](int step, int buf, int ids) {
#pragma unroll
    for (int x = 0; x < TPS; ++x)
      if (step * TPS + x < ntiles) issue_tile(tr.tile(step * TPS + x), buf, x, ids);
  };

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = f32x16{};
  float mrun = kNegBig, lsum = 0.f;
  const float c2 = p.scale_log2;

  // one 64-key tile: first key j0, operands in Kb / Vb
  auto tile_compute = [&](const int j0, const bf16_t *Kb, const bf16_t *Vb) __attribute__((always_inline)) {
    const bool skip = wmax < 0 || j0 > wmax ||
                      (cls == RK_LOCAL && j0 >= p.sink && j0 + BN - 1 <= wmin - p.window);
    const bool full = j0 + BN - 1 <= wmin &&
                      (cls == RK_GLOBAL || j0 + BN <= p.sink || j0 > wmax - p.window);
    if (skip) return;
    // S^T for the tile's 64 keys (two 32-key blocks) x this wave's 32 queries
    f32x16 s[2] = {};
    {
      bf16x8 ka[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) ka[0][kb] = *reinterpret_cast<const bf16x8 *>(Kb + k_rd[0] + 32 * kb * D);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int cur = c & 1;
        if (c + 1 < NC) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            ka[cur ^ 1][kb] = *reinterpret_cast<const bf16x8 *>(Kb + k_rd[c + 1] + 32 * kb * D);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[cur][kb], qf[c], s[kb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // V operands of the first PV group, read while the softmax runs
    bf16x8 va[2][ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) va[0][db] = *reinterpret_cast<const bf16x8 *>(Vb + v_rd[0] + db * 32 * BN);
    __builtin_amdgcn_sched_barrier(0);
    if (!full) {
      // key of register i of block kb: jb + 16 * (i / 8) + i % 8, jb = j0 + 32 kb + 8 hl
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int jb = j0 + 32 * kb + 8 * hl;
        const int hi = pos - jb;     // visible: off <= hi
        const int lo = win_lo - jb;  // local: off >= lo, or off < sk
        const int sk = p.sink - jb;
        if (cls == RK_GLOBAL) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = 16 * (i >> 3) + (i & 7);
            s[kb][i] = off <= hi ? s[kb][i] : -INFINITY;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = 16 * (i >> 3) + (i & 7);
            s[kb][i] = (off <= hi && (off >= lo || off < sk)) ? s[kb][i] : -INFINITY;
          }
        }
      }
    }
    float mt = s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, s[0][i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[1][i]);
    mt = halves_max(mt);
    // The running max is only raised when a score exceeds it by more than 2^8 in the exp2 domain;
    // O and the row sum are rescaled then.
    const float mts = mt * c2;
    if (__any(mts > mrun + kRescaleSlack)) {
      const float mnew = fmaxf(mrun, mts);
      const float alpha = fast_exp2(mrun - mnew);
#pragma unroll
      for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
      lsum *= alpha;
      mrun = mnew;
    }
    // bf16 weights; pk[kb][cc] is the B operand of the PV product for keys 32 kb + 16 cc .. + 15
    bf16x8 pk[2][2];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x8 e0, e1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e0[i] = fast_exp2(fmaf(s[kb][i], c2, -mrun));
        e1[i] = fast_exp2(fmaf(s[kb][i + 8], c2, -mrun));
        ps += e0[i] + e1[i];
      }
      pk[kb][0] = __builtin_convertvector(e0, bf16x8);
      pk[kb][1] = __builtin_convertvector(e1, bf16x8);
    }
    lsum += ps;
    // O^T += V^T P^T
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int cur = g4 & 1;
      if (g4 + 1 < 4) {
#pragma unroll
        for (int db = 0; db < ND; ++db)
          va[cur ^ 1][db] = *reinterpret_cast<const bf16x8 *>(Vb + v_rd[g4 + 1] + db * 32 * BN);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < ND; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[cur][db], pk[g4 >> 1][g4 & 1], oacc[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Loads retire in issue order.  Order per step: data of the next step, then the page ids of the
  // step after it; at the end of the step the next step's data must be in LDS and only the id load
  // (when one was issued) may still be in flight.
  constexpr int WAIT_ALL = 0x0f70;      // vmcnt(0)
  constexpr int WAIT_BUT_ONE = 0x0f71;  // vmcnt(1)
  int ids = load_ids(0);
  issue_step(0, 0, ids);
  bool ids_pending = nsteps > 1;
  if (ids_pending) ids = load_ids(1);
  if (ids_pending) __builtin_amdgcn_s_waitcnt(WAIT_BUT_ONE);
  else __builtin_amdgcn_s_waitcnt(WAIT_ALL);
  __syncthreads();

  // One step.  The LDS buffer index is a template constant (the loop below is unrolled by two),
  // so every operand address is a lane register plus an immediate offset.
  auto step = [&](const int s, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    ids_pending = false;
    if (s + 1 < nsteps) {
      issue_step(s + 1, buf ^ 1, ids);
      ids_pending = s + 2 < nsteps;
      if (ids_pending) ids = load_ids(s + 2);
    }
#pragma unroll
    for (int x = 0; x < TPS; ++x)
      if (s * TPS + x < ntiles) tile_compute(tr.tile(s * TPS + x) * BN, sm.k[buf][x], sm.v[buf][x]);
    if (ids_pending) __builtin_amdgcn_s_waitcnt(WAIT_BUT_ONE);
    else __builtin_amdgcn_s_waitcnt(WAIT_ALL);
    __syncthreads();
  };
  for (int s = 0; s < nsteps; s += 2) {
    step(s, IntC<0>{});
    if (s + 1 < nsteps) step(s + 1, IntC<1>{});
  }

  // ---- epilogue: O^T accumulator (lane column = query, 16 channels per 32-channel block)
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

}  // namespace

hipError_t launch_attention(const AttnParams &p, int dtype, int head_dim, hipStream_t stream) {
  if (p.n_items <= 0) return hipSuccess;
  dim3 grid(p.n_items);
  if (dtype == RK_BF16) {
    const dim3 block(2 * kRowsPerItem);
    if (head_dim == 128) {
      if (p.P < 16) hipLaunchKernelGGL((attn_bf16<128, true>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((attn_bf16<128, false>), grid, block, 0, stream, p);
    } else {
      if (p.P < 16) hipLaunchKernelGGL((attn_bf16<64, true>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((attn_bf16<64, false>), grid, block, 0, stream, p);
    }
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_f32<128>, grid, dim3(kF32Threads), 0, stream, p);
    else
      hipLaunchKernelGGL(attn_f32<64>, grid, dim3(kF32Threads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace rk
