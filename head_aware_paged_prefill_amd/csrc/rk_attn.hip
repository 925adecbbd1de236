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
//    each lane holds one query column and 16 keys per 32x32 block.
//  * K rows sit in LDS in a permuted order (bits 2 and 3 of the key index swapped) so that the S^T
//    accumulator register i of lane half h holds key 16*(i/8) + 8*h + i%8: the eight probabilities
//    a lane needs as the B operand of the PV product (O^T = V^T P^T) for a 16-key chunk are exactly
//    eight of its registers, converted to bf16 pairs in place -- no shuffles.
//  * V pages are stored channel-major ([D][P]) so the A operand of PV (8 consecutive keys of one
//    channel) is one 16-byte LDS read.
//  * Tiles reach LDS by direct 16-byte buffer->LDS loads (a descriptor on the page's scalar address,
//    32-bit lane offset), one 1 KB block per instruction; XOR swizzles of the 16-byte chunks keep the
//    operand reads free of bank conflicts.  The buffer form matters: with the global form in flight
//    the compiler makes every LDS operand read wait for all outstanding ones.
//  * A two-phase software pipeline over 32-key blocks keeps the matrix core busy while the VALU
//    turns scores into weights: the scores of block j+1 are multiplied beside the second half of
//    block j's exponentials, and block j's PV product beside the first half of block j+1's.  Operand
//    reads run four products ahead, across phases.
//  * Online softmax in fp32 with exp2, without a per-block max: weights are taken against the running
//    max, and only a block whose weight sum exceeds 2^20 (the one case where a weight can) rescales O
//    and recomputes its weights against its true max.  The reference point of the exponentials cancels
//    in O / (row sum) and is added back in the lse, so any point at or below the true max gives the
//    same result up to rounding (fp32 and bf16 keep their relative precision at any magnitude); the
//    bound only keeps the row sum and O far inside the fp32 range.
//  * Two 64-key tiles per LDS step, double-buffered, two barriers per step (K is consumed one block
//    ahead of V).  Block classes come from indices: full (no per-element work) or edge (scores
//    outside the row's visible set set to -inf in place); no mask tensor exists.
//  * The normalised output rows go through LDS, so each store instruction writes whole rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rk_device.h"
#include "rk_internal.h"
#include "rk_seg.h"

namespace rk {
namespace {

constexpr int BN = kKeyTile;
constexpr float kNegBig = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;  // log2 of the largest un-normalised weight allowed (attn_f32)
constexpr float kRescaleAt = 1048576.0f;  // 2^20: a lane's block weight sum that takes the rescale path

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
  int32_t ids[8][2][64];     // per wave: the page ids of the next steps into buffer 0 / 1
};

__device__ __forceinline__ int vswz(int d, int Pt) {
  return (d / (128 / Pt)) & (Pt / 8 - 1);
}

// One work item = 256 query rows; eight waves of 32 rows (one query column of S^T per lane).
// Each LDS step stages TPS key tiles of 64 keys (K and V) in one of two buffers.  A wave runs over
// the 32-key blocks of the item in a two-phase software pipeline, so the matrix core always has the
// products of one block while the VALU works on another:
//   phase A(j): S(j+1) = K(j+1) Q^T (NC products)    beside the exponentials of the second half of S(j)
//   phase B(j): O^T += V(j)^T P(j)^T (NC products)   beside the exponentials of the first half of S(j+1)
// The running max is not taken per block: the exponentials use the current one, and a block whose
// per-lane weight sum exceeds kRescaleAt = 2^20 (then, and only then, some weight may exceed it)
// takes a rare path that finds the block's true row max, rescales O and the row sum, and recomputes
// the block's weights.  A row's first visible block takes that path (the running max starts at
// -1e30) when the row has no visible key in the item's first block; otherwise block 0 sets the
// running max to its own row max.  Later blocks take it only when their scores rise 20 (log2 units)
// above the running max.  With 2^8
// a fifth of the blocks of rows whose keys carry 4x outliers took it.  Over at most 2^26 blocks of 16
// keys per lane the row sum stays below 2^46, and O below 2^46 max|v|.
// Operand reads run RING reads ahead of their products, across phases.  K is consumed one block
// ahead of V, so a step has two barriers: X1 before the first product that reads the next buffer's
// K (then the K tiles of the step after next are issued into this buffer), X2 before the first
// product that reads the next buffer's V (then this buffer's V tiles are issued).  Each waits for
// exactly the loads the following blocks need, so the step after next stays in flight: K and V
// both get a whole step of lead.
// SMALLP: 8-key pages, where one 1 KB load block spans two pages.
template <int D, bool SMALLP>
__global__ void __launch_bounds__(2 * kRowsPerItem, 1) attn_bf16(AttnParams p) {
  constexpr int NC = D / 16;                 // 16-channel chunks of the QK product = PV products per block
  constexpr int ND = D / 32;                 // 32-channel blocks of O^T
  constexpr int UNITS = BN * D * 2 / 1024;   // 1 KB load blocks per tile, for K and for V each
  constexpr int NU = UNITS / 8;              // per wave
  constexpr int KROWS_U = 512 / D;           // K rows per block
  constexpr int TPS = RK_TILES_PER_STEP;
#ifndef RK_RING
#define RK_RING 4
#endif
  constexpr int RING = RK_RING;              // operand reads in flight ahead of their products
  constexpr int EPM = 8 / NC;                // exponentials per product slice of a phase
  static_assert(TPS == 2, "the block pipeline assumes two tiles per step");
  static_assert(NU >= 1 && UNITS % 8 == 0, "tile does not split over the waves");
  static_assert(NC >= RING && RING >= 2 && EPM * NC == 8, "phase slicing");
  __shared__ __attribute__((aligned(1024))) AttnBf16Smem<D, TPS> sm;

  const int tid = threadIdx.x;
  // the wave index is uniform: keep it (and everything derived from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, m = lane & 31;
  const ItemCtx ic = p.ictx[blockIdx.x];
  if (ic.kvh_cls < 0) return;  // schedule padding: keeps the next items on their XCD
  const int g = ic.kvh_cls & 0xffff;
  const int cls = ic.kvh_cls >> 16;
  const int tok_end = min(ic.tok0 + p.T, ic.n_q);
  const int L = ic.kv_len;
  const int i_max = ic.q_start + tok_end - 1;
  const TileRange tr = tile_range(cls, ic.q_start + ic.tok0, i_max, p.sink, p.window);
  // An odd tile count is padded with the tile after the item's last one: its keys lie past every
  // row, so the index masks zero its weights, and its pages are held (or replaced by the fallback
  // page below), so everything it loads is finite.  Every step then holds two tiles and the loop has
  // no partial step (a partial last step made the compiler keep two homes for the accumulators).
  const int ntiles = (tr.count() + 1) & ~1;
  const int nsteps = ntiles / TPS;
  const int32_t *__restrict__ pt = p.page_ids + ic.page_off;
  const bf16_t *__restrict__ kpg = static_cast<const bf16_t *>(p.k_pages);
  const bf16_t *__restrict__ vpg = static_cast<const bf16_t *>(p.v_pages);
  const int P = p.P, log2P = p.log2P;
  const int Pt = P < BN ? P : BN;
  const int n_logical = (L + P - 1) >> log2P;
  const uint32_t page_bytes = (uint32_t)(P * D * 2);
  // Pages a tile touches but the head does not hold (or past the sequence's last page) are read
  // from this page instead: the page of the item's last query, held and fully written (the append
  // clears its slots past kv_len).  Its keys are masked out, so only finiteness matters.
  const int pg_fallback = ic.fallback;

  // ---- the query row (column of S^T) this lane owns
  const int r = wave * 32 + m;
  const int hh = r / p.T;
  const int tq = ic.tok0 + (r - hh * p.T);
  const bool valid = hh < p.G && tq < tok_end;
  const int pos = valid ? ic.q_start + tq : -1;
  const int hq = g * p.G + hh;
  const int win_lo = cls == RK_GLOBAL ? 0 : pos - p.window + 1;  // first window key of the row
  // Wave-uniform query range, in scalar registers, so block classes are scalar branches.  When T is a
  // multiple of 32 (G in {1, 2, 4, 8}) the wave's rows are 32 consecutive tokens of one head and the
  // range is exact; otherwise the item's range, which contains the wave's rows (block classes only
  // decide whether a block is masked, so a wider range costs masking work, never correctness).
  int wmin, wmax;
  if ((p.T & 31) == 0) {
    const int t0 = ic.tok0 + (wave * 32) % p.T;
    wmin = t0 < tok_end ? ic.q_start + t0 : INT32_MAX;
    wmax = t0 < tok_end ? ic.q_start + min(t0 + 31, tok_end - 1) : -1;
  } else {
    wmin = ic.q_start + ic.tok0;
    wmax = i_max;
  }

  bf16x8 qf[NC];

  // Page ids of a step's tiles: one direct 4-byte-per-lane load per wave into the wave's LDS slot
  // of that step's buffer (lane x * npt + i: the id of page i of the step's x-th tile), issued a step
  // ahead and read back with one LDS read after the step's first barrier.  A vector-register result
  // would make the compiler wait for every load in flight before its first use; the LDS slot is
  // covered by the step's own wait.  Lanes past the step's pages, and pages past the sequence, read
  // the last logical page (held: it holds kv_len - 1), so every id is a held page or -1.
  const int npt = P < BN ? BN / P : 1;
  auto issue_ids = [&](int step, auto slotc) {
    constexpr int slot = decltype(slotc)::value;
    const int x = min(lane / npt, TPS - 1), i = lane % npt;
    const int lp = min(((tr.tile(step * TPS + x) * BN) >> log2P) + i, n_logical - 1);
    load_lds4_buf(pt, (uint32_t)lp * 4u, (uint32_t)n_logical * 4u, &sm.ids[wave][slot][0]);
  };
  // the first step's ids and the queries load while the tile geometry below is computed
  issue_ids(0, IntC<0>{});
  asm volatile("" ::: "memory");  // the query loads below stay behind the ids load
  {
    // every lane loads (rows outside the item read the item's first row and are zeroed), so exactly
    // NC query loads follow the ids load
    const int tq_c = valid ? tq : ic.tok0, hq_c = valid ? hq : g * p.G;
    const bf16_t *qrow = static_cast<const bf16_t *>(p.q) + ((int64_t)(ic.cu_q + tq_c) * p.H + hq_c) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const bf16x8 z = {}, v = *reinterpret_cast<const bf16x8 *>(qrow + 16 * c + 8 * hl);
      qf[c] = valid ? v : z;
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

  // the ids with the fallback page in place of -1 (one select per step instead of one per load)
  auto read_ids = [&](auto slotc) -> int {
    constexpr int slot = decltype(slotc)::value;
    const int v = sm.ids[wave][slot][lane];
    return v >= 0 ? v : pg_fallback;
  };
  // Byte address of a byte offset within physical page pg: ids are non-negative, so the page offset
  // is one unsigned 32 x 32 -> 64-bit product (two scalar instructions per load).
  auto page_at = [&](const bf16_t *pool, int pg, uint32_t off) {
    return reinterpret_cast<const char *>(pool) + ((uint64_t)(uint32_t)pg * page_bytes + off);
  };
  // K (V) loads of the step's x-th tile (key tile `tile`) into slot x of buffer buf
  auto issue_k_tile = [&](int tile, int buf, int x, int ids) {
    const int lane0 = x * npt;
    const uint32_t ko = P > BN ? (uint32_t)((tile * BN) & (P - 1)) * D * 2 : 0u;  // tiles within a large page
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int b = wave * NU + u;
      if constexpr (k_split) {
        const int pg = __shfl(ids, lane0 + (swap_bits23(b * KROWS_U + lane / (D / 8)) >> log2P));
        load_lds16(page_at(kpg, pg, ko) + k_loff[u], &sm.k[buf][x][b * 512]);
      } else {
        const int pg = __builtin_amdgcn_readlane(ids, lane0 + (P < BN ? (k_key0[u] >> log2P) : 0));
        load_lds16_buf(page_at(kpg, pg, ko), k_loff[u], page_bytes, &sm.k[buf][x][b * 512]);
      }
    }
  };
  auto issue_v_tile = [&](int tile, int buf, int x, int ids) {
    const int lane0 = x * npt;
    const uint32_t vo = P > BN ? (uint32_t)((tile * BN) & (P - 1)) * 2 : 0u;  // key offset within a large page
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int b = wave * NU + u;
      if constexpr (v_split) {
        const int pg = __shfl(ids, lane0 + v_pi[u]);
        load_lds16(page_at(vpg, pg, vo) + v_loff[u], &sm.v[buf][x][b * 512]);
      } else {
        const int pg = __builtin_amdgcn_readlane(ids, lane0 + v_pi[u]);
        load_lds16_buf(page_at(vpg, pg, vo), v_loff[u], page_bytes, &sm.v[buf][x][b * 512]);
      }
    }
  };
  auto issue_k = [&](int step, int buf, int ids) {
#pragma unroll
    for (int x = 0; x < TPS; ++x)
      if (step * TPS + x < ntiles) issue_k_tile(tr.tile(step * TPS + x), buf, x, ids);
  };
  auto issue_v = [&](int step, int buf, int ids) {
#pragma unroll
    for (int x = 0; x < TPS; ++x)
      if (step * TPS + x < ntiles) issue_v_tile(tr.tile(step * TPS + x), buf, x, ids);
  };

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = f32x16{};
  float mrun = kNegBig, lsum = 0.f;
  const float c2 = p.scale_log2;

  f32x16 sc[2];      // scores of the even / odd blocks (S^T: 16 keys of one query column per lane)
  u32x4 pk[2][2];    // their bf16 weights (bf16 pairs): the B operands of the two 16-key chunks of PV
  float psum[2];     // the row sum of the first half of their weights (this lane's keys)
  bf16x8 kr[RING], vr[RING];

  // ---- blocks: block q (0..3) of a step sits in tile q >> 1, half q & 1 of the step's buffer.
  // Operand reads address LDS as a lane byte offset plus an immediate: the K offsets start at the K
  // image, the V offsets at the V image, and every buffer, tile and channel-block displacement
  // (< 64 KB from either) is the immediate.  opaque() keeps the compiler from folding the images'
  // base into per-buffer copies of the lane offsets.
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  typedef __attribute__((address_space(3))) bf16x8 lds_v8;
  lds_u8 *const lds_k = (lds_u8 *)&sm.k[0][0][0];
  lds_u8 *const lds_v = (lds_u8 *)&sm.v[0][0][0];
  uint32_t kofs[NC], vofs[4];
#pragma unroll
  for (int c = 0; c < NC; ++c) kofs[c] = opaque((uint32_t)k_rd[c] * 2);
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) vofs[q4] = opaque((uint32_t)v_rd[q4] * 2);
  auto first_key = [&](int s, int q) { return tr.tile(s * TPS + (q >> 1)) * BN + 32 * (q & 1); };
  auto read_k = [&](auto bufc, auto qc, int c) {
    constexpr int buf = decltype(bufc)::value, q = decltype(qc)::value;
    constexpr uint32_t imm = ((buf * TPS + (q >> 1)) * BN * D + 32 * (q & 1) * D) * 2;
    return *(lds_v8 *)(lds_k + kofs[c] + imm);
  };
  // V^T operand i of block q: 16-key chunk cc = i / ND, 32-channel block db = i % ND
  auto read_v = [&](auto bufc, auto qc, int i) {
    constexpr int buf = decltype(bufc)::value, q = decltype(qc)::value;
    const uint32_t imm = ((buf * TPS + (q >> 1)) * BN * D + (i % ND) * 32 * BN) * 2;
    return *(lds_v8 *)(lds_v + vofs[2 * (q & 1) + i / ND] + imm);
  };
  // every key of the block visible to every row of the wave: no per-element work
  auto is_full = [&](int jb0) {
    return jb0 + 31 <= wmin && (cls == RK_GLOBAL || jb0 + 32 <= p.sink || jb0 > wmax - p.window);
  };
  // key of register i of the block: jb0 + 8 hl + 16 (i / 8) + i % 8.  The visible keys of the
  // lane's 32-key window [jb0 + 8 hl, + 32) form a bit mask (bit o: key jb0 + 8 hl + o): causal up to
  // the row, minus the gap between the sink and the window for LOCAL heads.  Each score is then kept
  // or set to -inf in place (in_place_mask), so the block's scores keep their registers.
  auto mask_block = [&](f32x16 &s, int jb0) {
    const int jb = jb0 + 8 * hl;
    const int hi = pos - jb;  // visible: o <= hi
    uint32_t vis = hi >= 31 ? 0xffffffffu : (hi < 0 ? 0u : (2u << hi) - 1u);
    if (cls != RK_GLOBAL) {
      // LOCAL: o >= win_lo - jb (window) or o < sink - jb (sink) -- clear [max(sk, 0), lo)
      const int lo = min(max(win_lo - jb, 0), 32), sk = min(max(p.sink - jb, 0), 32);
      const uint32_t below_lo = lo >= 32 ? 0xffffffffu : (1u << lo) - 1u;
      const uint32_t below_sk = sk >= 32 ? 0xffffffffu : (1u << sk) - 1u;
      vis &= ~below_lo | below_sk;
    }
    in_place_mask(s, vis);
  };
  auto weight = [&](float s) { return fast_exp2(fmaf(s, c2, -mrun)); };
  auto pack = [&](float a, float b) {
    const f32x2 t = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(t, bf16x2));
  };

  // Phase A(j): S(j+1) = K(j+1) Q^T beside the second-half weights of S(j); the last RING slices read
  // the first V operands of PV(j).  NEXT: block j+1 exists; KPRE: its first RING K operands are in kr.
  auto phase_a = [&](auto nextc, auto kprec, auto par, auto bc, auto qc, auto bn, auto qn) -> float {
    constexpr bool NEXT = decltype(nextc)::value, KPRE = decltype(kprec)::value;
    constexpr int PR = decltype(par)::value;
    if constexpr (NEXT && !KPRE) {
#pragma unroll
      for (int c = 0; c < RING; ++c) kr[c] = read_k(bn, qn, c);
    }
    if constexpr (NEXT) sc[PR ^ 1] = f32x16{};
    float ev = 0.f, s2[4];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (i >= NC - RING) vr[i - (NC - RING)] = read_v(bc, qc, i - (NC - RING));
      if constexpr (NEXT) {
        sc[PR ^ 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[i % RING], qf[i], sc[PR ^ 1], 0, 0, 0);
        if (i + RING < NC) kr[i % RING] = read_k(bn, qn, i + RING);
      }
#pragma unroll
      for (int u = 0; u < EPM; ++u) {
        const int k = i * EPM + u;
        const float w = weight(sc[PR][8 + k]);
        if (k & 1) {
          pk[PR][1][k >> 1] = pack(ev, w);
          s2[k >> 1] = ev + w;
        } else {
          ev = w;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return (s2[0] + s2[1]) + (s2[2] + s2[3]);
  };
  // Phase B(j): O^T += V(j)^T P(j)^T beside the first-half weights of S(j+1); the last RING slices
  // read the first K operands of block j+2 (KPRE2) from buffer b2.
  auto phase_b = [&](auto nextc, auto kpre2c, auto par, auto bc, auto qc, auto b2, auto q2) {
    constexpr bool NEXT = decltype(nextc)::value, KPRE2 = decltype(kpre2c)::value;
    constexpr int PR = decltype(par)::value;
    float ev = 0.f, s2[4];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      oacc[i % ND] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[i % RING], __builtin_bit_cast(bf16x8, pk[PR][i / ND]),
                                                            oacc[i % ND], 0, 0, 0);
      if (i + RING < NC) vr[i % RING] = read_v(bc, qc, i + RING);
      if constexpr (KPRE2) {
        if (i >= NC - RING) kr[i - (NC - RING)] = read_k(b2, q2, i - (NC - RING));
      }
      if constexpr (NEXT) {
#pragma unroll
        for (int u = 0; u < EPM; ++u) {
          const int k = i * EPM + u;
          const float w = weight(sc[PR ^ 1][k]);
          if (k & 1) {
            pk[PR ^ 1][0][k >> 1] = pack(ev, w);
            s2[k >> 1] = ev + w;
          } else {
            ev = w;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (NEXT) psum[PR ^ 1] = (s2[0] + s2[1]) + (s2[2] + s2[3]);
  };
  // After phase A(j): accept block j's weights, or (rare) rescale to its true row max and redo them.
  auto settle = [&](auto par, float sum2) {
    constexpr int PR = decltype(par)::value;
    float tot = psum[PR] + sum2;
    if (__any(tot > kRescaleAt)) {
      float mt = sc[PR][0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sc[PR][i]);
      const float mnew = fmaxf(mrun, halves_max(mt) * c2);
      const float alpha = fast_exp2(mrun - mnew);
      mfma_result_wait();  // one wait for all tuples: the products that write them were issued before
#pragma unroll
      for (int db = 0; db < ND; ++db) in_place_scale_ready(oacc[db], alpha);
      lsum *= alpha;
      mrun = mnew;
      tot = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float w0 = weight(sc[PR][i]), w1 = weight(sc[PR][i + 1]);
        const float w2 = weight(sc[PR][8 + i]), w3 = weight(sc[PR][9 + i]);
        tot += (w0 + w1) + (w2 + w3);
        pk[PR][0][i >> 1] = pack(w0, w1);
        pk[PR][1][i >> 1] = pack(w2, w3);
      }
    }
    lsum += tot;
  };

  // Loads retire in issue order.  Prologue: the ids and tiles of step 0; after the barrier K(1),
  // the ids of step 2, V(1).  Then X1 of step s issues K(s + 2), X2 the ids of step s + 3 and
  // V(s + 2): every wait below names exactly the loads that may stay in flight.
  constexpr int NLD = NU * TPS;  // loads of one step's K (or V) per wave
  wait_vmcnt<NC>();  // the ids; the queries may still be in flight
  int idv = read_ids(IntC<0>{});
  issue_k(0, 0, idv);
  issue_v(0, 0, idv);
  if (nsteps > 1) issue_ids(1, IntC<1>{});
  wait_vmcnt<0>();
  __syncthreads();
  if (nsteps > 1) {
    idv = read_ids(IntC<1>{});
    issue_k(1, 1, idv);
    if (nsteps > 2) issue_ids(2, IntC<0>{});
    issue_v(1, 1, idv);
  }
  // block 0: its scores alone, then the first half of its weights
  {
    sc[0] = f32x16{};
#pragma unroll
    for (int c = 0; c < RING; ++c) kr[c] = read_k(IntC<0>{}, IntC<0>{}, c);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[i % RING], qf[i], sc[0], 0, 0, 0);
      if (i + RING < NC) kr[i % RING] = read_k(IntC<0>{}, IntC<0>{}, i + RING);
    }
#pragma unroll
    for (int c = 0; c < RING; ++c) kr[c] = read_k(IntC<0>{}, IntC<1>{}, c);
    const int jb0 = first_key(0, 0);
    if (!is_full(jb0)) mask_block(sc[0], jb0);
    // the running max starts at this block's row max, so the block needs no rescale; a row with no
    // visible key here keeps -1e30, and its first visible block takes the rescale path
    float mt = sc[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mt = fmaxf(mt, sc[0][i]);
    mrun = fmaxf(halves_max(mt) * c2, kNegBig);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float w0 = weight(sc[0][i]), w1 = weight(sc[0][i + 1]);
      sum += w0 + w1;
      pk[0][0][i >> 1] = pack(w0, w1);
    }
    psum[0] = sum;
  }

  const IntC<0> c0{};
  const IntC<1> c1{};
  const IntC<2> c2i{};
  const IntC<3> c3i{};
  const IntC<true> yes{};
  const IntC<false> no{};
  // One step: blocks 0..3 of buffer b.  After the item's last block the pipeline still runs the
  // scores of one more block, on whatever the other buffer holds (in bounds, no load in flight into
  // it), and never uses them: NC products per item instead of a second copy of the pipeline's tail.
  auto step = [&](const int s, auto bufc) __attribute__((always_inline)) {
    constexpr int b = decltype(bufc)::value;
    const IntC<b ^ 1> bn{};
    const bool last = s + 1 >= nsteps;
    settle(c0, phase_a(yes, yes, c0, bufc, c0, bufc, c1));
    if (!is_full(first_key(s, 1))) mask_block(sc[1], first_key(s, 1));
    phase_b(yes, yes, c0, bufc, c0, bufc, c2i);
    settle(c1, phase_a(yes, yes, c1, bufc, c1, bufc, c2i));
    if (!is_full(first_key(s, 2))) mask_block(sc[0], first_key(s, 2));
    phase_b(yes, yes, c1, bufc, c1, bufc, c3i);
    settle(c0, phase_a(yes, yes, c0, bufc, c2i, bufc, c3i));
    if (!is_full(first_key(s, 3))) mask_block(sc[1], first_key(s, 3));
    phase_b(yes, no, c0, bufc, c2i, bufc, c0);
    // X1: the next step's K is in LDS and every wave is done with this buffer's K.  In flight after
    // K(s + 1) and the ids of step s + 2: V(s + 1).
    if (!last) {
      wait_vmcnt<NLD>();
      lds_barrier();
      idv = read_ids(bufc);
      if (s + 2 < nsteps) issue_k(s + 2, b, idv);
    }
    // block 3; its successor is block 0 of the next step
    settle(c1, phase_a(yes, no, c1, bufc, c3i, bn, c0));
    if (!last && !is_full(first_key(s + 1, 0))) mask_block(sc[0], first_key(s + 1, 0));
    phase_b(yes, yes, c1, bufc, c3i, bn, c1);
    // X2: the next step's V is in LDS and every wave is done with this buffer's V.  In flight after
    // V(s + 1): K(s + 2), when it exists.
    if (!last) {
      if (s + 2 < nsteps) wait_vmcnt<NLD>();
      else wait_vmcnt<0>();
      lds_barrier();
      if (s + 2 < nsteps) {
        if (s + 3 < nsteps) issue_ids(s + 3, bn);
        issue_v(s + 2, b, idv);
      }
    }
  };
  for (int s = 0; s < nsteps; s += 2) {
    step(s, c0);
    if (s + 1 < nsteps) step(s + 1, c1);
  }

  // ---- epilogue: O^T accumulator (lane column = query, 16 channels per 32-channel block).  The
  // normalised rows go through LDS (the K image, free once every wave is past its last block), so
  // each global store writes whole 16-byte chunks of D / 8 lanes per row: D / 8 rows per instruction
  // instead of 32 rows with 8 bytes per lane.
  const float lt = halves_sum(lsum);
  const float inv = 1.0f / lt;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;              // rows per store instruction
  typedef __attribute__((address_space(3))) bf16x4 lds_b4;
  typedef __attribute__((address_space(3))) int64_t lds_i64;
  lds_u8 *const stage = lds_k + wave * 32 * D * 2;
  lds_i64 *const rowoff = (lds_i64 *)&sm.ids[wave][0][0];
  lds_barrier();
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      f32x4 w = {oacc[db][4 * a4 + 0] * inv, oacc[db][4 * a4 + 1] * inv, oacc[db][4 * a4 + 2] * inv,
                 oacc[db][4 * a4 + 3] * inv};
      const int c = 4 * db + a4;
      *(lds_b4 *)(stage + m * D * 2 + ((c ^ (m & (CPR - 1))) << 4) + 8 * hl) = __builtin_convertvector(w, bf16x4);
    }
  if (hl == 0) rowoff[m] = valid ? ((int64_t)(ic.cu_q + tq) * p.H + hq) * D : (int64_t)-1;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  bf16_t *const obase = static_cast<bf16_t *>(p.o);
  const int cl = lane % CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int rr = RPI * i + lane / CPR;
    const bf16x8 v = *(lds_v8 *)(stage + rr * D * 2 + ((cl ^ (rr & (CPR - 1))) << 4));
    const int64_t off = rowoff[rr];
    if (off >= 0) *reinterpret_cast<bf16x8 *>(obase + off + 8 * cl) = v;
  }
  if (p.lse && valid && hl == 0)
    p.lse[(int64_t)hq * p.total_q + ic.cu_q + tq] = (mrun + log2f(lt)) * 0.69314718055994531f;
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
