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

constexpr int kAttnWaves = 8;                 // 2 waves per SIMD: one wave's softmax overlaps the other's MFMA
constexpr int kAttnThreads = 64 * kAttnWaves;
static_assert(kAttnWaves * 32 == kRowsPerItem, "one 32-query column block per wave");

template <int D>
struct AttnBf16Smem {
  static constexpr int KP = D + 8;   // K row pitch (elements): +16 bytes spreads rows over all banks
  static constexpr int VP = BN + 8;  // V^T row pitch (elements), same reason
  bf16_t k[2][BN * KP];
  bf16_t v[2][D * VP];
};

// max / sum of a value over the two half-waves (lanes l and l ^ 32)
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ void __launch_bounds__(kAttnThreads, 1) attn_bf16(AttnParams p) {
  constexpr int KP = AttnBf16Smem<D>::KP;
  constexpr int VP = AttnBf16Smem<D>::VP;
  constexpr int NC = D / 16;                       // 16-channel chunks of the QK product
  constexpr int ND = D / 32;                       // 32-channel blocks of O^T
  constexpr int NLD = BN * D / 8 / kAttnThreads;   // 16-byte chunks per thread per tile (K and V each)
  constexpr int ROWS_PER_WAVE_LD = 64 * 8 / D;     // K rows one wave-wide chunk load covers
  static_assert(NLD >= 1, "tile too small for the workgroup");
  __shared__ __attribute__((aligned(16))) AttnBf16Smem<D> sm;

  const int tid = threadIdx.x;
  // the wave index is uniform: keep it (and everything derived from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, m = lane & 31;
  const Item it = p.items[blockIdx.x];
  const SeqInfo si = p.seqs[it.seq];
  const int g = it.kv_head;
  const int cls = p.head_class[g];
  const int tok_end = min(it.tok0 + p.T, si.n_q);
  const int L = si.kv_len;
  const TileRange tr = tile_range(cls, si.q_start + it.tok0, si.q_start + tok_end - 1, p.sink, p.window);
  const int ntiles = tr.count();
  const int32_t *__restrict__ pt = p.page_ids + p.page_base[g * p.num_seqs + it.seq];
  const bf16_t *__restrict__ kpg = static_cast<const bf16_t *>(p.k_pages);
  const bf16_t *__restrict__ vpg = static_cast<const bf16_t *>(p.v_pages);
  const int P = p.P, log2P = p.log2P;
  const int n_logical = (L + P - 1) >> log2P;
  const int64_t page_elems = (int64_t)P * D;

  // ---- the query row (column of S^T) this lane owns
  const int r = wave * 32 + m;
  const int hh = r / p.T;
  const int tq = it.tok0 + (r - hh * p.T);
  const bool valid = hh < p.G && tq < tok_end;
  const int pos = valid ? si.q_start + tq : -1;
  const int hq = g * p.G + hh;
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

  // ---- tile-invariant geometry of this thread's 16-byte chunks.  Chunk u of a wave covers a
  // contiguous kilobyte of one page: a scalar page base plus lane * 16 bytes.
  int k_lds[NLD], v_lds[NLD], v_key[NLD];
  int k_row0[NLD], v_pi[NLD], v_goff0[NLD];  // wave-uniform parts
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int c = tid + kAttnThreads * u;
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    k_lds[u] = swap_bits23(row) * KP + col;
    k_row0[u] = (wave * 64 + kAttnThreads * u) / (D / 8);
    int d, kof;
    if (P <= BN) {
      const int per_page = D * P / 8;
      const int pi = c / per_page;
      const int idx = c - pi * per_page;
      d = idx / (P / 8);
      kof = pi * P + (idx - d * (P / 8)) * 8;
      v_pi[u] = (wave * 64 + kAttnThreads * u) / per_page;  // == pi: a wave's 64 chunks share one page
      v_goff0[u] = ((wave * 64 + kAttnThreads * u) - v_pi[u] * per_page) * 8;  // + lane * 8
    } else {
      d = c >> 3;
      kof = (c & 7) * 8;
      v_pi[u] = 0;
      v_goff0[u] = ((wave * 64 + kAttnThreads * u) >> 3) * P;  // + (lane >> 3) * P + (lane & 7) * 8
    }
    v_key[u] = kof;
    v_lds[u] = d * VP + kof;
  }
  const int v_lane_off = P <= BN ? lane * 8 : (lane >> 3) * P + (lane & 7) * 8;

  u32x4 kr[NLD], vr[NLD];
  auto load_tile = [&](int tile) {
    const int j0 = tile * BN;
    const bool tail = j0 + BN > L;
    // page ids first (scalar loads, all in flight together), then the 16-byte data loads
    int pgk[NLD], pgv[NLD];
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int lk = (j0 + k_row0[u]) >> log2P;
      const int lv = (j0 >> log2P) + v_pi[u];
      pgk[u] = lk < n_logical ? pt[lk] : -1;
      pgv[u] = lv < n_logical ? pt[lv] : -1;
    }
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      const int jw = j0 + k_row0[u];  // first key of the wave's kilobyte
      u32x4 val = {0u, 0u, 0u, 0u};
      const bf16_t *src = kpg + (int64_t)pgk[u] * page_elems + (int64_t)(jw & (P - 1)) * D + lane * 8;
      if (pgk[u] >= 0 && (!tail || jw + lane / (D / 8) < L)) val = *reinterpret_cast<const u32x4 *>(src);
      kr[u] = val;
    }
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      u32x4 val = {0u, 0u, 0u, 0u};
      const bf16_t *src =
          vpg + (int64_t)pgv[u] * page_elems + v_goff0[u] + (P > BN ? (j0 & (P - 1)) : 0) + v_lane_off;
      const int j = j0 + v_key[u];
      if (pgv[u] >= 0 && (!tail || j < L)) {
        val = *reinterpret_cast<const u32x4 *>(src);
        if (tail && j + 8 > L) val = keep_first_bf16(val, L - j);
      }
      vr[u] = val;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NLD; ++u) {
      *reinterpret_cast<u32x4 *>(&sm.k[buf][k_lds[u]]) = kr[u];
      *reinterpret_cast<u32x4 *>(&sm.v[buf][v_lds[u]]) = vr[u];
    }
  };

  f32x16 oacc[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) oacc[db] = f32x16{};
  float mrun = kNegBig, lsum = 0.f;
  const float c2 = p.scale_log2;
  const int win_lo = cls == RK_GLOBAL ? 0 : pos - p.window + 1;  // first window key of this row

  load_tile(tr.tile(0));
  store_tile(0);
  __syncthreads();

  for (int idx = 0; idx < ntiles; ++idx) {
    const int buf = idx & 1;
    const bool more = idx + 1 < ntiles;
    if (more) load_tile(tr.tile(idx + 1));
    const int j0 = tr.tile(idx) * BN;
    const bool skip = wmax < 0 || j0 > wmax ||
                      (cls == RK_LOCAL && j0 >= p.sink && j0 + BN - 1 <= wmin - p.window);
    const bool full = j0 + BN - 1 <= wmin &&
                      (cls == RK_GLOBAL || j0 + BN <= p.sink || j0 > wmax - p.window);
    if (!skip) {
      const bf16_t *Kb = sm.k[buf];
      const bf16_t *Vb = sm.v[buf];
      // S^T for the tile's 64 keys (two 32-key blocks) x this wave's 32 queries
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(Kb + (32 * kb + m) * KP + 16 * c + 8 * hl);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[kb], 0, 0, 0);
        }
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
      const float mts = mt * c2;
      if (__any(mts > mrun + kRescaleSlack)) {
        const float mnew = fmaxf(mrun, mts);
        const float alpha = fast_exp2(mrun - mnew);
#pragma unroll
        for (int db = 0; db < ND; ++db) oacc[db] *= alpha;
        lsum *= alpha;
        mrun = mnew;
      }
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
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int db = 0; db < ND; ++db) {
            const bf16x8 a =
                *reinterpret_cast<const bf16x8 *>(Vb + (32 * db + m) * VP + 32 * kb + 16 * cc + 8 * hl);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kb][cc], oacc[db], 0, 0, 0);
          }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
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
    if (head_dim == 128)
      hipLaunchKernelGGL(attn_bf16<128>, grid, dim3(kAttnThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(attn_bf16<64>, grid, dim3(kAttnThreads), 0, stream, p);
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
