// gfx950 (CDNA4) kernel of the per-key attention mass: for each q head h and key j of a sequence,
// the sum over the call's queries i of head h of the attention weight p_ij = exp(scale q_i.k_j -
// lse_i) over visible pairs.  It is the routing signal of the pages' sparse FFN: the dense FFN runs
// only on the top-k tokens by attention score, the rest take the residual path (page "小红书把 KV
// Cache 按「头」拆了…" (zhichai.net), section 事件内容, item 2; page "RedKnot – 小红书研发并开源的
// 长上下文大模型推理引擎" (shshi.cn), section RedKnot技术原理, 3).
//
// Design: key-stationary, so that every output is written once (a query-stationary pass would need
// one global atomic per (head, key, query tile)).  A workgroup owns 8 KPW keys of one (sequence, KV
// head); each of its eight waves holds the K fragments of KPW keys in registers (KPW = 64 when G <= 8,
// else 32).  It steps over the call's query tokens in steps of 256 rows (G heads x T tokens, T the
// largest multiple of 16 with G T <= 256): the rows are staged in LDS by direct 16-byte global->LDS
// loads (double-buffered, XOR-swizzled as in the attention kernel), with lse * log2(e) beside them.
// S = Q K^T runs on v_mfma_f32_32x32x16_bf16 with keys as the N dimension, so each lane owns one key
// and sums its weights over the 16 query rows it holds; the two half-waves are combined with
// v_permlane32_swap.  Each lane keeps one running total per (32-row block, key set) in registers over
// all steps (a block's rows belong to the same head on every step), so the step loop does no LDS
// writes besides the staged rows: an LDS add there would wait for the next step's direct loads, as
// the compiler cannot tell their LDS area apart.  At the end the totals go to per-(head, key) LDS sums
// (ds_add_f32), which the workgroup adds to the zero-filled output (one global atomic per (head, key,
// query chunk)).
// Rows outside the call (past kv_len, or of a LOCAL head below its start) read a valid row and get
// lse = +inf, so their weight is exactly 0; the visibility mask (causal, sink, window) comes from
// indices, on edge blocks only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rk_device.h"
#include "rk_ops.h"
#include "rk_seg.h"

#include <algorithm>

namespace rk {
namespace {

template <int D>
struct MassSmem {
  bf16_t q[2][kRowsPerItem * D];
  float lse2[2][kRowsPerItem];
  float acc[kMassAccFloats];  // [head][key of the workgroup]
};

// KPW keys per wave (64 when G <= 8, else 32, so that G x 8 KPW sums fit kMassAccFloats).
template <int D, int KPW>
__global__ void __launch_bounds__(512, 1) key_mass_bf16(MassParams p) {
  constexpr int NC = D / 16;                                // 16-channel chunks of the QK product
  constexpr int NS = KPW / 32;                              // 32-key sets per wave
  constexpr int KEYS = 8 * KPW;                             // keys per workgroup
  constexpr int ROWS_U = 512 / D;                           // Q rows per 1 KB load block
  constexpr int NU = kRowsPerItem * D * 2 / 1024 / 8;       // load blocks per wave and step
  constexpr int NRB = kRowsPerItem / 32;                    // 32-row MFMA blocks per step
  constexpr float kLog2e = 1.4426950408889634f;
  static_assert(KEYS * (256 / (16 * (KPW == 64 ? 2 : 1))) <= kMassAccFloats, "LDS sums");
  __shared__ __attribute__((aligned(1024))) MassSmem<D> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hl = lane >> 5, m = lane & 31;
  // work unit (seq, kv head, key block, query chunk) from the host's list, which places runs of
  // key blocks reading the same query rows on one XCD (workgroup i runs on XCD i % 8)
  const MassUnit u = p.units[blockIdx.x];
  if (u.seq < 0) return;  // schedule padding
  const int b = u.seq, g = u.kv_head;
  const SeqInfo si = p.seqs[b];
  const int L = si.kv_len;
  const int j0 = u.kblk * KEYS;
  const bool global = p.head_class[g] == RK_GLOBAL;
  const int start = global ? si.q_start : si.q_start_local;
  const int G = p.G, T = p.T, W = p.window, SK = p.sink;

  // query tokens that can see a key of this block: from max(j0, start); a LOCAL block past the
  // sink is seen only by the window after its last key.  Steps run on a token grid of T tokens
  // from the class start; query chunk qc takes grid steps [qc S, qc S + S - 1].
  const int t_first = max(j0, start);
  int t_last = L - 1;
  if (!global && j0 >= SK) t_last = min(t_last, j0 + KEYS - 1 + W - 1);
  if (t_first > t_last) return;  // no query sees this block
  const int S = p.steps_per_chunk;
  const int k_first = max((t_first - start) / T, u.qc * S), k_last = min((t_last - start) / T, u.qc * S + S - 1);
  if (k_first > k_last) return;
  const int nsteps = k_last - k_first + 1;
  for (int i = tid; i < G * KEYS; i += 512) sm.acc[i] = 0.f;

  // K fragments of this wave's keys (B operand: key = lane % 32, channels 16 c + 8 hl .. + 7);
  // a key past kv_len or on a page the head does not hold is never visible: zeros
  const int kw = j0 + KPW * wave;
  bf16x8 kf[NS][NC];
  {
    const int32_t *pt = p.page_ids + p.page_base[g * p.num_seqs + b];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int key = kw + 32 * st + m;
      const int pg = key < L ? pt[key >> p.log2P] : -1;
      const bf16_t *row = static_cast<const bf16_t *>(p.k_pages) + ((int64_t)max(pg, 0) * p.P + (key & (p.P - 1))) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        bf16x8 z = {};
        kf[st][c] = pg >= 0 ? *reinterpret_cast<const bf16x8 *>(row + 16 * c + 8 * hl) : z;
      }
    }
  }

  // Staged row r = h T + tq of a step starting at token ts: token ts + tq of q head g G + h.  Rows
  // past the group (h >= G) or past t_last read a valid row of the step and get lse = +inf, so
  // their weight is exactly 0.  Byte offset of this lane's 16-byte chunk of load block u from the
  // step's first token, with tokens past tq_max replaced by the step's first token:
  const int64_t tok_bytes = (int64_t)p.H * D * 2;
  auto lane_off = [&](int uu, int tq_max) -> uint32_t {
    const int r = (wave * NU + uu) * ROWS_U + lane / (D / 8);
    const int ch = (lane % (D / 8)) ^ kswz<D>(r);
    const int h = r / T, tq = r - h * T;
    const bool ok = h < G && tq <= tq_max;
    return (uint32_t)((((ok ? tq * p.H : 0) + g * G + (ok ? h : 0)) * D + ch * 8) * 2);
  };
  uint32_t qoff[NU];
#pragma unroll
  for (int uu = 0; uu < NU; ++uu) qoff[uu] = lane_off(uu, INT32_MAX);
  const char *qbytes = static_cast<const char *>(p.q);
  auto stage_q = [&](int s, int buf) {
    const int ts = start + (k_last - s) * T;
    const int lim = t_last - ts;  // last valid tq of the step
    const char *base = qbytes + (int64_t)(si.cu_q + ts - si.q_start) * tok_bytes;  // uniform
    if (lim >= T - 1) {
#pragma unroll
      for (int uu = 0; uu < NU; ++uu) load_lds16(base + opaque(qoff[uu]), &sm.q[buf][(wave * NU + uu) * 512]);
    } else {  // the step past t_last (at most the first one)
#pragma unroll
      for (int uu = 0; uu < NU; ++uu) load_lds16(base + lane_off(uu, lim), &sm.q[buf][(wave * NU + uu) * 512]);
    }
  };
  // thread tid < kRowsPerItem stages row tid's lse x log2(e): loaded into a register with the
  // step's Q, written to LDS after the current step's compute (no wait in the prefetch)
  int l_tq = INT32_MAX;
  const float *lsep = p.lse;
  if (tid < kRowsPerItem) {
    const int h = tid / T, tq = tid - h * T;
    if (h < G) {
      l_tq = tq;
      lsep = p.lse + (int64_t)(g * G + h) * p.total_q + (si.cu_q - si.q_start) + tq;
    }
  }
  float lreg = INFINITY;
  auto lse_issue = [&](int s) {
    const int ts = start + (k_last - s) * T;
    lreg = l_tq <= t_last - ts ? lsep[ts] : INFINITY;
  };
  auto lse_store = [&](int buf) {
    if (tid < kRowsPerItem) sm.lse2[buf][tid] = lreg * kLog2e;
  };

  // head of 16-row half k of a step (the rows of a head are whole halves): bit k of hstart is set
  // where a head begins, so head(k) = popcount of bits 0..k, minus one
  uint32_t hstart = 0;
  for (int k = 0; k < 2 * NRB; k += T / 16) hstart |= 1u << k;
  auto head_of = [&](int k) { return (int)__builtin_popcount(hstart & ((2u << k) - 1u)) - 1; };

  const float c2 = p.scale_log2;
  // per-lane totals of each (MFMA block, key set) over all steps: added to the LDS sums once, at the end
  float accr[NRB][NS];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int st = 0; st < NS; ++st) accr[rb][st] = 0.f;
  // Weights of MFMA block (rb, key set st), summed per head: register i holds row rb 32 + 8 (i / 4)
  // + 4 hl + i % 4 of this lane's key, i < 8 in half 2 rb, i >= 8 in half 2 rb + 1.  Lane m gets
  // the first half's total over both lane halves, lane m + 32 the second's; both add to LDS.
  auto reduce = [&](int rb, int st, const f32x16 &sacc, const f32x4 *lv, bool full, int ts) {
    const int h0 = head_of(2 * rb), h1 = head_of(2 * rb + 1);
    float lo = 0.f, hi = 0.f;
    if (full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float w = fast_exp2(fmaf(sacc[i], c2, -lv[i / 4][i % 4]));
        if (i < 8) lo += w;
        else hi += w;
      }
    } else {
      // visible: 0 <= pos - key, and pos - key < W unless the head is GLOBAL or the key a sink key,
      // with pos = ts + tq0 + 4 hl + c_i (tq0: the half's first tq, c_i = 8 ((i % 8) / 4) + i % 4);
      // one unsigned compare of pos - key against the limit
      const int key = kw + 32 * st + m;
      const uint32_t lim = global || key < SK ? 0x80000000u : (uint32_t)W;
      const int e0 = ts + (32 * rb - h0 * T) + 4 * hl - key;
      const int e1 = ts + (32 * rb + 16 - h1 * T) + 4 * hl - key;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ci = 8 * ((i % 8) / 4) + i % 4;
        const bool vis = (uint32_t)(ci + (i < 8 ? e0 : e1)) < lim;
        const float w = fast_exp2(fmaf(sacc[i], c2, -lv[i / 4][i % 4]));
        if (i < 8) lo += vis ? w : 0.f;
        else hi += vis ? w : 0.f;
      }
    }
    // after the swap, r[0] + r[1] is lo of both lane halves on lanes < 32, hi of both on the rest
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    accr[rb][st] += __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };

  // Two key sets per wave, every pair of the step visible (the common case: a wave's 64 keys straddle
  // the causal diagonal or a window edge on a few steps only): a software pipeline over the row
  // blocks in which every MFMA chain runs beside the weight work of the other chain --
  //   phase A of block rb: set 1's MFMAs of rb, beside set 0's weights of rb;
  //   phase B of block rb: set 0's MFMAs of rb + 1, beside set 1's weights of rb --
  // one MFMA, then a slice of the weights, fenced so that the compiler keeps the order.  The Q
  // fragments of rb + 1 are loaded into a[c] once the last MFMA reading a[c] is issued, the lse of
  // rb + 1 into lv[q] once no weight needs lv[q], so that the pipeline takes no extra registers.
  auto compute_pipe = [&](int buf) {
    constexpr int EP = 16 / NC;  // weights (of this lane's 16) formed after each MFMA of a chain
    const bf16_t *Qb = sm.q[buf];
    const float *l2 = sm.lse2[buf];
    auto qfrag = [&](int rb, int c) {
      const int qr = rb * 32 + m;
      return *reinterpret_cast<const bf16x8 *>(Qb + qr * D + (((2 * c + hl) ^ kswz<D>(qr)) << 3));
    };
    auto lvec = [&](int rb, int q4) { return *reinterpret_cast<const f32x4 *>(l2 + rb * 32 + 8 * q4 + 4 * hl); };
    bf16x8 a[NC];
    f32x4 lv[4];
    float lo = 0.f, hi = 0.f;
    auto piece = [&](const f32x16 &acc, int c) {
#pragma unroll
      for (int k = 0; k < EP; ++k) {
        const int i = c * EP + k;
        const float w = fast_exp2(fmaf(acc[i], c2, -lv[i / 4][i % 4]));
        if (i < 8) lo += w;
        else hi += w;
      }
    };
    auto finish = [&](int rb, int st) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
      accr[rb][st] += __uint_as_float(r[0]) + __uint_as_float(r[1]);
      lo = hi = 0.f;
    };
#pragma unroll
    for (int c = 0; c < NC; ++c) a[c] = qfrag(0, c);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) lv[q4] = lvec(0, q4);
    f32x16 s0 = {}, s1;
#pragma unroll
    for (int c = 0; c < NC; ++c) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], kf[0][c], s0, 0, 0, 0);
    auto block = [&](const int rb) __attribute__((always_inline)) {
      s1 = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {  // phase A
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], kf[NS - 1][c], s1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        piece(s0, c);
        if (rb + 1 < NRB) a[c] = qfrag(rb + 1, c);
        __builtin_amdgcn_sched_barrier(0);
      }
      finish(rb, 0);
      if (rb + 1 < NRB) {
        s0 = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {  // phase B
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], kf[0][c], s0, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          piece(s1, c);
          if ((c * EP + EP) % 4 == 0) lv[(c * EP) / 4] = lvec(rb + 1, (c * EP) / 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) piece(s1, c);
      }
      finish(rb, 1);
    };
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) block(rb);
  };

  auto compute = [&](int s, int buf) {
    const int ts = start + (k_last - s) * T;
    const int tmax = min(ts + T - 1, t_last);
    // per key set: some pair of the step visible / every pair visible
    bool any = false;
    bool vis[NS], full[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int kmin = kw + 32 * st, kmax = kmin + 31;
      vis[st] = kmin <= tmax && (global || kmin < SK || kmax > ts - W);
      any = any || vis[st];
      full[st] = kmax <= ts && (global || kmax < SK || kmin > tmax - W);
    }
    if (!any) return;  // no row of the step sees a key of this wave
    if (NS == 2 && full[0] && full[NS - 1]) {  // the common case: both sets fully visible
      compute_pipe(buf);
      return;
    }
    const bf16_t *Qb = sm.q[buf];
    const float *l2 = sm.lse2[buf];
    // one key set with no visible pair in the step (on the causal diagonal or the window edge): only
    // the other set's products and weights
    auto one_set = [&](auto stc) __attribute__((always_inline)) {
      constexpr int st = decltype(stc)::value;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        bf16x8 a[NC];
        const int qr = rb * 32 + m;
#pragma unroll
        for (int c = 0; c < NC; ++c) a[c] = *reinterpret_cast<const bf16x8 *>(Qb + qr * D + (((2 * c + hl) ^ kswz<D>(qr)) << 3));
        f32x16 sacc = {};
#pragma unroll
        for (int c = 0; c < NC; ++c) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], kf[st][c], sacc, 0, 0, 0);
        f32x4 lv[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) lv[q4] = *reinterpret_cast<const f32x4 *>(l2 + rb * 32 + 8 * q4 + 4 * hl);
        reduce(rb, st, sacc, lv, full[st], ts);
      }
    };
    if (NS == 2 && !vis[NS - 1]) {
      one_set(IntC<0>{});
      return;
    }
    if (NS == 2 && !vis[0]) {
      one_set(IntC<NS - 1>{});
      return;
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      bf16x8 a[NC];
      const int qr = rb * 32 + m;
#pragma unroll
      for (int c = 0; c < NC; ++c) a[c] = *reinterpret_cast<const bf16x8 *>(Qb + qr * D + (((2 * c + hl) ^ kswz<D>(qr)) << 3));
      f32x16 sacc[NS];
#pragma unroll
      for (int st = 0; st < NS; ++st) sacc[st] = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int st = 0; st < NS; ++st) sacc[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], kf[st][c], sacc[st], 0, 0, 0);
      f32x4 lv[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) lv[q4] = *reinterpret_cast<const f32x4 *>(l2 + rb * 32 + 8 * q4 + 4 * hl);
#pragma unroll
      for (int st = 0; st < NS; ++st) reduce(rb, st, sacc[st], lv, full[st], ts);
    }
  };

  stage_q(0, 0);
  lse_issue(0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  lse_store(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nsteps;
    if (more) {
      stage_q(s + 1, buf ^ 1);
      lse_issue(s + 1);
    }
    compute(s, buf);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    if (more) lse_store(buf ^ 1);
    __syncthreads();
  }
  // the lane totals into the per-(head, key) sums
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int h = hl ? head_of(2 * rb + 1) : head_of(2 * rb);
#pragma unroll
    for (int st = 0; st < NS; ++st) atomicAdd(&sm.acc[h * KEYS + KPW * wave + 32 * st + m], accr[rb][st]);
  }
  __syncthreads();
  // partial sums of this query chunk: added to the zero-filled output
  for (int i = tid; i < G * KEYS; i += 512) {
    const int h = i / KEYS, kk = i - h * KEYS;
    if (j0 + kk < L) atomicAdd(&p.mass[(int64_t)(g * G + h) * p.total_kv + si.kv_off + j0 + kk], sm.acc[i]);
  }
}

__global__ void __launch_bounds__(256) fill_zero(float *x, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) x[i] = 0.f;
}

}  // namespace

hipError_t launch_key_mass(const MassParams &p, int head_dim, hipStream_t stream) {
  // every output entry is written: zero first (keys no query sees, also when the call has no query
  // row at all), then the units add their partial sums
  const int64_t n_out = (int64_t)p.H * p.total_kv;
  if (n_out > 0)
    hipLaunchKernelGGL(fill_zero, dim3((unsigned)std::min<int64_t>((n_out + 255) / 256, 1 << 16)), dim3(256), 0, stream,
                       p.mass, n_out);
  if (p.n_units <= 0) return hipGetLastError();
  const dim3 grid((unsigned)p.n_units);
  const bool wide = mass_keys_per_wave(p.G) == 64;
  if (head_dim == 128) {
    if (wide) hipLaunchKernelGGL((key_mass_bf16<128, 64>), grid, dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((key_mass_bf16<128, 32>), grid, dim3(512), 0, stream, p);
  } else {
    if (wide) hipLaunchKernelGGL((key_mass_bf16<64, 64>), grid, dim3(512), 0, stream, p);
    else hipLaunchKernelGGL((key_mass_bf16<64, 32>), grid, dim3(512), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace rk
