// gfx950 (CDNA4) kernels of decode over the segmented pool: one query row per sequence, after the
// prefill call whose state the pool keeps (page "RedKnot – 小红书研发并开源的长上下文大模型推理引擎"
// (shshi.cn), section RedKnot核心特点: sessions per GPU at long context; page "小红书把 KV Cache 按
// 「头」拆了…" (zhichai.net), section 事件内容: GLOBAL heads read every context page, LOCAL heads only
// their sink and recent-window pages).
//
//  * decode_bf16<D>: one wave per split-KV item (seq, kv head, key range).  The G <= 16 query rows of
//    the KV head are the N = 16 columns of v_mfma_f32_16x16x32_bf16: S^T = K Q^T with keys as M, then
//    O^T += V^T P^T with channels as M, so P never leaves registers (the two 16-key halves of a 32-key
//    tile give each lane the 8 keys its B operand needs, in the order the V loads follow).  K and V
//    come straight from the pages into registers (16- and 8-byte loads off a scalar page base), one
//    32-key tile ahead.  Online softmax in fp32; the item writes its normalised partial output and lse.
//  * decode_combine<D>: merges the partials of each (seq, kv head): lse = log sum_s e^{lse_s},
//    o = sum_s e^{lse_s - lse} o_s (the split-KV combine).
// Decode reads every visible K/V byte once, so it is bound by HBM bandwidth, not by the MFMAs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rk_device.h"
#include "rk_internal.h"
#include "rk_seg.h"

namespace rk {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct DecTile {
  bf16x8 k[2][D / 32];  // A operand of S^T: keys kt + 16 h + (lane % 16), channels 32 ks + 8 (lane / 16) ..
  u32x2 va[D / 16];     // V^T rows 16 dt + lane % 16, keys kt + 4 (lane / 16) .. + 3
  u32x2 vb[D / 16];     // the same, keys kt + 16 + 4 (lane / 16) .. + 3
};

template <int D>
__global__ void __launch_bounds__(64) decode_bf16(DecodeParams p) {
  constexpr int KS = D / 32;  // 32-channel steps of QK
  constexpr int DT = D / 16;  // 16-channel tiles of PV
  const int lane = threadIdx.x, c16 = lane & 15, q4 = lane >> 4;
  const DecItem it = p.items[blockIdx.x];
  const int b = it.seq, g = it.kv_head, k0 = it.k0, k1 = it.k1;
  const SeqInfo si = p.seqs[b];
  const int L = si.kv_len, P = p.P, G = p.G;
  const int32_t *pt = p.page_ids + p.page_base[g * p.num_seqs + b];
  // a key past kv_len or on a page the head does not hold reads the page of k0 (held) and is masked
  const int pg0 = pt[k0 >> p.log2P];
  auto page_of = [&](int key) {  // uniform: a scalar load of the page table
    const int pg = pt[min(key, L - 1) >> p.log2P];
    return key < L && pg >= 0 ? pg : pg0;
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

  const char *kbytes = static_cast<const char *>(p.k_pages);
  const char *vbytes = static_cast<const char *>(p.v_pages);
  const uint32_t k_lane = (uint32_t)((c16 * D + 8 * q4) * 2);  // bytes within a 16-key block of a K page
  const uint32_t v_lane = (uint32_t)((c16 * P + 4 * q4) * 2);  // bytes within a 16-channel block of a V page
  auto load = [&](int kt, DecTile<D> &T) {
    const int pa = page_of(kt), pb = page_of(kt + 16);  // uniform; equal when P >= 32
    const int sa = kt & (P - 1), sb = (kt + 16) & (P - 1);
    const char *ka = kbytes + ((int64_t)pa * P + sa) * D * 2;
    const char *kb = kbytes + ((int64_t)pb * P + sb) * D * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      T.k[0][ks] = *reinterpret_cast<const bf16x8 *>(ka + opaque(k_lane) + 64 * ks);
      T.k[1][ks] = *reinterpret_cast<const bf16x8 *>(kb + opaque(k_lane) + 64 * ks);
    }
    const char *va = vbytes + ((int64_t)pa * D * P + sa) * 2;
    const char *vb = vbytes + ((int64_t)pb * D * P + sb) * 2;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      T.va[dt] = *reinterpret_cast<const u32x2 *>(va + opaque(v_lane) + dt * 16 * P * 2);
      T.vb[dt] = *reinterpret_cast<const u32x2 *>(vb + opaque(v_lane) + dt * 16 * P * 2);
    }
  };

  const float c2 = p.scale_log2;
  float m = -INFINITY, l = 0.f;  // running max (log2 units) and this lane's part of the row sum
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int kt, const DecTile<D> &T) {
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
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
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

  const int t0 = k0 & ~31;
  const int ntiles = ((k1 - 1 - t0) >> 5) + 1;
  DecTile<D> buf[2];
  load(t0, buf[0]);
  for (int t = 0; t < ntiles; t += 2) {
    if (t + 1 < ntiles) load(t0 + 32 * (t + 1), buf[1]);
    compute(t0 + 32 * t, buf[0]);
    if (t + 1 < ntiles) {
      if (t + 2 < ntiles) load(t0 + 32 * (t + 2), buf[0]);
      compute(t0 + 32 * (t + 1), buf[1]);
    }
  }

  // row sum over the four lane groups; normalised partial output and lse (natural log)
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (c16 < G) {
    const float inv = 1.0f / l;
    float *po = p.part_o + ((int64_t)blockIdx.x * G + c16) * D + 4 * q4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4 *>(po + 16 * dt) = o[dt] * inv;
    if (q4 == 0) p.part_lse[(int64_t)blockIdx.x * G + c16] = (m + __log2f(l)) * 0.6931471805599453f;
  }
}

// One workgroup per (seq, kv head): lse = max + log sum_s e^{lse_s - max}; o = sum_s e^{lse_s - lse} o_s.
template <int D>
__global__ void __launch_bounds__(256) decode_combine(DecodeParams p) {
  const int bg = blockIdx.x;
  const int b = bg / p.Hkv, g = bg - b * p.Hkv;
  const int s0 = p.comb_off[bg], s1 = p.comb_off[bg + 1];
  if (s0 == s1) return;  // the sequence has no query row
  const SeqInfo si = p.seqs[b];
  const int G = p.G;
  for (int e = threadIdx.x; e < G * (D / 4); e += blockDim.x) {
    const int r = e / (D / 4), d4 = e - r * (D / 4);
    float mx = -INFINITY;
    for (int s = s0; s < s1; ++s) mx = fmaxf(mx, p.part_lse[(int64_t)s * G + r]);
    float tot = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = s0; s < s1; ++s) {
      const float w = expf(p.part_lse[(int64_t)s * G + r] - mx);
      tot += w;
      acc += w * *reinterpret_cast<const f32x4 *>(p.part_o + ((int64_t)s * G + r) * D + 4 * d4);
    }
    const int64_t row = (int64_t)si.cu_q * p.H + g * G + r;
    *reinterpret_cast<bf16x4 *>(static_cast<bf16_t *>(p.o) + row * D + 4 * d4) = __builtin_convertvector(acc / tot, bf16x4);
    if (d4 == 0 && p.lse) p.lse[(int64_t)(g * G + r) * p.total_q + si.cu_q] = mx + logf(tot);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int head_dim, hipStream_t stream) {
  if (p.n_items <= 0) return hipSuccess;
  const dim3 grid((unsigned)p.n_items), comb((unsigned)(p.num_seqs * p.Hkv));
  if (head_dim == 128) {
    hipLaunchKernelGGL(decode_bf16<128>, grid, dim3(64), 0, stream, p);
    hipLaunchKernelGGL(decode_combine<128>, comb, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL(decode_bf16<64>, grid, dim3(64), 0, stream, p);
    hipLaunchKernelGGL(decode_combine<64>, comb, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace rk
