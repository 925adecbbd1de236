// gfx950 (CDNA4) page-writing kernels of the SegPagedAttention prefill library.
//
//  * page_copy<PACK>: copies whole held pages to or from a packed buffer (the page hand-off).
//  * kv_write<...>: writes token rows into held pages, either the new tokens of the call (the online
//    KV write of EXECUTE, aiboss88.com section 使い方) or a reused document whose keys are rotated from
//    their offline to their actual position (page "RedKnot – 小红书研发并开源的长上下文大模型推理引擎"
//    (shshi.cn), section RedKnot技术原理, 2. 位置无关缓存复用).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rk_device.h"
#include "rk_ops.h"
#include "rk_seg.h"

namespace rk {
namespace {

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

  const int tid = threadIdx.x;
  const int g = blockIdx.y;
  const int P = p.P;
  int seq, lp, t_lo, t_hi;
  SeqInfo si{};
  if (IMPORT) {
    seq = p.seq;
    lp = p.page0 + blockIdx.x;
    si = p.seqs[seq];
    // tokens from the head's class start on are the call's own (its append writes them): not imported
    const int start = p.head_class[g] == RK_GLOBAL ? si.q_start : si.q_start_local;
    t_lo = max(lp * P, p.tok_begin);
    t_hi = min(min(lp * P + P, p.tok_begin + p.n_tok), start);
  } else {
    seq = p.app_items[2 * blockIdx.x];
    lp = p.app_items[2 * blockIdx.x + 1];
    si = p.seqs[seq];
    // a GLOBAL head writes from the sequence's first packed position, a LOCAL head from its own
    // (later) start: below it the head keeps its reused KV
    t_lo = max(lp * P, p.head_class[g] == RK_GLOBAL ? si.q_start : si.q_start_local);
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

  // K
  if (!IMPORT) {
    for (int c = tid; c < n * (D / VEC); c += blockDim.x) {
      const int tk = c / (D / VEC), ch = c - tk * (D / VEC);
      *reinterpret_cast<u32x4 *>(kdst + (int64_t)tk * D + ch * VEC) =
          *reinterpret_cast<const u32x4 *>(src_row(ksrc, t_lo + tk) + ch * VEC);
    }
  } else {
    // VEC consecutive pairs per thread: rotate-half pairs (m, m + D/2) are two 16-byte runs of the
    // row; interleaved pairs (2m, 2m + 1) are two consecutive 16-byte runs
    constexpr int NJ = D / 2 / VEC;  // pair groups per row
    typedef T TV __attribute__((ext_vector_type(VEC)));
    for (int c = tid; c < n * NJ; c += blockDim.x) {
      const int tk = c / NJ, j = c - tk * NJ, m0 = VEC * j;
      const T *s = src_row(ksrc, t_lo + tk);
      T *d = kdst + (int64_t)tk * D;
      const bool half = p.rope_style == RK_ROPE_ROTATE_HALF;
      const int oa = half ? m0 : 2 * m0, ob = half ? m0 + D / 2 : 2 * m0 + VEC;
      const TV ra = *reinterpret_cast<const TV *>(s + oa), rb = *reinterpret_cast<const TV *>(s + ob);
      TV wa, wb;
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        // pair k of the group: rotate-half (ra[k], rb[k]); interleaved (r[2k], r[2k + 1]) over ra | rb
        const int m = m0 + k;
        const float xa = to_f(half ? ra[k] : (2 * k < VEC ? ra[2 * k] : rb[2 * k - VEC]));
        const float xb = to_f(half ? rb[k] : (2 * k + 1 < VEC ? ra[2 * k + 1] : rb[2 * k + 1 - VEC]));
        const float ya = xa * p.rope_cos[m] - xb * p.rope_sin[m];
        const float yb = xb * p.rope_cos[m] + xa * p.rope_sin[m];
        if (half) {
          wa[k] = from_f<T>(ya);
          wb[k] = from_f<T>(yb);
        } else {
          if (2 * k < VEC) wa[2 * k] = from_f<T>(ya); else wb[2 * k - VEC] = from_f<T>(ya);
          if (2 * k + 1 < VEC) wa[2 * k + 1] = from_f<T>(yb); else wb[2 * k + 1 - VEC] = from_f<T>(yb);
        }
      }
      *reinterpret_cast<TV *>(d + oa) = wa;
      *reinterpret_cast<TV *>(d + ob) = wb;
    }
  }

  // Every slot of a held page that attention may load must hold a finite value.  The append into
  // the sequence's last page clears the slots past kv_len; on a LOCAL head's first written page it
  // clears the slots below its window and above the sink (tokens no query of this call or a later one
  // sees), which a page newly taken for a window that moved on would otherwise leave unwritten.
  if (!IMPORT) {
    int z0 = 0, z1 = 0;  // slots [z0, z1) to clear
    if (t_hi == si.kv_len && t_hi < lp * P + P) z0 = t_hi - lp * P, z1 = P;
    T *kz = static_cast<T *>(p.k_pages) + (int64_t)pg * P * D;
    for (int pass = 0; pass < 2; ++pass) {
      if (pass == 1) {
        z0 = z1 = 0;
        if (p.head_class[g] != RK_GLOBAL) {
          z0 = max(lp * P, p.sink) - lp * P;
          z1 = min(t_lo, si.q_start_local - p.window + 1) - lp * P;
        }
      }
      const int nz = z1 - z0;
      if (nz <= 0) continue;
      for (int c = tid; c < nz * D; c += blockDim.x) kz[(int64_t)z0 * D + c] = from_f<T>(0.f);
      for (int c = tid; c < nz * D; c += blockDim.x) {
        const int d = c / nz, sl = z0 + c % nz;
        vdst[(int64_t)d * P + sl] = from_f<T>(0.f);
      }
    }
  }

  // V: transpose [tokens][D] -> page [D][P] through LDS, kTokBlock tokens at a time.  Rows are read
  // 16 bytes per thread; each channel row of the page is written in 16-byte groups of VEC slots where
  // a group lies wholly inside the block's slots, element by element at the block's ragged ends.
  typedef T TV __attribute__((ext_vector_type(VEC)));
  for (int tb = 0; tb < n; tb += kTokBlock) {
    const int nb = min(kTokBlock, n - tb);
    __syncthreads();
    for (int c = tid; c < nb * (D / VEC); c += blockDim.x) {
      const int tk = c / (D / VEC), ch = c - tk * (D / VEC);
      const TV v = *reinterpret_cast<const TV *>(src_row(vsrc, t_lo + tb + tk) + ch * VEC);
#pragma unroll
      for (int k = 0; k < VEC; ++k) sv[tk * VPITCH + ch * VEC + k] = v[k];
    }
    __syncthreads();
    const int sa = s0 + tb, se = sa + nb;      // slots [sa, se) of this block
    const int g0 = (sa + VEC - 1) / VEC, g1 = se / VEC;  // whole VEC-slot groups inside
    const int ng = max(0, g1 - g0);
    for (int c = tid; c < ng * D; c += blockDim.x) {
      const int d = c / ng, gi = g0 + (c - d * ng);
      TV w;
#pragma unroll
      for (int k = 0; k < VEC; ++k) w[k] = sv[(gi * VEC + k - sa) * VPITCH + d];
      *reinterpret_cast<TV *>(vdst + (int64_t)d * P + gi * VEC) = w;
    }
    // ragged ends: slots [sa, g0 VEC) and [max(g1 VEC, sa), se) that no whole group covers
    const int h0 = min(se, g0 * VEC), t0 = max(sa, max(g1, g0) * VEC);
    const int nh = h0 - sa, nt = max(0, se - t0);  // no tail when the block lies inside one group
    for (int c = tid; c < (nh + nt) * D; c += blockDim.x) {
      const int d = c / (nh + nt), i = c - d * (nh + nt);
      const int sl = i < nh ? sa + i : t0 + (i - nh);
      vdst[(int64_t)d * P + sl] = sv[(sl - sa) * VPITCH + d];
    }
  }
}

// One workgroup per page: the page's K then V, 16 bytes per thread and step, pool <-> packed buffer.
template <bool PACK>
__global__ void __launch_bounds__(256) page_copy(PageCopyParams p) {
  const int64_t i = blockIdx.x;
  const int64_t pg = p.ids[i];
  const int64_t nv = p.page_bytes / 16;
  char *kp = static_cast<char *>(p.k_pages) + pg * p.page_bytes;
  char *vp = static_cast<char *>(p.v_pages) + pg * p.page_bytes;
  char *bk = static_cast<char *>(p.buf) + 2 * i * p.page_bytes;
  char *bv = bk + p.page_bytes;
  for (int64_t c = threadIdx.x; c < nv; c += blockDim.x) {
    if (PACK) {
      const u32x4 a = reinterpret_cast<const u32x4 *>(kp)[c];
      const u32x4 b = reinterpret_cast<const u32x4 *>(vp)[c];
      reinterpret_cast<u32x4 *>(bk)[c] = a;
      reinterpret_cast<u32x4 *>(bv)[c] = b;
    } else {
      const u32x4 a = reinterpret_cast<const u32x4 *>(bk)[c];
      const u32x4 b = reinterpret_cast<const u32x4 *>(bv)[c];
      reinterpret_cast<u32x4 *>(kp)[c] = a;
      reinterpret_cast<u32x4 *>(vp)[c] = b;
    }
  }
}

}  // namespace

hipError_t launch_page_copy(const PageCopyParams &p, bool pack, hipStream_t stream) {
  if (p.n <= 0) return hipSuccess;
  if (pack)
    hipLaunchKernelGGL(page_copy<true>, dim3((unsigned)p.n), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(page_copy<false>, dim3((unsigned)p.n), dim3(256), 0, stream, p);
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
