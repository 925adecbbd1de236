// Device-side vector types and small helpers shared by the gfx950 kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rk_seg.h"

namespace rk {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int V>
struct IntC {
  static constexpr int value = V;
};

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

__device__ __forceinline__ bool visible(int cls, int i, int j, int sink, int window) {
  return j <= i && (cls == RK_GLOBAL || j < sink || j > i - window);
}

// Swizzle of the 16-byte chunks of a row of D bf16 values staged in LDS by direct 16-byte loads:
// chunk c of row r sits in slot c ^ kswz(r), so 16 consecutive lanes reading 16 consecutive rows at
// one chunk index touch 16 distinct 16-byte slots of every 256-byte bank window.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
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

// The value unchanged, hidden from code motion: a loop-invariant 32-bit lane offset then stays
// 32-bit at its use, where it forms the scalar-base + 32-bit-offset address of a global load
// (instead of a hoisted 64-bit vector address that holds two registers for the whole loop).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// 16 bytes per lane from a wave-uniform base plus a 32-bit lane offset into a dense 1 KB LDS block,
// in the buffer form (a raw descriptor whose range is `bytes`; offsets past it read zeros).  The
// compiler's wait insertion treats an LDS load in the global form as an LDS access of unknown order,
// so while one is in flight every later LDS read waits for all of them (lgkmcnt(0)); in the buffer
// form the LDS operand reads keep their partial waits and can run ahead of the products using them.
__device__ __forceinline__ void load_lds16_buf(const void *base, uint32_t voff, uint32_t bytes, void *lds_block) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_block, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ void load_lds16(const void *gsrc, void *lds_block) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)gsrc,
                                   (__attribute__((address_space(3))) void *)lds_block, 16, 0, 0);
}


// vmcnt(N): wait until at most N vector memory operations of this wave are outstanding (they retire
// in issue order)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// A workgroup barrier without __syncthreads()'s memory fences.  Those make the compiler wait for
// every outstanding load into LDS (vmcnt(0)), also the tiles of later steps still in flight; the
// caller waits for exactly the loads it needs first (wait_vmcnt).  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 4 bytes per lane from base + a 32-bit lane offset into a dense 256-byte LDS block (lane l writes
// bytes 4 l .. 4 l + 3), buffer form with range `bytes`
__device__ __forceinline__ void load_lds4_buf(const void *base, uint32_t voff, uint32_t bytes, void *lds_block) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds_block, 4, voff, 0, 0, 0);
}

// In-place updates of a 16-register accumulator tuple.  Written as inline asm with tied operands so
// the tuple keeps its registers (a compiler-generated select or multiply may write a fresh tuple and
// copy it back).  The values come from matrix products, which the hardware does not interlock with
// VALU reads: the leading s_nops give the wait states an 8-pass product needs before its result is
// read, whatever came between.
__device__ __forceinline__ void mfma_result_wait() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" ::: "memory"); }

// s[i] = bit o(i) of vis ? s[i] : -inf, o(i) = 16 (i / 8) + i % 8 (the key offset of register i)
__device__ __forceinline__ void in_place_mask(f32x16 &s, uint32_t vis) {
  mfma_result_wait();
  const float ninf = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = s[i];
    uint32_t t;
    asm volatile("v_bfe_i32 %1, %2, %3, 1\n\tv_bfi_b32 %0, %1, %0, %4"
                 : "+v"(x), "=&v"(t)
                 : "v"(vis), "i"(16 * (i >> 3) + (i & 7)), "v"(ninf));
    s[i] = x;
  }
}

// v *= a for every element, in place, where the products writing v have already been waited for
// (mfma_result_wait)
__device__ __forceinline__ void in_place_scale_ready(f32x16 &v, float a) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x = v[i];
    asm volatile("v_mul_f32 %0, %1, %0" : "+v"(x) : "v"(a));
    v[i] = x;
  }
  // the tuple is the accumulator of later products: wait states between a VALU write and a
  // matrix product reading it (the compiler does not see the writes inside the asm)
  asm volatile("s_nop 4" ::: "memory");
}

}  // namespace rk
