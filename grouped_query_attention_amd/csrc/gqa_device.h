// Device-side helpers shared by the libgqa kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

constexpr int D_MODEL = 4096;
constexpr int N_HEADS = 32;
constexpr int N_KV = 8;
constexpr int D_HEAD = 128;
constexpr int N_REP = N_HEADS / N_KV;     // query heads per KV head (4)
constexpr int N_QKV = D_MODEL + 2 * N_KV * D_HEAD;  // 6144 fused projection columns
constexpr int D_FF = 14336;               // SwiGLU MLP hidden width
// log2(e)/sqrt(128): the score scale 1/sqrt(d_head) of the softmax, in base 2
constexpr float QK_SCALE_LOG2 = 0.12751743082459868f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// D(32x32) += A(32x16) * B(16x32), bf16 in, fp32 accumulate.
// Operand lane layout: lane l holds row/column (l & 31), k = 8*(l >> 5) .. +7.
// Result lane layout: lane l holds column (l & 31), rows 8*(i/4) + 4*(l>>5) + (i&3).
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16).
// Operand lane layout: lane l holds row/column (l & 15), k = 8*(l >> 4) .. +7.
// Result lane layout: lane l holds column (l & 15), rows 4*(l>>4) + i.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// s_waitcnt with vmcnt(n) and the other counters left free (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Waits until at most n of this wave's K steps (PER load instructions each)
// are still in flight; n <= MAXN, resolved to an immediate vmcnt.
template <int PER, int MAXN>
__device__ __forceinline__ void wait_keep(int n) {
  if constexpr (MAXN <= 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAXN) wait_vmcnt<PER * MAXN>();
    else wait_keep<PER, MAXN - 1>(n);
  }
}

// 16-byte-per-lane direct-to-LDS load (global_load_lds_dwordx4): lane l's 16
// bytes from `src` land at LDS byte lds_dst + 16*l (lds_dst wave-uniform). It is
// issued through inline asm so that the compiler's wait-count pass does not see
// it: that pass cannot count these loads across loop iterations and would
// otherwise wait for every load in flight (vmcnt(0)) before the next use of any
// register loaded from memory, or before LDS reads it cannot disambiguate,
// draining the prefetch ring every step. The kernels issue their own waits
// (wait_vmcnt / wait_keep) before a stage is read. M0 is written here and used
// by nothing else in these kernels (a test checks the generated assembly).
// The destination is an LDS byte address (lds_addr of the __shared__ array plus
// a byte offset) computed from wave-uniform values, so that it stays in scalar
// registers: a destination passed as a generic pointer is converted back with a
// null check, and one built from a per-lane wave index is moved to a scalar
// register with v_readfirstlane, both on every load (about 8 dependent VALU and
// SALU instructions per load in the step loops).
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_byte) : "memory");
}

// dma16 from a wave-uniform 64-bit base (SGPR pair) plus a per-lane 32-bit
// byte offset: a tile's loads then need no per-lane address arithmetic, only
// scalar adds to the base.
__device__ __forceinline__ void dma16_sv(const void* sbase, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_byte) : "memory");
}

// dma16 with the non-temporal hint, for data that is read exactly once (the
// decode kernel's K/V cache stream): the lines are not kept in L2 and the
// Infinity Cache. A 2.1 GB single-pass stream runs 13 % faster this way
// (6.7 against 5.8 TB/s, caches flushed before each call): allocating the
// lines it never re-reads costs more than the loads themselves.
__device__ __forceinline__ void dma16_nt(const void* src, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt"
               :: "v"(src), "s"(lds_byte) : "memory");
}

// LDS byte address of a __shared__ array (apply to the array itself: the
// conversion of its generic address then folds to a constant).
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* shared_array) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T*)shared_array;
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Workgroup barrier without the memory fence __syncthreads() carries: the
// fence would wait for every outstanding load (vmcnt(0)), draining prefetched
// pipeline stages. Used where LDS is only written by direct-to-LDS loads and
// each wave has already waited (wait_vmcnt / wait_keep) for its own loads of
// the stage it is about to read. The "memory" clobber keeps the compiler from
// moving LDS reads across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace gqa
