// Direct global -> LDS loads (buffer_load ... lds) for gfx950 and the
// explicit waits and barriers that go with them.
//
// The loads are written as inline asm on purpose: the compiler then inserts
// no vmcnt waits of its own before LDS reads of the ring slots (it would
// otherwise wait for every DMA issued so far, which serialises the ring).
// Every consumer of a slot is therefore ordered by an explicit
// s_waitcnt vmcnt(N) in the issuing wave followed by a barrier.
#pragma once

#include <type_traits>

#include "device_common.h"

typedef int i32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Raw buffer descriptor words: base, stride 0, num_records bytes (an offset at
// or beyond it reads as zero), 32-bit data format.
__device__ __forceinline__ i32x4v rsrc_words(const void* p, uint32_t nrec) {
  const uint64_t a = (uint64_t)p;
  i32x4v r;
  r.x = (int)(uint32_t)a;
  r.y = (int)((uint32_t)(a >> 32) & 0xffffu);
  r.z = (int)nrec;
  r.w = 0x00020000;
  return r;
}

// LDS byte address of a __shared__ pointer, as a wave-uniform scalar.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p);
}

// 16 bytes per lane from rsrc + voff + soff into LDS at la + 16 * lane.  The
// s_nop covers the M0-write -> LDS-DMA hazard.
__device__ __forceinline__ void dma16(i32x4v rs, int voff, int soff, uint32_t la) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(la), "v"(voff), "s"(rs), "s"(soff) : "memory");
}
// dma16 with the LDS address formed as lbase + IMM in M0 itself (one scalar
// instruction per DMA, no SGPR for the sum).
template <int IMM>
__device__ __forceinline__ void dma16k(i32x4v rs, int voff, int soff, uint32_t lbase) {
  asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lbase), "v"(voff), "s"(rs), "s"(soff), "n"(IMM) : "scc", "memory");
}
// Calls f(std::integral_constant<int, J>) for J = J0 .. N - 1 (compile-time
// indices for dma16k).
template <int J, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (J < N) {
    f(std::integral_constant<int, J>());
    static_for<J + 1, N>(f);
  }
}
// 4 bytes per lane into LDS at la + 4 * lane.
__device__ __forceinline__ void dma4(i32x4v rs, int voff, int soff, uint32_t la) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(la), "v"(voff), "s"(rs), "s"(soff) : "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}
// s_waitcnt lgkmcnt(0)
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_barrier without the fence __syncthreads adds (which would also wait for
// every outstanding vector memory operation of the wave).
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Two floats to packed bf16 (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}
