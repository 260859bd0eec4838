// LDS helpers shared by the bf16 attention kernels (forward and backward):
// vector types, the LDS address of a shared-memory location, and direct
// global-to-LDS loads.
#pragma once

#include "common.h"

namespace dma {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

// LDS byte address of a location in the workgroup's shared memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void*)p;
}

// Direct global-to-LDS loads, written as inline asm so that the compiler
// neither tracks them nor inserts waits for them: every wait for them is an
// explicit s_waitcnt vmcnt in the caller.  Lane L's data lands at the LDS
// byte address m0 + size*L; the instruction after an m0 write needs one wait
// state.  They have no register results, and their address registers are
// read when they issue.
__device__ __forceinline__ void dma_b128(const void* src, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(lds)
      : "m0");
}
// The same with the global address split into a uniform base (scalar
// registers) and a 32-bit per-lane byte offset: one vector register per load
// instead of a 64-bit pair.
__device__ __forceinline__ void dma_b128_s(const void* base, uint32_t off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds)
      : "m0");
}
// The same with the LDS address read from lane 0 just before the m0 write,
// for callers whose uniform address the compiler may keep in a vector
// register.
__device__ __forceinline__ void dma_b128_u(const void* src, uint32_t lds) {
  dma_b128(src, (uint32_t)__builtin_amdgcn_readfirstlane((int)lds));
}
__device__ __forceinline__ void dma_b32(const void* src, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(src), "s"(lds)
      : "m0");
}

// Eight fp32 values as a bf16 MFMA operand (round to nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = (__bf16)p[t];
  return r;
}

}  // namespace dma
