// Direct global -> LDS loads and explicit memory-counter waits (gfx950).
#pragma once

#include "common.h"

namespace hp {

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 16-byte direct load per active lane into LDS at m0 + 16 * lane
// (lds_base must be wave-uniform).  Completion is counted by vmcnt.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(g), "s"(lds_base)
      : "memory", "m0");
}

// One 4-byte direct load per active lane into LDS at m0 + 4 * lane.
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(g), "s"(lds_base)
      : "memory", "m0");
}

// The same two loads with the address split into a wave-uniform base
// (kept in an SGPR pair) and a per-lane 32-bit byte offset.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(uniform_ptr(base)), "s"(lds_base)
      : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(uniform_ptr(base)), "s"(lds_base)
      : "memory", "m0");
}

// s_waitcnt vmcnt(n) lgkmcnt(l) (gfx9 encoding; expcnt unconstrained).
template <int n, int l = 15>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64 && l >= 0 && l < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (l << 8) | ((n >> 4) << 14));
}

}  // namespace hp
