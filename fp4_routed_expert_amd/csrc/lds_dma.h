// LDS-DMA helpers shared by the LDS-staged GEMMs (gfx950): global_load_lds
// with a wave-uniform base, and the vector-memory wait that gates a stage.
#pragma once

#include "common.h"

namespace moe {

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Wave-uniform values for the scalar operands of the DMA instructions (no-ops
// when the compiler already holds them in scalar registers).
__device__ __forceinline__ uint32_t wave_u32(uint32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ const uint8_t* wave_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint64_t lo = wave_u32((uint32_t)v), hi = wave_u32((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>((uintptr_t)(lo | (hi << 32)));
}

// LDS-DMA with a uniform 64-bit base in SGPRs and a per-lane 32-bit offset
// (the saddr form): every lane loads 16 (or 4) bytes from base + its offset;
// lane l's bytes land at LDS byte address m0 + 16 l (or 4 l).  The LDS
// addresses are wave-uniform.  M0 is restored after; one wait state
// separates each M0 write from the load that reads it.
__device__ __forceinline__ void dma_x4(const uint8_t* base, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}

__device__ __forceinline__ void dma_x1(const uint8_t* base, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace moe
