// Direct global -> LDS loads (gfx950 global_load_lds_dwordx4) shared by the MFMA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ozk {

// Lane i of the wave copies 16 bytes from g into LDS bytes [lds_base + 16 i, +16).  Issued
// through inline assembly so the compiler neither reorders it nor inserts conservative
// waits; completion is tracked with explicit s_waitcnt vmcnt and made visible to other
// waves with s_barrier.  M0 (the LDS base) is written by a scalar move, with one wait
// state before the load that reads it.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(g), "s"(lds_base)
      : "memory", "m0");
}

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset
// (global address = base + offset): advancing the source only takes scalar adds.
__device__ __forceinline__ void dma16_sbase(uint32_t voffset, uint64_t sbase, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voffset), "s"(sbase), "s"(lds_base)
      : "memory", "m0");
}

// Byte address of a __shared__ object in the LDS aperture.
template <typename T>
__device__ __forceinline__ uint32_t lds_address(T* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T*)p;
}

}  // namespace ozk
