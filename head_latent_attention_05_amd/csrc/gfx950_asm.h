// gfx950 instructions that the decode kernel issues as inline asm, because the
// compiler's own forms would add waits it cannot prove unnecessary.
#ifndef MLA_GFX950_ASM_H
#define MLA_GFX950_ASM_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#define LDS_AS __attribute__((address_space(3)))

namespace mla {

// Workgroup barrier without the memory fence that __syncthreads implies (that
// fence waits for every outstanding load, which would drain a tile pipeline);
// callers order LDS data with an explicit s_waitcnt before it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// One 16-byte-per-lane direct-to-LDS load: lane l's 16 bytes from base + voff
// land at lds_dst + 16*l.  Written as inline asm so the compiler does not treat
// every later LDS read as a possible reader of the in-flight data (it would then
// wait for all outstanding loads before each tile); callers order it with an
// explicit s_waitcnt vmcnt + barrier() before the data is read.  The
// instruction has no destination register; its address operands are read at
// issue.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is set here and used by nothing else
__device__ __forceinline__ void dma16(const char* base_, uint32_t voff, char* lds_dst) {
  // both addresses are wave-uniform; make that explicit for the scalar operands
  // (readfirstlane yields a signed int: go through uint32_t so the low half is
  // zero-extended, not sign-extended, when the pointer is rebuilt)
  const uint64_t bv = (uint64_t)base_;
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(bv >> 32));
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bv);
  const char* base = (const char*)((hi << 32) | lo);
  const uint32_t m0v = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS char*)lds_dst);
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "s"(m0v)
      : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace mla

#endif  // MLA_GFX950_ASM_H
