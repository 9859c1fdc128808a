// gfx950 instructions that the decode kernel issues as inline asm, because the
// compiler's own forms would add waits it cannot prove unnecessary.
#ifndef MLA_GFX950_ASM_H
#define MLA_GFX950_ASM_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uniform_ptr.h"

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
  const char* base = (const char*)uniform_u64(
      (uint64_t)base_, [](uint32_t x) { return __builtin_amdgcn_readfirstlane(x); });
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

// Returns x unchanged, but the optimizer can no longer see its value: an
// address formed from it is computed where it is used instead of being hoisted
// out of a loop into a register of its own (which, in a kernel at its register
// limit, ends up spilled).  Emits no instruction.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Stores through a buffer resource: a wave-uniform base address and byte size
// (scalar registers) plus a 32-bit per-lane byte offset, a wave-uniform byte
// offset and an immediate.  Kernels under register pressure use them so that
// no 64-bit per-lane address has to stay live for a rare store.  A store whose
// offset reaches past `bytes` is dropped by the hardware.
typedef __amdgpu_buffer_rsrc_t buf_t;
__device__ __forceinline__ buf_t buf_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}
__device__ __forceinline__ void buf_store_b32(uint32_t v, buf_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store_b64(uint32_t lo, uint32_t hi, buf_t r, uint32_t voff,
                                              uint32_t soff) {
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_raw_buffer_store_b64(v2u{lo, hi}, r, voff, soff, 0);
}

}  // namespace mla

#endif  // MLA_GFX950_ASM_H
