// Emulator versions of the library's inline-asm helpers (csrc/gfx950_asm.h).
// Force-included before a kernel source; defining that header's include guard
// here makes the source use these definitions instead of the asm ones.
#pragma once
#define MLA_GFX950_ASM_H

#include <stdint.h>
#include <string.h>

#include "hip/hip_runtime.h"

#define LDS_AS __attribute__((address_space(3)))

namespace mla {

__forceinline__ void barrier() { ::emu::block_barrier(); }

// lane l's 16 bytes from base + voff land at lds_dst + 16*l, asynchronously:
// only an s_waitcnt vmcnt that counts this load guarantees they have landed
__forceinline__ void dma16(const char* base, uint32_t voff, char* lds_dst) {
  // the instruction takes its base and LDS destination from scalar registers:
  // they must be the same in every lane
  const uint64_t b = (uint64_t)(uintptr_t)base;
  if ((uint32_t)::emu::readfirstlane((unsigned)(b >> 32)) != (uint32_t)(b >> 32) ||
      (uint32_t)::emu::readfirstlane((unsigned)b) != (uint32_t)b)
    ::emu::fail("dma16: base differs between lanes");
  ::emu::dma16(base + voff, lds_dst);
}

inline uint32_t opaque(uint32_t x) { return x; }

// Buffer-resource stores: bounds-checked against the resource's byte size
// (the hardware drops such a store; in the emulator it is an error, since no
// kernel here means to rely on that).
struct buf_t {
  char* base;
  uint32_t bytes;
};
inline buf_t buf_rsrc(void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  if ((uint32_t)::emu::readfirstlane((unsigned)(b >> 32)) != (uint32_t)(b >> 32) ||
      (uint32_t)::emu::readfirstlane((unsigned)b) != (uint32_t)b ||
      (uint32_t)::emu::readfirstlane(bytes) != bytes)
    ::emu::fail("buffer resource differs between lanes");
  return buf_t{(char*)base, bytes};
}
inline void buf_store_b32(uint32_t v, buf_t r, uint32_t voff, uint32_t soff) {
  if ((uint64_t)voff + soff + 4 > r.bytes) ::emu::fail("buffer store out of range");
  memcpy(r.base + voff + soff, &v, 4);
}
inline void buf_store_b64(uint32_t lo, uint32_t hi, buf_t r, uint32_t voff, uint32_t soff) {
  if ((uint64_t)voff + soff + 8 > r.bytes) ::emu::fail("buffer store out of range");
  memcpy(r.base + voff + soff, &lo, 4);
  memcpy(r.base + voff + soff + 4, &hi, 4);
}

}  // namespace mla
