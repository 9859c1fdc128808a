// Rebuilding a 64-bit address from two 32-bit wave-uniform halves.
//
// A scalar (wave-uniform) copy of a pointer is taken one 32-bit half at a
// time with readfirstlane, whose result type is a signed int.  Widening that
// int straight to 64 bits sign-extends it: a low half with bit 31 set would
// fill the high word with ones and the rebuilt address would be wrong.  Both
// halves therefore go through uint32_t before they are joined.  The helper is
// plain C++ so the host test suite compiles and checks it with the same code
// the kernels use.
#ifndef MLA_UNIFORM_PTR_H
#define MLA_UNIFORM_PTR_H

#include <stdint.h>

#ifndef __HIPCC__
#ifndef __host__
#define __host__
#endif
#ifndef __device__
#define __device__
#endif
#endif

namespace mla {

// `first` maps a 32-bit value to its wave-uniform copy (readfirstlane on the
// device); it may return a signed int.
template <typename First>
__host__ __device__ inline uint64_t uniform_u64(uint64_t v, First first) {
  const uint32_t hi = (uint32_t)first((uint32_t)(v >> 32));
  const uint32_t lo = (uint32_t)first((uint32_t)v);
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}

}  // namespace mla

#endif  // MLA_UNIFORM_PTR_H
