// Pieces shared by the split-KV latent decode kernels (bf16 and e4m3 caches):
// the wave-uniform walk over the 32-row tiles of a workgroup's unit range, the
// wait on a wave-uniform count of outstanding loads, and the reductions over
// the four lanes that hold one head's scores.
#pragma once

#include "gfx950_asm.h"
#include "plan_device.h"

namespace mla {
namespace tiles {

constexpr int kBS = 64;    // rows per cache block
constexpr int kTile = 32;  // rows per tile (half a cache block)

// s_waitcnt with vmcnt = n (other counters unconstrained).  The instruction
// takes an immediate, so a wave-uniform count is dispatched through a switch.
__device__ __forceinline__ void wait_vm(int n) {
#define MLA_VM(N) \
  case N: __builtin_amdgcn_s_waitcnt(0x3f70 | ((N) & 0xf) | (((N) >> 4) << 14)); break;
  switch (n) {
    MLA_VM(0) MLA_VM(1) MLA_VM(2) MLA_VM(3) MLA_VM(4) MLA_VM(5) MLA_VM(6) MLA_VM(7)
    MLA_VM(8) MLA_VM(9) MLA_VM(10) MLA_VM(11) MLA_VM(12) MLA_VM(13) MLA_VM(14) MLA_VM(15)
    MLA_VM(16) MLA_VM(17) MLA_VM(18) MLA_VM(19) MLA_VM(20) MLA_VM(21) MLA_VM(22) MLA_VM(23)
    MLA_VM(24) MLA_VM(25) MLA_VM(26) MLA_VM(27) MLA_VM(28) MLA_VM(29) MLA_VM(30) MLA_VM(31)
    MLA_VM(32) MLA_VM(33) MLA_VM(34) MLA_VM(35) MLA_VM(36) MLA_VM(37) MLA_VM(38) MLA_VM(39)
    MLA_VM(40) MLA_VM(41) MLA_VM(42) MLA_VM(43) MLA_VM(44) MLA_VM(45) MLA_VM(46) MLA_VM(47)
    default: __builtin_amdgcn_s_waitcnt(0x3f70 | 0xf | (3 << 14)); break;  // 63
  }
#undef MLA_VM
}

// Per-tile descriptor flags (low byte: valid rows of the tile).
enum : int {
  kFirstOfSeg = 1 << 8,   // first tile of a query token within this range
  kLastOfSeg = 1 << 9,    // last tile of a query token within this range
  kWhole = 1 << 10,       // the token's rows all lie in this range: write o_lat
  kBad = 1 << 11,         // block-table entry out of range: skipped
  kSecondSlot = 1 << 12,  // not the range's first token: partial goes to slot 2w+1
};

// Walks the tiles (half cache blocks) of one workgroup's unit range in order.
// Every field is wave-uniform.  The block-table entry of a block is read when
// the walk enters it, one tile ahead of its issue for the second half.
struct Loader {
  TokenCursor c;
  int u1;
  int ub, ub_beg, ub_end;  // block range of the current segment (within the token)
  int half;
  int rows;     // valid rows of the current block
  int nvalid;   // valid rows of the current tile (1..32)
  int blk_raw;  // block-table entry of the current block
  int valid;
  int first;    // first tile of a segment
  int nseg;     // segments entered so far

  __device__ __forceinline__ void fill(const PlanArgs& p, const int32_t* bt, int stride,
                                       bool new_block) {
    const int A = p.causal ? c.L - c.q + c.j + 1 : c.L;
    rows = uni(min(kBS, A - ub * kBS));
    nvalid = min(kTile, rows - kTile * half);
    if (new_block) blk_raw = ldc(bt, c.b * stride + ub);  // host keeps B*stride < 2^31
  }
  __device__ __forceinline__ void init(const PlanArgs& p, const int32_t* bt, int stride, int u0,
                                       int u1_) {
    u1 = u1_;
    c = locate_unit(p, u0);
    ub = ub_beg = u0 - c.ts;
    ub_end = uni(min(u1, c.ts + c.nu) - c.ts);
    half = 0;
    valid = 1;
    first = 1;
    nseg = 0;
    fill(p, bt, stride, true);
  }
  __device__ __forceinline__ bool last_of_segment() const {
    return ub == ub_end - 1 && (half == 1 || rows <= kTile);
  }
  __device__ __forceinline__ bool whole_token() const { return ub_beg == 0 && ub_end == c.nu; }
  __device__ __forceinline__ void next(const PlanArgs& p, const int32_t* bt, int stride) {
    first = 0;
    if (half == 0 && rows > kTile) {
      half = 1;
      fill(p, bt, stride, false);
      return;
    }
    half = 0;
    ++ub;
    if (ub == ub_end) {
      if (c.ts + c.nu >= u1) {
        valid = 0;
        return;
      }
      cursor_next(p, c);
      ub = ub_beg = 0;
      ub_end = uni(min(u1, c.ts + c.nu) - c.ts);
      first = 1;
      ++nseg;
    }
    fill(p, bt, stride, true);
  }
};

// max / sum over the 4 lanes that share a head (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float head_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float head_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace tiles
}  // namespace mla
