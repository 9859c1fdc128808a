// Device-side walk of the split plan (see PlanArgs in mla_internal.h).  Every
// wave evaluates it redundantly from the device length arrays, so the kernels
// need no plan buffer and the host no upload.  Unit counts fit in 32 bits (the
// host rejects plans with 2^31 or more units).
#pragma once

#include "mla_internal.h"

namespace mla {

// Wave-uniform copies in scalar registers (the plan walk is identical in every
// lane; keeping it scalar keeps its loads on the scalar path).
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Loads of the length arrays and the block table go through the constant
// address space: they are read-only for the whole call, so uniform loads can use
// the scalar cache even in kernels that also write global memory.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ int ldc(const int32_t* p, int64_t i) {
  return ((const_i32_ptr)p)[i];
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// units of query tokens j < jn of sequence b
__device__ __forceinline__ int seq_units_upto(const PlanArgs& p, int L, int q, int jn) {
  return (int)seq_units_before(L, q, jn, p.block_size, p.causal);
}

__device__ __forceinline__ int seq_units(const PlanArgs& p, int b) {
  const int L = ldc(p.kv_lens, b);
  const int q = ldc(p.q_start, b + 1) - ldc(p.q_start, b);
  return seq_units_upto(p, L, q, q);
}

// Sum of the units of sequences [0, b_end).  Wave-uniform result.
__device__ inline int units_before_seq(const PlanArgs& p, int b_end) {
  const int lane = threadIdx.x & 63;
  int acc = 0;
  for (int base = 0; base < b_end; base += 64) {
    const int b = base + lane;
    int v = (b < b_end) ? seq_units(p, b) : 0;
    v = wave_incl_scan(v);
    acc += __shfl(v, 63, 64);
  }
  return uni(acc);
}

// True when the device length arrays describe a valid batch whose unit and
// query-token totals equal the host plan's (U, T): q_start[0] = 0, every
// sequence has 0 <= q <= L, L >= 1 and ceil(L / block_size) <= max_blocks,
// q_start[B] = T and the units add up to U.  Every index the kernels derive
// from the device arrays (token, block-table column, unit, range, partial
// slot) then stays inside buffers sized from the host copies.  Wave-uniform.
__device__ inline bool plan_consistent(const PlanArgs& p, int max_blocks) {
  const int lane = threadIdx.x & 63;
  int64_t tot = 0;
  int bad = (ldc(p.q_start, 0) != 0 || ldc(p.q_start, p.B) != p.T) ? 1 : 0;
  for (int base = 0; base < p.B; base += 64) {
    const int b = base + lane;
    int64_t v = 0;
    if (b < p.B) {
      const int q = ldc(p.q_start, b + 1) - ldc(p.q_start, b);
      const int L = ldc(p.kv_lens, b);
      if (q < 0 || L < 1 || q > L || (L + p.block_size - 1) / p.block_size > max_blocks)
        bad = 1;
      else
        v = seq_units_before(L, q, q, p.block_size, p.causal);
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) v += __shfl_xor(v, d, 64);
    tot += v;
  }
  return __ballot(bad) == 0 && uni((int)(tot == p.U)) != 0;
}

struct TokenCursor {
  int b;   // sequence
  int j;   // query token index within the sequence
  int L;   // kv length of b
  int q;   // query tokens of b
  int ts;  // first unit of this token
  int nu;  // units of this token
  int t;   // global query-token index
};

__device__ __forceinline__ void cursor_fill(const PlanArgs& p, TokenCursor& c) {
  c.b = uni(c.b);
  c.j = uni(c.j);
  c.ts = uni(c.ts);
  const int qs = uni(ldc(p.q_start, c.b));
  c.L = uni(ldc(p.kv_lens, c.b));
  c.q = uni(ldc(p.q_start, c.b + 1)) - qs;
  const int A = p.causal ? c.L - c.q + c.j + 1 : c.L;
  c.nu = (A + p.block_size - 1) / p.block_size;
  c.t = qs + c.j;
}

// Token holding unit u (0 <= u < U).  Wave-uniform (scalar) result.
__device__ __forceinline__ TokenCursor locate_unit(const PlanArgs& p, int u) {
  const int lane = threadIdx.x & 63;
  TokenCursor c;
  int acc = 0, found = -1, before = 0;
  for (int base = 0; base < p.B && found < 0; base += 64) {
    const int b = base + lane;
    const int v = (b < p.B) ? seq_units(p, b) : 0;
    const int incl = wave_incl_scan(v) + acc;
    // first lane whose inclusive prefix exceeds u
    const unsigned long long m = __ballot(b < p.B && incl > u);
    if (m) {
      const int l = __ffsll((long long)m) - 1;
      found = base + l;
      before = __shfl(incl - v, l, 64);
    }
    acc = __shfl(incl, 63, 64);
  }
  if (found < 0) found = p.B - 1;  // only reachable with inconsistent lengths
  c.b = uni(found);
  before = uni(before);
  const int L = ldc(p.kv_lens, c.b);
  const int q = ldc(p.q_start, c.b + 1) - ldc(p.q_start, c.b);
  const int rem = u - before;
  int j;
  if (!p.causal) {
    const int nb = (L + p.block_size - 1) / p.block_size;
    j = rem / nb;
  } else {  // largest j with units_before(j) <= rem
    int lo = 0, hi = q - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seq_units_upto(p, L, q, mid) <= rem) lo = mid; else hi = mid - 1;
    }
    j = lo;
  }
  if (j >= q) j = q - 1;
  c.j = uni(j);
  c.ts = before + seq_units_upto(p, L, q, c.j);
  cursor_fill(p, c);
  return c;
}

// Advance to the next token that has at least one unit.
__device__ __forceinline__ void cursor_next(const PlanArgs& p, TokenCursor& c) {
  c.ts += c.nu;
  c.j += 1;
  while (c.j >= c.q && c.b + 1 < p.B) {
    c.b = uni(c.b + 1);
    c.j = 0;
    c.q = uni(ldc(p.q_start, c.b + 1) - ldc(p.q_start, c.b));
  }
  cursor_fill(p, c);
}

// First unit (ts) and unit count (nu) of global query token t, from one
// wave-parallel pass over the sequences.  Wave-uniform results.
__device__ inline void locate_token(const PlanArgs& p, int t, int& ts, int& nu) {
  const int lane = threadIdx.x & 63;
  int acc = 0, f_ts = 0, f_nu = 0;
  for (int base = 0; base < p.B; base += 64) {
    const int b = base + lane;
    int qs0 = 0, qs1 = 0, L = 0, v = 0;
    if (b < p.B) {
      qs0 = ldc(p.q_start, b);
      qs1 = ldc(p.q_start, b + 1);
      L = ldc(p.kv_lens, b);
      v = seq_units_upto(p, L, qs1 - qs0, qs1 - qs0);
    }
    const int incl = wave_incl_scan(v) + acc;
    const bool mine = b < p.B && qs0 <= t && t < qs1;
    const unsigned long long m = __ballot(mine);
    if (m) {  // wave-uniform
      int my_ts = 0, my_nu = 0;
      if (mine) {
        const int q = qs1 - qs0, j = t - qs0;
        my_ts = incl - v + seq_units_upto(p, L, q, j);
        const int A = p.causal ? L - q + j + 1 : L;
        my_nu = (A + p.block_size - 1) / p.block_size;
      }
      const int l = __ffsll((long long)m) - 1;
      f_ts = __shfl(my_ts, l, 64);
      f_nu = __shfl(my_nu, l, 64);
      break;
    }
    acc = __shfl(incl, 63, 64);
  }
  ts = uni(f_ts);
  nu = uni(f_nu);
}

// Sequence index of global query token t (largest b with q_start[b] <= t).
__device__ inline int seq_of_token(const PlanArgs& p, int t) {
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (ldc(p.q_start, mid) <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace mla
