// Device-side walk of the split plan (see PlanArgs in mla_internal.h).  Every
// wave evaluates it redundantly from the device length arrays, so the kernels
// need no plan buffer and the host no upload.
#pragma once

#include "mla_internal.h"

namespace mla {

__device__ __forceinline__ int64_t wave_incl_scan(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int64_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ int64_t seq_units(const PlanArgs& p, int b) {
  int64_t L = p.kv_lens[b];
  int64_t q = (int64_t)p.q_start[b + 1] - p.q_start[b];
  return seq_units_before(L, q, q, p.block_size, p.causal);
}

// Sum of the units of sequences [0, b_end).  Wave-uniform result.
__device__ inline int64_t units_before_seq(const PlanArgs& p, int b_end) {
  const int lane = threadIdx.x & 63;
  int64_t acc = 0;
  for (int base = 0; base < b_end; base += 64) {
    int b = base + lane;
    int64_t v = (b < b_end) ? seq_units(p, b) : 0;
    v = wave_incl_scan(v);
    acc += __shfl(v, 63, 64);
  }
  return acc;
}

struct TokenCursor {
  int b;          // sequence
  int j;          // query token index within the sequence
  int64_t L, q;   // kv length and query count of b
  int64_t ts;     // first unit of this token
  int64_t nu;     // units of this token
  int t;          // global query-token index
};

__device__ inline void cursor_fill(const PlanArgs& p, TokenCursor& c) {
  c.L = p.kv_lens[c.b];
  c.q = (int64_t)p.q_start[c.b + 1] - p.q_start[c.b];
  int64_t A = attend_len(c.L, c.q, c.j, p.causal);
  c.nu = (A + p.block_size - 1) / p.block_size;
  c.t = p.q_start[c.b] + c.j;
}

// Token holding unit u (0 <= u < U).  Wave-uniform.
__device__ inline TokenCursor locate_unit(const PlanArgs& p, int64_t u) {
  const int lane = threadIdx.x & 63;
  TokenCursor c;
  int64_t acc = 0;
  int found = -1;
  int64_t before = 0;
  for (int base = 0; base < p.B && found < 0; base += 64) {
    int b = base + lane;
    int64_t v = (b < p.B) ? seq_units(p, b) : 0;
    int64_t incl = wave_incl_scan(v) + acc;
    // first lane whose inclusive prefix exceeds u
    unsigned long long m = __ballot(b < p.B && incl > u);
    if (m) {
      int l = __ffsll((long long)m) - 1;
      found = base + l;
      before = __shfl(incl - v, l, 64);
    }
    acc = __shfl(incl, 63, 64);
  }
  if (found < 0) found = p.B - 1;  // only reachable with inconsistent lengths
  c.b = found;
  int64_t L = p.kv_lens[found];
  int64_t q = (int64_t)p.q_start[found + 1] - p.q_start[found];
  int64_t rem = u - before;
  int j;
  if (!p.causal) {
    int64_t nb = (L + p.block_size - 1) / p.block_size;
    j = (int)(rem / nb);
  } else {  // largest j with units_before(j) <= rem
    int lo = 0, hi = (int)q - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (seq_units_before(L, q, mid, p.block_size, 1) <= rem) lo = mid; else hi = mid - 1;
    }
    j = lo;
  }
  if (j >= q) j = (int)q - 1;
  c.j = j;
  c.ts = before + seq_units_before(L, q, j, p.block_size, p.causal);
  cursor_fill(p, c);
  return c;
}

// Advance to the next token that has at least one unit.
__device__ inline void cursor_next(const PlanArgs& p, TokenCursor& c) {
  c.ts += c.nu;
  c.j += 1;
  while (c.j >= c.q && c.b + 1 < p.B) {
    c.b += 1;
    c.j = 0;
    c.q = (int64_t)p.q_start[c.b + 1] - p.q_start[c.b];
  }
  cursor_fill(p, c);
}

// Sequence index of global query token t (largest b with q_start[b] <= t).
__device__ inline int seq_of_token(const PlanArgs& p, int t) {
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (p.q_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace mla
