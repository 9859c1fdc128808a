// Split-KV absorbed latent attention, generic version (any supported dims, fp32
// or bf16 storage), and the split merge.
//
// [MLA explainer] stage 2B and forward_inference_absorbed: the score of a cached
// token is the latent score q_lat.c_kv plus the RoPE score q_pe.k_pe, scaled by
// 1/sqrt(d_nope + d_rope); the output is the softmax-weighted sum of the cached
// latents c_kv.  Both scores are one dot product over the 576-wide row here.
//
// Work split (see PlanArgs): grid.x = KV workgroups, grid.y = groups of 4 heads.
// One wave per head; lanes stride over the row; per cached row the wave reduces
// the score, then updates a running max / sum / accumulator (online softmax in
// the log2 domain).  This is the all-fp32 test path and a cross-check for the
// MFMA kernel; the V3 bf16 hot path lives in decode_v3.hip.
#include <math.h>

#include "plan_device.h"

namespace mla {
namespace {

constexpr int kMaxRowPerLane = 9;  // row <= 576
constexpr int kMaxLatPerLane = 8;  // d_c <= 512, d_c % 64 == 0

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

template <typename S>
__global__ __launch_bounds__(256) void decode_generic_kernel(DecodeArgs a, int H, int dc, int dr) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + wave;
  if (h >= H) return;
  const int row = dc + dr;
  const int nlat = dc >> 6;
  const int64_t w = blockIdx.x;
  const PlanArgs& p = a.plan;
  if (!plan_consistent(p, a.max_blocks)) {  // device lengths disagree with the host plan
    if (w == 0 && blockIdx.y == 0 && threadIdx.x == 0 && a.err) atomicOr(a.err, MLA_DEVERR_LENGTH);
    return;
  }
  const int64_t u0 = range_start(w, p.U, p.G), u1 = range_start(w + 1, p.U, p.G);
  if (u0 >= u1) return;
  const S* pool = (const S*)a.pool;
  const S* qlat = (const S*)a.q_lat;
  const int bs = p.block_size;
  TokenCursor c = locate_unit(p, (int)u0);
  bool first = true;
  while (true) {
    const int64_t seg_s = max(u0, c.ts), seg_e = min(u1, c.ts + c.nu);
    const int64_t A = attend_len(c.L, c.q, c.j, p.causal);
    float q[kMaxRowPerLane];
#pragma unroll
    for (int r = 0; r < kMaxRowPerLane; ++r) {
      int idx = lane + 64 * r;
      q[r] = idx < row ? Storage<S>::load(qlat + ((int64_t)c.t * H + h) * row + idx) : 0.f;
    }
    float m = -INFINITY, l = 0.f;
    float acc[kMaxLatPerLane];
#pragma unroll
    for (int r = 0; r < kMaxLatPerLane; ++r) acc[r] = 0.f;
    for (int64_t ub = seg_s - c.ts; ub < seg_e - c.ts; ++ub) {
      int64_t blk = a.block_table[(int64_t)c.b * a.max_blocks + ub];
      if (blk < 0 || blk >= a.num_blocks) {
        if (lane == 0 && a.err) atomicOr(a.err, MLA_DEVERR_BLOCK);
        continue;
      }
      const int64_t r0 = ub * bs;
      const int nrows = (int)min((int64_t)bs, A - r0);
      for (int rr = 0; rr < nrows; ++rr) {
        const S* x = pool + (blk * bs + rr) * (int64_t)row;
        float xv[kMaxRowPerLane];
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < kMaxRowPerLane; ++r) {
          int idx = lane + 64 * r;
          xv[r] = idx < row ? Storage<S>::load(x + idx) : 0.f;
          part += q[r] * xv[r];
        }
        float s2 = wave_sum(part) * a.scale_log2;
        float mn = fmaxf(m, s2);
        float alpha = exp2f(m - mn);
        float pe = exp2f(s2 - mn);
        l = l * alpha + pe;
#pragma unroll
        for (int r = 0; r < kMaxLatPerLane; ++r)
          if (r < nlat) acc[r] = acc[r] * alpha + pe * xv[r];
        m = mn;
      }
    }
    const float inv = 1.f / l;
    if (seg_s == c.ts && seg_e == c.ts + c.nu) {
      S* o = (S*)a.o_lat + ((int64_t)c.t * H + h) * dc;
#pragma unroll
      for (int r = 0; r < kMaxLatPerLane; ++r)
        if (r < nlat) Storage<S>::store(o + lane + 64 * r, acc[r] * inv);
    } else {
      const int64_t slot = first ? 2 * w : 2 * w + 1;
      S* o = (S*)a.ws_o + (slot * H + h) * dc;
#pragma unroll
      for (int r = 0; r < kMaxLatPerLane; ++r)
        if (r < nlat) Storage<S>::store(o + lane + 64 * r, acc[r] * inv);
      if (lane == 0) a.ws_lse[slot * H + h] = m + log2f(l);
    }
    if (seg_e >= u1) break;
    cursor_next(p, c);
    first = false;
  }
}

// One wave per (query token, head): combine the partials of a token that was
// split over several KV workgroups, in increasing workgroup order.
template <typename S>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a, int H, int dc) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + wave;
  if (h >= H) return;
  const int t = blockIdx.x;
  const PlanArgs& p = a.plan;
  const int b = seq_of_token(p, t);
  const int L = p.kv_lens[b];
  const int q = p.q_start[b + 1] - p.q_start[b];
  const int j = t - p.q_start[b];
  const int64_t ts = units_before_seq(p, b) + seq_units_before(L, q, j, p.block_size, p.causal);
  const int64_t nu = (attend_len(L, q, j, p.causal) + p.block_size - 1) / p.block_size;
  // ranges clamped to [0, G): device lengths that disagree with the host's (the
  // decode kernel flags that) must not take a slot index out of the workspace
  const int64_t whi = max<int64_t>(0, min<int64_t>(range_of((int64_t)ts + nu - 1, p.U, p.G), p.G - 1));
  const int64_t wlo = max<int64_t>(0, min<int64_t>(range_of(ts, p.U, p.G), whi));
  if (wlo == whi) return;  // finished in place by one workgroup
  const int nlat = dc >> 6;
  float mx = -INFINITY;
  for (int64_t w = wlo; w <= whi; ++w) {
    const int64_t slot = range_start(w, p.U, p.G) >= ts ? 2 * w : 2 * w + 1;
    mx = fmaxf(mx, a.ws_lse[slot * H + h]);
  }
  float acc[kMaxLatPerLane];
#pragma unroll
  for (int r = 0; r < kMaxLatPerLane; ++r) acc[r] = 0.f;
  float den = 0.f;
  for (int64_t w = wlo; w <= whi; ++w) {
    const int64_t slot = range_start(w, p.U, p.G) >= ts ? 2 * w : 2 * w + 1;
    const float e = exp2f(a.ws_lse[slot * H + h] - mx);
    den += e;
    const S* o = (const S*)a.ws_o + (slot * H + h) * dc;
#pragma unroll
    for (int r = 0; r < kMaxLatPerLane; ++r)
      if (r < nlat) acc[r] += e * Storage<S>::load(o + lane + 64 * r);
  }
  const float inv = 1.f / den;
  S* o = (S*)a.o_lat + ((int64_t)t * H + h) * dc;
#pragma unroll
  for (int r = 0; r < kMaxLatPerLane; ++r)
    if (r < nlat) Storage<S>::store(o + lane + 64 * r, acc[r] * inv);
}

}  // namespace

hipError_t launch_decode_generic(const mla_config& c, const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.plan.G, (c.num_heads + 3) / 4), block(256);
  if (c.dtype == MLA_BF16)
    hipLaunchKernelGGL(decode_generic_kernel<uint16_t>, grid, block, 0, st, a, c.num_heads,
                       c.d_latent, c.d_rope);
  else
    hipLaunchKernelGGL(decode_generic_kernel<float>, grid, block, 0, st, a, c.num_heads,
                       c.d_latent, c.d_rope);
  return hipGetLastError();
}

hipError_t launch_merge(const mla_config& c, const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.plan.T, (c.num_heads + 3) / 4), block(256);
  if (c.dtype == MLA_BF16)
    hipLaunchKernelGGL(merge_kernel<uint16_t>, grid, block, 0, st, a, c.num_heads, c.d_latent);
  else
    hipLaunchKernelGGL(merge_kernel<float>, grid, block, 0, st, a, c.num_heads, c.d_latent);
  return hipGetLastError();
}

}  // namespace mla
