// Merge of split-KV partial results for DeepSeek-V3 shapes (128 heads, 512
// latent features, bf16 partials).
//
// A token whose cache blocks were split over KV ranges wlo..whi has, per range,
// an output normalised over that range's rows and the log2-sum-exp of its
// scaled scores.  The softmax over all rows is the lse-weighted mix:
//   o = sum_w 2^(lse_w - M) o_w / sum_w 2^(lse_w - M),   M = max_w lse_w,
// taken in a fixed order, so results are deterministic for a split plan.  This
// is the online-softmax identity that [MLA explainer] stage 2B's softmax
// reduces to when its rows are processed in pieces.
//
// Workgroup = one token x 4 heads, one wave per head; a lane owns 8 features,
// so every range's partial of the head is one 16-byte load per lane.  Eight
// ranges per round are in flight, and rounds combine online (running maximum,
// earlier sums rescaled when it grows) in increasing range order.  The kernel
// holds few registers, so the grid of a large batch is resident at once and
// the merge streams the partials at close to the copy rate; a token split over
// many ranges (a single long sequence) takes one round per eight ranges.  The
// token's unit range comes from one wave-parallel pass over the sequences.
#include <math.h>

#include "plan_device.h"

namespace mla {
namespace {

constexpr int kH = 128;
constexpr int kDC = 512;
constexpr int kBS = 64;

// Partial slot of range w for a token whose first unit is ts, among the ranges
// wlo..whi that touch it: a range after wlo starts inside the token, so the
// token is that range's first segment (slot 2w); range wlo holds it as its
// first segment (2w) only if it starts exactly at ts, else as its last (2w+1).
__device__ __forceinline__ int64_t slot_of(int64_t w, int64_t wlo, int64_t slot_lo) {
  return w == wlo ? slot_lo : 2 * w;
}

__global__ __launch_bounds__(256) void merge_v3_kernel(PlanArgs p, const float* __restrict__ ws_lse,
                                                       const uint16_t* __restrict__ ws_o,
                                                       uint16_t* __restrict__ o_lat) {
  p.block_size = kBS;
  const int t = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int f0 = (threadIdx.x & 63) * 8;
  int ts, nu;
  locate_token(p, t, ts, nu);
  const int64_t whi = max<int64_t>(0, min<int64_t>(range_of((int64_t)ts + nu - 1, p.U, p.G), p.G - 1));
  const int64_t wlo = max<int64_t>(0, min<int64_t>(range_of(ts, p.U, p.G), whi));
  if (wlo == whi) return;  // finished in place by one workgroup
  const int64_t slot_lo = range_start(wlo, p.U, p.G) == ts ? 2 * wlo : 2 * wlo + 1;
  float mx = -INFINITY, den = 0.f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int64_t w0 = wlo; w0 <= whi; w0 += 8) {
    u32x4 x[8];
    float l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t slot = slot_of(min(w0 + j, whi), wlo, slot_lo);
      x[j] = *(const u32x4*)(ws_o + (slot * kH + h) * kDC + f0);
      l[j] = ws_lse[slot * kH + h];
    }
#pragma unroll
    for (int j = 1; j < 8; ++j) l[j] = w0 + j <= whi ? l[j] : -INFINITY;
    float mn = mx;
#pragma unroll
    for (int j = 0; j < 8; ++j) mn = fmaxf(mn, l[j]);
    const float sc = exp2f(mx - mn);  // 0 in the first round (mx = -inf, mn finite)
    den *= sc;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= sc;
    mx = mn;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = exp2f(l[j] - mx);
      den += e;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] += e * __uint_as_float(x[j][k] << 16);
        acc[2 * k + 1] += e * __uint_as_float(x[j][k] & 0xffff0000u);
      }
    }
  }
  const float inv = 1.f / den;
  *(u32x4*)(o_lat + ((int64_t)t * kH + h) * kDC + f0) =
      u32x4{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
            pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
}

}  // namespace

hipError_t launch_merge_v3(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(merge_v3_kernel, dim3(a.plan.T, kH / 4), dim3(256), 0, st, a.plan, a.ws_lse,
                     (const uint16_t*)a.ws_o, (uint16_t*)a.o_lat);
  return hipGetLastError();
}

}  // namespace mla
