// Merge of split-KV partial results for DeepSeek-V3 shapes (128 heads, 512
// latent features, bf16 partials).
//
// A token whose cache blocks were split over KV ranges wlo..whi has, per range,
// an output normalised over that range's rows and the log2-sum-exp of its
// scaled scores.  The softmax over all rows is the lse-weighted mix:
//   o = sum_w 2^(lse_w - M) o_w / sum_w 2^(lse_w - M),   M = max_w lse_w,
// taken in increasing w, so results are deterministic for a split plan.  This
// is the online-softmax identity that [MLA explainer] stage 2B's softmax
// reduces to when its rows are processed in pieces.
//
// Workgroup = one token x 16 heads; thread = one head x 32 features (four
// 16-byte loads per range, four ranges' loads in flight together).  The
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

__device__ __forceinline__ void load4(const uint16_t* p, u32x4* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = ((const u32x4*)p)[i];
}

__global__ __launch_bounds__(256) void merge_v3_kernel(PlanArgs p, const float* __restrict__ ws_lse,
                                                       const uint16_t* __restrict__ ws_o,
                                                       uint16_t* __restrict__ o_lat) {
  p.block_size = kBS;  // a compile-time block size turns the unit arithmetic into shifts
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int h = blockIdx.y * 16 + (tid >> 4);
  const int f0 = (tid & 15) * 32;
  int ts, nu;
  locate_token(p, t, ts, nu);
  // ranges clamped to [0, G): device lengths that disagree with the host's (the
  // decode kernel flags that) must not take a slot index out of the workspace
  const int64_t whi = max<int64_t>(0, min<int64_t>(range_of((int64_t)ts + nu - 1, p.U, p.G), p.G - 1));
  const int64_t wlo = max<int64_t>(0, min<int64_t>(range_of(ts, p.U, p.G), whi));
  if (wlo == whi) return;  // finished in place by one workgroup
  const int64_t slot_lo = range_start(wlo, p.U, p.G) == ts ? 2 * wlo : 2 * wlo + 1;

  // Ranges are taken four at a time with branch-free loads (indices past the
  // last range repeat it and get weight 0), so a token's partials are all in
  // flight together for up to four ranges.
  float mx = -INFINITY;
  for (int64_t w = wlo; w <= whi; w += 4) {
    float l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) l[j] = ws_lse[slot_of(min(w + j, whi), wlo, slot_lo) * kH + h];
    mx = fmaxf(mx, fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3])));
  }

  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  float den = 0.f;
  for (int64_t w = wlo; w <= whi; w += 4) {
    u32x4 x[4][4];
    float l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t slot = slot_of(min(w + j, whi), wlo, slot_lo);
      load4(ws_o + (slot * kH + h) * kDC + f0, x[j]);
      l[j] = ws_lse[slot * kH + h];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = w + j <= whi ? exp2f(l[j] - mx) : 0.f;
      den += e;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[8 * i + 2 * k] += e * __uint_as_float(x[j][i][k] << 16);
          acc[8 * i + 2 * k + 1] += e * __uint_as_float(x[j][i][k] & 0xffff0000u);
        }
    }
  }
  const float inv = 1.f / den;
  u32x4* dst = (u32x4*)(o_lat + ((int64_t)t * kH + h) * kDC + f0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dst[i] = u32x4{pack_bf16x2(acc[8 * i] * inv, acc[8 * i + 1] * inv),
                   pack_bf16x2(acc[8 * i + 2] * inv, acc[8 * i + 3] * inv),
                   pack_bf16x2(acc[8 * i + 4] * inv, acc[8 * i + 5] * inv),
                   pack_bf16x2(acc[8 * i + 6] * inv, acc[8 * i + 7] * inv)};
}

}  // namespace

hipError_t launch_merge_v3(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(merge_v3_kernel, dim3(a.plan.T, kH / 16), dim3(256), 0, st, a.plan,
                     a.ws_lse, (const uint16_t*)a.ws_o, (uint16_t*)a.o_lat);
  return hipGetLastError();
}

}  // namespace mla
