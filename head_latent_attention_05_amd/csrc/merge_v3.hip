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
// Workgroup = one token x 16/R heads in 4 waves, R = 1, 2 or 4 range groups:
// wave v is range group v % R for head quad v / R, and a lane owns one head x 32
// features.  Group rg takes ranges wlo + rg, wlo + rg + R, ..., four per round
// with all their loads in flight, combining rounds online; with R > 1 the
// groups' (maximum, denominator, weighted sum) meet in LDS and are combined in
// increasing rg.  R trades workgroups for round trips; the host picks it from
// the most-split token and the token count.
// The token's unit range comes from one wave-parallel pass over the sequences.
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

template <int kRG>
__global__ __launch_bounds__(256) void merge_v3_kernel(PlanArgs p, const float* __restrict__ ws_lse,
                                                       const uint16_t* __restrict__ ws_o,
                                                       uint16_t* __restrict__ o_lat) {
  constexpr int kHG = 16 / kRG;  // heads per workgroup
  constexpr int kSl = 256 / kRG;  // lanes of one range group
  __shared__ float st_m[kRG][kSl];     // per range group: running maximum,
  __shared__ float st_d[kRG][kSl];     // denominator
  __shared__ f32x4 st_a[kRG][8][kSl];  // and weighted sum of 32 features
  p.block_size = kBS;  // a compile-time block size turns the unit arithmetic into shifts
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int rg = wave % kRG, hq = wave / kRG;
  const int sl = 64 * hq + lane;  // this lane's index within its range group
  const int h = blockIdx.y * kHG + 4 * hq + (lane >> 4);
  const int f0 = (lane & 15) * 32;
  int ts, nu;
  locate_token(p, t, ts, nu);
  // ranges clamped to [0, G): device lengths that disagree with the host's (the
  // decode kernel flags that) must not take a slot index out of the workspace
  const int64_t whi = max<int64_t>(0, min<int64_t>(range_of((int64_t)ts + nu - 1, p.U, p.G), p.G - 1));
  const int64_t wlo = max<int64_t>(0, min<int64_t>(range_of(ts, p.U, p.G), whi));
  if (wlo == whi) return;  // finished in place by one workgroup
  const int64_t slot_lo = range_start(wlo, p.U, p.G) == ts ? 2 * wlo : 2 * wlo + 1;

  // Range group rg takes ranges wlo + rg + kRG*j, four per round with
  // branch-free loads (indices past the last range repeat it and get weight 0),
  // combining rounds online: running maximum, earlier sums rescaled when it grows.
  float mx = -INFINITY, den = 0.f;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  for (int64_t w0 = wlo + rg; w0 <= whi; w0 += 4 * kRG) {
    u32x4 x[4][4];
    float l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t slot = slot_of(min(w0 + kRG * j, whi), wlo, slot_lo);
      load4(ws_o + (slot * kH + h) * kDC + f0, x[j]);
      l[j] = ws_lse[slot * kH + h];
    }
#pragma unroll
    for (int j = 1; j < 4; ++j) l[j] = w0 + kRG * j <= whi ? l[j] : -INFINITY;
    const float mn = fmaxf(mx, fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3])));
    const float sc = exp2f(mx - mn);  // 0 in the first round (mx = -inf, mn finite)
    den *= sc;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] *= sc;
    mx = mn;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = exp2f(l[j] - mx);
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
  f32x4 A[8];
  float D;
  if constexpr (kRG == 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
    D = den;
  } else {
    // a group without ranges keeps (-inf, 0, 0), which adds nothing below
    st_m[rg][sl] = mx;
    st_d[rg][sl] = den;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      st_a[rg][i][sl] = f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
    __syncthreads();
    if (rg != 0) return;
    float M = st_m[0][sl];  // group 0 always holds range wlo: finite
#pragma unroll
    for (int r = 1; r < kRG; ++r) M = fmaxf(M, st_m[r][sl]);
    D = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < kRG; ++r) {
      const float e = exp2f(st_m[r][sl] - M);
      D += e * st_d[r][sl];
#pragma unroll
      for (int i = 0; i < 8; ++i) A[i] += e * st_a[r][i][sl];
    }
  }
  const float inv = 1.f / D;
  u32x4* dst = (u32x4*)(o_lat + ((int64_t)t * kH + h) * kDC + f0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    dst[i] = u32x4{pack_bf16x2(A[2 * i][0] * inv, A[2 * i][1] * inv),
                   pack_bf16x2(A[2 * i][2] * inv, A[2 * i][3] * inv),
                   pack_bf16x2(A[2 * i + 1][0] * inv, A[2 * i + 1][1] * inv),
                   pack_bf16x2(A[2 * i + 1][2] * inv, A[2 * i + 1][3] * inv)};
}

}  // namespace

hipError_t launch_merge_v3(const DecodeArgs& a, hipStream_t st) {
  const int rg = a.merge_groups;
  const dim3 grid(a.plan.T, kH * rg / 16);
  const uint16_t* ws_o = (const uint16_t*)a.ws_o;
  uint16_t* o_lat = (uint16_t*)a.o_lat;
  if (rg == 1)
    hipLaunchKernelGGL(merge_v3_kernel<1>, grid, dim3(256), 0, st, a.plan, a.ws_lse, ws_o, o_lat);
  else if (rg == 2)
    hipLaunchKernelGGL(merge_v3_kernel<2>, grid, dim3(256), 0, st, a.plan, a.ws_lse, ws_o, o_lat);
  else
    hipLaunchKernelGGL(merge_v3_kernel<4>, grid, dim3(256), 0, st, a.plan, a.ws_lse, ws_o, o_lat);
  return hipGetLastError();
}

}  // namespace mla
