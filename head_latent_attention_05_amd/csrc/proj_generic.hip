// Per-head projections on both sides of the latent attention, generic version.
//
// absorb_q : q_lat[t][h][c] = sum_d q_nope[t][h][d] * W_UK[h][d][c]
//            ([MLA explainer] stage 2B / forward_inference_absorbed: the query is
//            taken into the latent space through W_UK; [MLA deep dive] 2.3)
// out_proj : out[t][h][v]   = sum_c o_lat[t][h][c] * W_UV[h][v][c]
//            ([MLA explainer] forward_inference_absorbed: the attended latent goes
//            through W_UV per head)
// fp32 accumulation.  Used for the fp32 test mode and as the fallback for bf16
// shapes the MFMA kernels do not cover.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kTokTile = 8;

// grid: (ceil(dc/256), H, ceil(T/8)); thread = one latent column, 8 tokens.
template <typename S>
__global__ __launch_bounds__(256) void absorb_generic_kernel(int T, int H, int dn, int dc, int dr,
                                                             const S* __restrict__ q_nope,
                                                             const S* __restrict__ w_uk,
                                                             S* __restrict__ q_lat) {
  __shared__ float qs[kTokTile][256];
  const int h = blockIdx.y;
  const int t0 = blockIdx.z * kTokTile;
  const int nt = min(kTokTile, T - t0);
  for (int k = threadIdx.x; k < kTokTile * dn; k += blockDim.x) {
    int tt = k / dn, d = k - tt * dn;
    qs[tt][d] = tt < nt ? Storage<S>::load(q_nope + ((int64_t)(t0 + tt) * H + h) * dn + d) : 0.f;
  }
  __syncthreads();
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= dc) return;
  float acc[kTokTile] = {};
  const S* w = w_uk + (int64_t)h * dn * dc + col;
  for (int d = 0; d < dn; ++d) {
    float wv = Storage<S>::load(w + (int64_t)d * dc);
#pragma unroll
    for (int tt = 0; tt < kTokTile; ++tt) acc[tt] += qs[tt][d] * wv;
  }
  const int row = dc + dr;
  for (int tt = 0; tt < nt; ++tt)
    Storage<S>::store(q_lat + ((int64_t)(t0 + tt) * H + h) * row + col, acc[tt]);
}

// grid: (H, ceil(T/8)); one wave per output v (strided), lanes along c.
template <typename S>
__global__ __launch_bounds__(256) void out_proj_generic_kernel(int T, int H, int dc, int dv,
                                                               const S* __restrict__ o_lat,
                                                               const S* __restrict__ w_uv,
                                                               float* __restrict__ out) {
  __shared__ float os[kTokTile][512];
  const int h = blockIdx.x;
  const int t0 = blockIdx.y * kTokTile;
  const int nt = min(kTokTile, T - t0);
  for (int k = threadIdx.x; k < kTokTile * dc; k += blockDim.x) {
    int tt = k / dc, c = k - tt * dc;
    os[tt][c] = tt < nt ? Storage<S>::load(o_lat + ((int64_t)(t0 + tt) * H + h) * dc + c) : 0.f;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int v = wave; v < dv; v += 4) {
    const S* w = w_uv + ((int64_t)h * dv + v) * dc;
    float part[kTokTile] = {};
    for (int c = lane; c < dc; c += 64) {
      float wv = Storage<S>::load(w + c);
#pragma unroll
      for (int tt = 0; tt < kTokTile; ++tt) part[tt] += os[tt][c] * wv;
    }
#pragma unroll
    for (int tt = 0; tt < kTokTile; ++tt) {
      float s = part[tt];
#pragma unroll
      for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
      part[tt] = s;
    }
    if (lane == 0)
      for (int tt = 0; tt < nt; ++tt) out[((int64_t)(t0 + tt) * H + h) * dv + v] = part[tt];
  }
}

}  // namespace

hipError_t launch_absorb_generic(const mla_config& c, int T, const void* q_nope,
                                 const void* w_uk, void* q_lat, hipStream_t st) {
  dim3 grid((c.d_latent + 255) / 256, c.num_heads, (T + kTokTile - 1) / kTokTile), block(256);
  if (c.dtype == MLA_BF16)
    hipLaunchKernelGGL(absorb_generic_kernel<uint16_t>, grid, block, 0, st,
        T, c.num_heads, c.d_nope, c.d_latent, c.d_rope, (const uint16_t*)q_nope,
        (const uint16_t*)w_uk, (uint16_t*)q_lat);
  else
    hipLaunchKernelGGL(absorb_generic_kernel<float>, grid, block, 0, st,
        T, c.num_heads, c.d_nope, c.d_latent, c.d_rope, (const float*)q_nope,
        (const float*)w_uk, (float*)q_lat);
  return hipGetLastError();
}

hipError_t launch_out_proj_generic(const mla_config& c, int T, const void* o_lat,
                                   const void* w_uv, float* out, hipStream_t st) {
  dim3 grid(c.num_heads, (T + kTokTile - 1) / kTokTile), block(256);
  if (c.dtype == MLA_BF16)
    hipLaunchKernelGGL(out_proj_generic_kernel<uint16_t>, grid, block, 0, st,
        T, c.num_heads, c.d_latent, c.d_v, (const uint16_t*)o_lat, (const uint16_t*)w_uv, out);
  else
    hipLaunchKernelGGL(out_proj_generic_kernel<float>, grid, block, 0, st,
        T, c.num_heads, c.d_latent, c.d_v, (const float*)o_lat, (const float*)w_uv, out);
  return hipGetLastError();
}

}  // namespace mla
