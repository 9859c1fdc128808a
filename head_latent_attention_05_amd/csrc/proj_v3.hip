// Per-head projections on both sides of the latent attention, DeepSeek-V3
// shapes (128 heads, d_nope = d_v = 128, d_c = 512), bf16 in, fp32 accumulate,
// on gfx950 MFMA.
//
// absorb_q : q_lat[t][h][c] = sum_d q_nope[t][h][d] * W_UK[h][d][c]
//            ([MLA explainer] stage 2B / forward_inference_absorbed: the query
//            enters the latent space through W_UK; [MLA deep dive] 2.3)
// out_proj : out[t][h][v]   = sum_c o_lat[t][h][c] * W_UV[h][v][c]
//            ([MLA explainer] forward_inference_absorbed: the attended latent
//            leaves through W_UV, per head)
//
// Both are batched GEMMs whose token dimension is small at decode: per head a
// tile of up to 64 tokens meets the head's 128 KiB weight, so the weights are
// the traffic (16 MiB each for 128 heads).  A workgroup owns one head, one half
// of the weight's output columns and one 64-token tile: it stages its weight
// slice and token tile in LDS with 16-byte loads (every load in flight at once),
// then 4 waves run v_mfma_f32_16x16x32_bf16 from LDS.  LDS rows are padded so
// that the operand reads of 16 lanes (one LDS cycle) hit distinct banks.
//
// MFMA operand layout (lane l = 16g + i): A[i][k], B[k][i] with the 8 k-slots
// of group g; D[4g + r][i], r = 0..3.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kH = 128;
constexpr int kDN = 128;
constexpr int kDC = 512;
constexpr int kDV = 128;
constexpr int kRow = 576;  // q_lat row: latent part + RoPE part
constexpr int kTT = 64;    // tokens per workgroup

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

// ---------------------------------------------------------------- absorb_q
// Workgroup: latent half c0 = 256 * blockIdx.x, head blockIdx.y, tokens
// 64 * blockIdx.z ...  Per wave: latent columns c0 + 64w .. +63 (4 blocks of 16)
// x 64 tokens (4 blocks of 16), contraction over d in 4 steps of 32.
// D = q_lat^T tile: A = W_UK^T (m = latent column, k = d), B = q_nope^T
// (k = d, n = token).  W_UK is stored [d][c], so the A operand (8 d-values of
// one column per lane) comes from the transposing LDS read ds_read_b64_tr_b16:
// in a 16-lane group, lane j points at 4 columns of row 4g + j/4 and lane i
// receives column i of those 4 rows.  Two such reads (rows +0 and +16) fill the
// 8 k-slots of group g with d = 4g..4g+3 and 16+4g..16+4g+3 of the step; the
// B operand takes the same d-values from the token rows.
constexpr int kAbsCols = 256;                  // latent columns per workgroup
constexpr int kAbsWRow = kAbsCols * 2 + 32;    // W_UK tile row (bytes, padded)
constexpr int kAbsQRow = kDN * 2 + 16;         // q_nope tile row (bytes, padded)

__global__ __launch_bounds__(256) void absorb_v3_kernel(int T, const uint16_t* __restrict__ q_nope,
                                                        const uint16_t* __restrict__ w_uk,
                                                        uint16_t* __restrict__ q_lat) {
  __shared__ __attribute__((aligned(16))) char wt[kDN * kAbsWRow];  // W_UK[h][d][c0 + c]
  __shared__ __attribute__((aligned(16))) char qt[kTT * kAbsQRow];  // q_nope[t0 + t][h][d]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.x * kAbsCols, h = blockIdx.y, t0 = blockIdx.z * kTT;

  // stage: W tile 128 rows x 32 chunks of 16 B, token tile 64 rows x 16 chunks
  const uint16_t* wsrc = w_uk + (int64_t)h * kDN * kDC + c0;
  u32x4 wv[16], qv[4];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int k = tid + 256 * i, r = k >> 5, c = k & 31;
    wv[i] = *(const u32x4*)(wsrc + r * kDC + c * 8);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // rows past the last token repeat the last token: a token's outputs depend
    // on its own row only, and those columns are not stored (no branch or select
    // on the loads, so all of them are in flight at once)
    const int k = tid + 256 * i, r = k >> 4, c = k & 15;
    qv[i] = *(const u32x4*)(q_nope + ((int64_t)min(t0 + r, T - 1) * kH + h) * kDN + c * 8);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int k = tid + 256 * i, r = k >> 5, c = k & 31;
    *(u32x4*)(wt + r * kAbsWRow + c * 16) = wv[i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = tid + 256 * i, r = k >> 4, c = k & 15;
    *(u32x4*)(qt + r * kAbsQRow + c * 16) = qv[i];
  }
  __syncthreads();

  f32x4 acc[4][4];  // [latent block][token block]
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[cb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this lane's transposing-read address: row 4g + i16/4, column 4*(i16 & 3) of
  // the wave's latent block
  const char* wa = wt + (4 * g + (i16 >> 2)) * kAbsWRow + (64 * wave + 4 * (i16 & 3)) * 2;
  const char* qa = qt + i16 * kAbsQRow + 4 * g * 2;
#pragma unroll
  for (int kk = 0; kk < kDN / 32; ++kk) {
    bf16x8 a[4], b[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const char* p = wa + 32 * kk * kAbsWRow + 16 * cb * 2;
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)p);
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p + 16 * kAbsWRow));
      a[cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const char* p = qa + 16 * tb * kAbsQRow + 32 * kk * 2;
      const u32x2 x0 = *(const u32x2*)p;
      const u32x2 x1 = *(const u32x2*)(p + 16 * 2);
      b[tb] = __builtin_bit_cast(bf16x8, u32x4{x0.x, x0.y, x1.x, x1.y});
    }
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        acc[cb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[cb], b[tb], acc[cb][tb], 0, 0, 0);
  }

  // lane holds latent columns c0 + 64w + 16cb + 4g + r (r = 0..3) of token 16tb + i16
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int t = t0 + 16 * tb + i16;
    if (t >= T) continue;
    uint16_t* dst = q_lat + ((int64_t)t * kH + h) * kRow + c0 + 64 * wave + 4 * g;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      u32x2 v;
      v.x = pack_bf16x2(acc[cb][tb][0], acc[cb][tb][1]);
      v.y = pack_bf16x2(acc[cb][tb][2], acc[cb][tb][3]);
      *(u32x2*)(dst + 16 * cb) = v;
    }
  }
}

// ---------------------------------------------------------------- out_proj
// Workgroup: outputs v0 = 64 * blockIdx.x .. +63, head blockIdx.y, tokens
// 64 * blockIdx.z ...  Per wave: 16 outputs (v0 + 16w ..) x 64 tokens,
// contraction over c in 16 steps of 32.  D = out^T tile: A = W_UV (m = v,
// k = c; rows are contiguous in c), B = o_lat^T (k = c, n = token; token rows
// are contiguous in c): both operands are plain 16-byte row reads.
constexpr int kOpRowB = kDC * 2 + 16;  // tile row (bytes, padded)

__global__ __launch_bounds__(256) void out_proj_v3_kernel(int T, const uint16_t* __restrict__ o_lat,
                                                          const uint16_t* __restrict__ w_uv,
                                                          float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) char wt[64 * kOpRowB];   // W_UV[h][v0 + v][c]
  __shared__ __attribute__((aligned(16))) char ot[kTT * kOpRowB];  // o_lat[t0 + t][h][c]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int v0 = blockIdx.x * 64, h = blockIdx.y, t0 = blockIdx.z * kTT;

  // stage: both tiles are 64 rows x 64 chunks of 16 B
  const uint16_t* wsrc = w_uv + ((int64_t)h * kDV + v0) * kDC;
  u32x4 wv[16], ov[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int k = tid + 256 * i, r = k >> 6, c = k & 63;
    wv[i] = *(const u32x4*)(wsrc + r * kDC + c * 8);
    // rows past the last token repeat the last token (their outputs are not stored)
    ov[i] = *(const u32x4*)(o_lat + ((int64_t)min(t0 + r, T - 1) * kH + h) * kDC + c * 8);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int k = tid + 256 * i, r = k >> 6, c = k & 63;
    *(u32x4*)(wt + r * kOpRowB + c * 16) = wv[i];
    *(u32x4*)(ot + r * kOpRowB + c * 16) = ov[i];
  }
  __syncthreads();

  f32x4 acc[4];  // [token block]
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const char* wa = wt + (16 * wave + i16) * kOpRowB + 8 * g * 2;
  const char* oa = ot + i16 * kOpRowB + 8 * g * 2;
#pragma unroll 4
  for (int kk = 0; kk < kDC / 32; ++kk) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(wa + 32 * kk * 2));
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const bf16x8 b =
          __builtin_bit_cast(bf16x8, *(const u32x4*)(oa + 16 * tb * kOpRowB + 32 * kk * 2));
      acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[tb], 0, 0, 0);
    }
  }

  // lane holds outputs v0 + 16w + 4g + r (r = 0..3) of token 16tb + i16
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int t = t0 + 16 * tb + i16;
    if (t >= T) continue;
    *(f32x4*)(out + ((int64_t)t * kH + h) * kDV + v0 + 16 * wave + 4 * g) = acc[tb];
  }
}

}  // namespace

hipError_t launch_absorb_q(const mla_config&, int T, const void* q_nope, const void* w_uk,
                           void* q_lat, hipStream_t st) {
  hipLaunchKernelGGL(absorb_v3_kernel, dim3(kDC / kAbsCols, kH, (T + kTT - 1) / kTT), dim3(256),
                     0, st, T, (const uint16_t*)q_nope, (const uint16_t*)w_uk,
                     (uint16_t*)q_lat);
  return hipGetLastError();
}

hipError_t launch_out_proj(const mla_config&, int T, const void* o_lat, const void* w_uv,
                           float* out, hipStream_t st) {
  hipLaunchKernelGGL(out_proj_v3_kernel, dim3(kDV / 64, kH, (T + kTT - 1) / kTT), dim3(256), 0,
                     st, T, (const uint16_t*)o_lat, (const uint16_t*)w_uv, out);
  return hipGetLastError();
}

}  // namespace mla
