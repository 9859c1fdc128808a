// Joint KV down-projection fused with the latent RMSNorm and the cache append,
// DeepSeek-V3 shapes (d_c 512, d_r 64), bf16 storage, fp32 arithmetic.
//
// [MLA architecture] 2.2: kv_a_proj_with_mqa maps a token's hidden state
// (d_model values) to the 512-d latent and the 64-d shared RoPE key in one
// product, and kv_a_layernorm RMS-normalises the latent; 4.2: the RoPE of the
// key is fused with the cache update.  Per new token t at position p:
//   y    = W_DKV x_t (+ b)               fp32 accumulation, rounded to bf16
//   c    = bf16(gamma * y[0:512] / sqrt(mean(y[0:512]^2) + eps))
//   row  = [c | RoPE_p(y[512:576])]      (the RoPE of mla_append_cache)
//
// kv_down_gemm_kernel: split-K product on v_mfma_f32_16x16x32_bf16.  A
// workgroup owns 64 tokens x 32 outputs x one 512-deep slice of d_model: it
// stages the weight tile (32 KiB) and the token tile (64 KiB) in LDS with
// 16-byte loads, all in flight at once, then wave w computes outputs
// 16(w & 1) .. +15 for tokens 32(w >> 1) .. +31.  Weight rows and hidden-state
// rows are both contiguous in k, so both MFMA operands are plain 16-byte row
// reads.  fp32 partial sums go to the workspace, [S][T][576] for
// S = d_model / 512 slices.
//
// kv_down_rows_kernel: one workgroup per token (plus two per token for the
// RoPE columns of q_lat, as the append does).  Sums the S partials of each
// output in increasing slice order (results do not depend on timing; eight
// slices' loads in flight at a time), adds the
// bias, rounds to bf16, normalises the latent (wave 0: 64 lanes x 8 values, the
// sum of squares by a butterfly over the wave), rotates the key (wave 1) and
// stores the row.
//
// MFMA operand layout (lane l = 16g + i): A[i][k], B[k][i] with the 8 k-slots
// of group g; D[4g + r][i], r = 0..3.
#include "rope.h"

namespace mla {
namespace {

constexpr int kN = kV3Dc + kV3Dr;  // 576 projected values per token
constexpr int kKC = 512;           // depth of one slice of d_model
constexpr int kTT = 64;            // tokens per workgroup
constexpr int kNT = 32;            // outputs per workgroup

constexpr int kRowB = kKC * 2 + 16;  // LDS tile row (bytes, padded)

__global__ __launch_bounds__(256) void kv_down_gemm_kernel(int T, int K,
                                                           const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ w,
                                                           float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) char wt[kNT * kRowB];  // W_DKV[n0 + n][k0 + k]
  __shared__ __attribute__((aligned(16))) char xt[kTT * kRowB];  // x[t0 + t][k0 + k]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * kNT;
  const int s = blockIdx.y;
  const int k0 = s * kKC;
  const int t0 = blockIdx.z * kTT;

  // stage both tiles (rows of 64 chunks of 16 B): 8 weight and 16 token loads
  // per thread, all in flight; token rows past T repeat the last token (their
  // sums are not stored)
  u32x4 wv[kNT * 64 / 256], xv[kTT * 64 / 256];
#pragma unroll
  for (int i = 0; i < kNT * 64 / 256; ++i) {
    const int k = tid + 256 * i, r = k >> 6, c = k & 63;
    wv[i] = *(const u32x4*)(w + (int64_t)(n0 + r) * K + k0 + 8 * c);
  }
#pragma unroll
  for (int i = 0; i < kTT * 64 / 256; ++i) {
    const int k = tid + 256 * i, r = k >> 6, c = k & 63;
    xv[i] = *(const u32x4*)(x + (int64_t)min(t0 + r, T - 1) * K + k0 + 8 * c);
  }
#pragma unroll
  for (int i = 0; i < kNT * 64 / 256; ++i) {
    const int k = tid + 256 * i, r = k >> 6, c = k & 63;
    *(u32x4*)(wt + r * kRowB + 16 * c) = wv[i];
  }
#pragma unroll
  for (int i = 0; i < kTT * 64 / 256; ++i) {
    const int k = tid + 256 * i, r = k >> 6, c = k & 63;
    *(u32x4*)(xt + r * kRowB + 16 * c) = xv[i];
  }
  __syncthreads();

  // wave w: outputs n0 + 16(w & 1) + i (A = weight rows), tokens
  // t0 + 32(w >> 1) + 16tb + i (B = token rows), both 16-byte row reads
  const char* wa = wt + (16 * (wave & 1) + i16) * kRowB + 16 * g;
  const char* xa = xt + (32 * (wave >> 1) + i16) * kRowB + 16 * g;
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
  for (int kk = 0; kk < kKC / 32; ++kk) {
    const bf16x8 av = __builtin_bit_cast(bf16x8, *(const u32x4*)(wa + 64 * kk));
    const bf16x8 b0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xa + 64 * kk));
    const bf16x8 b1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(xa + 16 * kRowB + 64 * kk));
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b0, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b1, acc1, 0, 0, 0);
  }
  // lane holds outputs n0 + 16(w & 1) + 4g + r (r = 0..3) of tokens
  // t0 + 32(w >> 1) + i16 and the same + 16
  const int nn = n0 + 16 * (wave & 1) + 4 * g;
  const int ta = t0 + 32 * (wave >> 1) + i16, tb = ta + 16;
  if (ta < T) *(f32x4*)(part + ((int64_t)s * T + ta) * kN + nn) = acc0;
  if (tb < T) *(f32x4*)(part + ((int64_t)s * T + tb) * kN + nn) = acc1;
}

__global__ __launch_bounds__(256) void kv_down_rows_kernel(
    int T, int S, const float* __restrict__ part, const uint16_t* __restrict__ bias,
    const uint16_t* __restrict__ gamma, float eps, const uint16_t* __restrict__ q_pe,
    const int32_t* __restrict__ seq, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ bt, int num_seqs, int max_blocks, int64_t num_blocks,
    const float* __restrict__ cosT, const float* __restrict__ sinT, int max_pos,
    uint16_t* __restrict__ pool, uint16_t* __restrict__ q_lat, uint32_t* err) {
  __shared__ __attribute__((aligned(16))) uint16_t key[kV3Dr];
  const int t = blockIdx.y, blk_part = blockIdx.x, tid = threadIdx.x;

  // part 0: outputs n .. n+7, the latent for wave 0, the key for lanes 0..7 of
  // wave 1.  The partial sums do not depend on the entry's checks, so their
  // loads go out first.
  const int n = tid < 64 ? 8 * tid : kV3Dc + 8 * (tid - 64);
  const bool summer = blk_part == 0 && tid < 72;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = 0.f;
  if (summer) {
    // eight slices' loads in flight at a time (indices past the last slice
    // repeat it and are not added), summed in increasing slice order
    const float* src = part + (int64_t)t * kN + n;
    const int64_t stride = (int64_t)T * kN;
    for (int s0 = 0; s0 < S; s0 += 8) {
      f32x4 u[8], v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = min(s0 + j, S - 1);
        u[j] = *(const f32x4*)(src + s * stride);
        v[j] = *(const f32x4*)(src + s * stride + 4);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (s0 + j < S) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            y[i] += u[j][i];
            y[4 + i] += v[j][i];
          }
        }
      }
    }
  }

  const int s_id = seq[t];
  const int p = pos[t];
  uint32_t bad = 0;
  if (s_id < 0 || s_id >= num_seqs) bad |= MLA_DEVERR_SEQ;
  if (p < 0 || p >= max_pos) bad |= MLA_DEVERR_POSITION;
  int64_t blk = -1;
  if (!bad) {
    if (p / 64 >= max_blocks) {
      bad |= MLA_DEVERR_POSITION;
    } else {
      blk = bt[(int64_t)s_id * max_blocks + p / 64];
      if (blk < 0 || blk >= num_blocks) bad |= MLA_DEVERR_BLOCK;
    }
  }
  if (bad) {  // uniform over the workgroup
    if (blk_part == 0 && tid == 0 && err) atomicOr(err, bad);
    return;
  }
  const float* cr = cosT + (int64_t)p * kV3Half;
  const float* sr = sinT + (int64_t)p * kV3Half;
  if (blk_part > 0) {
    // parts 1, 2: RoPE columns of q_lat for heads 64(part-1) .. +63, as the append
    const int h = 64 * (blk_part - 1) + (tid >> 2), i0 = (tid & 3) * 8;
    rope8_bf16(q_pe + ((int64_t)t * kV3H + h) * kV3Dr, cr, sr, i0,
               q_lat + ((int64_t)t * kV3H + h) * kV3Row + kV3Dc);
    return;
  }
  uint16_t* row = pool + (blk * 64 + p % 64) * (int64_t)kV3Row;
  if (summer) {
    if (bias) {
      const u32x4 bv = *(const u32x4*)(bias + n);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] += bf16_bits_to_f32((uint16_t)(bv[i >> 1] >> (16 * (i & 1))));
    }
    // the projection's output is a bf16 tensor
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = bf16_bits_to_f32(f32_to_bf16_bits(y[i]));
  }
  if (tid < 64) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += y[i] * y[i];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) ss += __shfl_xor(ss, d, 64);
    const float r = 1.0f / sqrtf(ss * (1.0f / kV3Dc) + eps);
    const u32x4 gv = *(const u32x4*)(gamma + n);
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float g0 = bf16_bits_to_f32((uint16_t)gv[k]);
      const float g1 = bf16_bits_to_f32((uint16_t)(gv[k] >> 16));
      o[k] = (uint32_t)f32_to_bf16_bits(g0 * (y[2 * k] * r)) |
             ((uint32_t)f32_to_bf16_bits(g1 * (y[2 * k + 1] * r)) << 16);
    }
    *(u32x4*)(row + n) = u32x4{o[0], o[1], o[2], o[3]};
  } else if (tid < 72) {
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = (uint32_t)f32_to_bf16_bits(y[2 * k]) |
             ((uint32_t)f32_to_bf16_bits(y[2 * k + 1]) << 16);
    *(u32x4*)(key + (n - kV3Dc)) = u32x4{o[0], o[1], o[2], o[3]};
  }
  __syncthreads();
  if (tid >= 64 && tid < 68) rope8_bf16(key, cr, sr, (tid - 64) * 8, row + kV3Dc);
}

}  // namespace

size_t kv_down_workspace_bytes(int T, int d_model) {
  return (size_t)(d_model / kKC) * (size_t)T * kN * sizeof(float);
}

hipError_t launch_kv_down_append(int T, int d_model, const void* x, const void* w_dkv,
                                 const void* b_dkv, const void* gamma, float eps,
                                 const void* q_pe, const int32_t* seq, const int32_t* pos,
                                 const int32_t* bt, int num_seqs, int max_blocks,
                                 int64_t num_blocks, const float* cosT, const float* sinT,
                                 int max_pos, void* workspace, void* pool, void* q_lat,
                                 uint32_t* err, hipStream_t st) {
  const int S = d_model / kKC;
  hipLaunchKernelGGL(kv_down_gemm_kernel, dim3(kN / kNT, S, (T + kTT - 1) / kTT), dim3(256), 0,
                     st, T, d_model, (const uint16_t*)x, (const uint16_t*)w_dkv,
                     (float*)workspace);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // parts 1 and 2 (q_lat RoPE columns) only when queries are given
  hipLaunchKernelGGL(kv_down_rows_kernel, dim3(q_pe ? 3 : 1, T), dim3(256), 0, st, T, S,
                     (const float*)workspace, (const uint16_t*)b_dkv, (const uint16_t*)gamma, eps,
                     (const uint16_t*)q_pe, seq, pos, bt, num_seqs, max_blocks, num_blocks, cosT,
                     sinT, max_pos, (uint16_t*)pool, (uint16_t*)q_lat, err);
  return hipGetLastError();
}

}  // namespace mla
