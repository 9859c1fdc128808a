// Weight-level absorbed projections, DeepSeek-V3 shapes (128 heads, d_c 512),
// bf16 in, fp32 accumulation, on gfx950 MFMA.
//
// [MLA explainer] forward_inference_absorbed: w_q_absorbed = W_UQ^T W_UK per
// head ([d_cq x d_c]) takes the compressed query c_q straight into the latent
// space, and w_o_absorbed = W_UV^T W_O per head ([d_c x d_model]) takes the
// attended latent straight to the model width, summed over the heads
// ("MLA的常见问题" Q3: the fused weights are larger than the factors).
//   absorb_q_fused : q_lat[t][h][c] = sum_j c_q[t][j] * W_KQ[h][j][c]
//   out_proj_fused : out[t][m]      = sum_{h,c} o_lat[t][h][c] * W_OV[h][c][m]
// Both are C[t][n] = sum_k A[t][k] * W[k][n] with W row-major (n contiguous)
// and few tokens, so the weight is the traffic.  On the output side k runs
// over (h, c) flattened, which is how o_lat [T][H][d_c] and W_OV
// [H][d_c][d_model] are laid out already.
//
// stream_tile: a workgroup computes 64 tokens x 256 columns over one k range;
// wave w owns columns 64w .. 64w+63 (4 blocks of 16) x the 64 tokens (4 blocks).
// The k range streams in chunks of 32 rows (16 KiB of weight, 4 KiB of
// tokens).  Every thread keeps the 16-byte loads of the next four chunks in
// flight in registers; a landed chunk goes to one of two LDS buffers (one
// barrier per chunk: a wave past the barrier of chunk i has every wave's reads
// of chunk i-1 behind it, so the buffer of chunk i+1 is free), and the waves
// run 16 v_mfma_f32_16x16x32_bf16 on it.  A operand = W^T (m = column, k)
// through the transposing LDS read ds_read_b64_tr_b16, as in the per-head
// absorption: in a 16-lane group, lane j points at 4 columns of row 4g + j/4
// and lane i receives column i of those 4 rows; two reads (rows +0, +16) fill
// the 8 k-slots of group g.  B operand = token rows (k, n = token).
//   absorb_fused_kernel: one workgroup per (256-column half, head, token tile),
//     k over all of d_cq; the bf16 result goes into q_lat.
//   out_fused_kernel: the H*d_c-deep contraction is cut into S ranges; fp32
//     partial sums go to the workspace [S][T][d_model] and reduce_kernel adds
//     them in increasing range order, so results do not depend on timing.
//
// MFMA operand layout (lane l = 16g + i): A[i][k], B[k][i] with the 8 k-slots
// of group g; D[4g + r][i], r = 0..3.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kH = 128;
constexpr int kDC = 512;
constexpr int kRow = 576;
constexpr int kTT = 64;                // tokens per workgroup
constexpr int kKC = 32;                // k rows per chunk
constexpr int kCB = 4;                 // 16-column blocks per wave
constexpr int kNT = 64 * kCB;          // columns per workgroup
constexpr int kWCh = kNT / 8;          // 16-byte pieces per weight chunk row
constexpr int kWL = kKC * kWCh / 256;  // weight loads per thread per chunk
constexpr int kDepth = 4;              // chunks in flight per thread
constexpr int kWRowB = kNT * 2 + 32;   // weight chunk row in LDS (bytes, padded)
constexpr int kARowB = kKC * 2 + 16;   // token row of a chunk in LDS (bytes, padded)
constexpr int kWBuf = kKC * kWRowB;
constexpr int kABuf = kTT * kARowB;
constexpr int kOutSplits = 16;         // k ranges of the output-side contraction

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

// acc[cb][tb]: columns 64w + 16cb + 4g + r of token 16tb + i16, over k rows
// [0, nk) of A (token rows t0 .., row stride lda) and W (row stride ldw), both
// already offset to the range's first k (and W to the tile's first column).
// nk is a multiple of kKC * kDepth.
__device__ __forceinline__ void stream_tile(int T, int t0, const uint16_t* __restrict__ A,
                                            int64_t lda, const uint16_t* __restrict__ W,
                                            int64_t ldw, int nk, char* lds, f32x4 (&acc)[kCB][4]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[cb][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per chunk and thread: 4 weight loads (row k >> 5, 16-byte column k & 31)
  // and 1 token load (token tid >> 2, 16-byte column tid & 3); token rows past
  // T repeat the last token (their results are not stored)
  // (uniform chunk base + per-lane offset, so the addresses stay cheap)
  const uint16_t* arow = A + (int64_t)min(t0 + (tid >> 2), T - 1) * lda + 8 * (tid & 3);
  const int wlane = (tid / kWCh) * (int)ldw + 8 * (tid % kWCh);
  u32x4 wr[kDepth][kWL], ar[kDepth];
  auto load = [&](int ch, int d) {
    const uint16_t* wsrc = W + (int64_t)ch * kKC * ldw;
#pragma unroll
    for (int i = 0; i < kWL; ++i)
      wr[d][i] = *(const u32x4*)(wsrc + (256 / kWCh) * i * ldw + wlane);
    ar[d] = *(const u32x4*)(arow + ch * kKC);
  };
  const int nchunks = nk / kKC;
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    load(d, d);
    __builtin_amdgcn_sched_barrier(0);  // issue order = chunk order (the waits rely on it)
  }

  // transposing-read address of this lane (row 4g + i16/4, column
  // 64w + 4(i16 & 3)) and token-row address (token i16, k 4g)
  const int wa = (4 * g + (i16 >> 2)) * kWRowB + (16 * kCB * wave + 4 * (i16 & 3)) * 2;
  const int qa = i16 * kARowB + 4 * g * 2;
  // chunk ch sits in registers slot ch % kDepth and LDS buffer ch % 2
  auto step = [&](int d, bool refill, int next) {
    // keep the scheduler from hoisting this chunk's LDS writes (and so the wait
    // for its loads) into the previous step
    __builtin_amdgcn_sched_barrier(0);
    char* wt = lds + (d & 1) * (kWBuf + kABuf);
    char* at = wt + kWBuf;
#pragma unroll
    for (int i = 0; i < kWL; ++i) {
      const int k = tid + 256 * i;
      *(u32x4*)(wt + (k / kWCh) * kWRowB + 16 * (k % kWCh)) = wr[d][i];
    }
    *(u32x4*)(at + (tid >> 2) * kARowB + 16 * (tid & 3)) = ar[d];
    __syncthreads();
    if (refill) load(next, d);
    bf16x8 a[kCB], b[4];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const char* p = wt + wa + 16 * cb * 2;
      const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)p);
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p + 16 * kWRowB));
      a[cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const char* p = at + qa + 16 * tb * kARowB;
      const u32x2 x0 = *(const u32x2*)p;
      const u32x2 x1 = *(const u32x2*)(p + 16 * 2);
      b[tb] = __builtin_bit_cast(bf16x8, u32x4{x0.x, x0.y, x1.x, x1.y});
    }
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
        acc[cb][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[cb], b[tb], acc[cb][tb], 0, 0, 0);
  };
  // The refills are unconditional inside the loop and the last group is
  // peeled, so the loop body is straight-line code and the compiler's waits
  // before each LDS write cover only the oldest chunk (not every load in flight).
  int c0 = 0;
  for (; c0 < nchunks - kDepth; c0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) step(d, true, c0 + d + kDepth);
  }
#pragma unroll
  for (int d = 0; d < kDepth; ++d) step(d, false, 0);
}

__global__ __launch_bounds__(256, 2) void absorb_fused_kernel(int T, int d_cq,
                                                           const uint16_t* __restrict__ c_q,
                                                           const uint16_t* __restrict__ w_kq,
                                                           uint16_t* __restrict__ q_lat) {
  __shared__ __attribute__((aligned(16))) char lds[2 * (kWBuf + kABuf)];
  const int n0 = blockIdx.x * kNT, h = blockIdx.y, t0 = blockIdx.z * kTT;
  f32x4 acc[kCB][4];
  stream_tile(T, t0, c_q, d_cq, w_kq + (int64_t)h * d_cq * kDC + n0, kDC, d_cq, lds, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int t = t0 + 16 * tb + i16;
    if (t >= T) continue;
    uint16_t* dst = q_lat + ((int64_t)t * kH + h) * kRow + n0 + 16 * kCB * wave + 4 * g;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      u32x2 v;
      v.x = pack_bf16x2(acc[cb][tb][0], acc[cb][tb][1]);
      v.y = pack_bf16x2(acc[cb][tb][2], acc[cb][tb][3]);
      *(u32x2*)(dst + 16 * cb) = v;
    }
  }
}

__global__ __launch_bounds__(256, 2) void out_fused_kernel(int T, int d_model,
                                                        const uint16_t* __restrict__ o_lat,
                                                        const uint16_t* __restrict__ w_ov,
                                                        float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) char lds[2 * (kWBuf + kABuf)];
  const int n0 = blockIdx.x * kNT, s = blockIdx.y, t0 = blockIdx.z * kTT;
  constexpr int kRange = kH * kDC / kOutSplits;
  const int64_t k0 = (int64_t)s * kRange;
  f32x4 acc[kCB][4];
  stream_tile(T, t0, o_lat + k0, kH * kDC, w_ov + k0 * d_model + n0, d_model, kRange, lds, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int t = t0 + 16 * tb + i16;
    if (t >= T) continue;
    float* dst = part + ((int64_t)s * T + t) * d_model + n0 + 16 * kCB * wave + 4 * g;
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) *(f32x4*)(dst + 16 * cb) = acc[cb][tb];
  }
}

// out[i] = sum_s part[s][i] for i < n (n a multiple of 4), s in increasing order
__global__ __launch_bounds__(256) void reduce_kernel(int64_t n, const float* __restrict__ part,
                                                     float* __restrict__ out) {
  const int64_t i = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
  if (i >= n) return;
  f32x4 v[kOutSplits];
#pragma unroll
  for (int s = 0; s < kOutSplits; ++s) v[s] = *(const f32x4*)(part + s * n + i);
  f32x4 sum = v[0];
#pragma unroll
  for (int s = 1; s < kOutSplits; ++s) sum += v[s];
  *(f32x4*)(out + i) = sum;
}

}  // namespace

size_t out_fused_workspace_bytes(int T, int d_model) {
  return (size_t)kOutSplits * (size_t)T * d_model * sizeof(float);
}

hipError_t launch_absorb_q_fused(int T, int d_cq, const void* c_q, const void* w_kq, void* q_lat,
                                 hipStream_t st) {
  hipLaunchKernelGGL(absorb_fused_kernel, dim3(kDC / kNT, kH, (T + kTT - 1) / kTT), dim3(256), 0,
                     st, T, d_cq, (const uint16_t*)c_q, (const uint16_t*)w_kq, (uint16_t*)q_lat);
  return hipGetLastError();
}

hipError_t launch_out_proj_fused(int T, int d_model, const void* o_lat, const void* w_ov,
                                 float* out, void* workspace, hipStream_t st) {
  hipLaunchKernelGGL(out_fused_kernel, dim3(d_model / kNT, kOutSplits, (T + kTT - 1) / kTT),
                     dim3(256), 0, st, T, d_model, (const uint16_t*)o_lat, (const uint16_t*)w_ov,
                     (float*)workspace);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)T * d_model;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st, n,
                     (const float*)workspace, out);
  return hipGetLastError();
}

}  // namespace mla
