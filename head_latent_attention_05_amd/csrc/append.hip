// Fused RoPE + latent-cache append.
//
// [MLA architecture] 4.2 fuses the RoPE of the shared key with the cache update
// into one kernel; 3.2 keeps two parts per token (512-d latent, 64-d RoPE key),
// stored here as one 576-wide row.  [MLA explainer] "MLA的实现", RoPE module:
// rotate-half pairing (i, i + d_r/2), y = x*cos + rotate_half(x)*sin.
//
// One workgroup per new token: copies c_kv into the row, rotates k_pe into the
// row, and rotates the token's per-head q_pe into the RoPE columns of q_lat.
// Products and sums are rounded to fp32 one by one (no fused multiply-add), so
// the row is bit-exact and independent of the device.
#include "mla_internal.h"

namespace mla {
namespace {

// y1 = x1*c - x2*s ; y2 = x2*c + x1*s, each op rounded to fp32.
__device__ __forceinline__ void rope_pair(float x1, float x2, float c, float s, float& y1,
                                          float& y2) {
#pragma clang fp contract(off)
  float a = x1 * c;
  float b = x2 * s;
  float d = x2 * c;
  float e = x1 * s;
  y1 = a - b;
  y2 = d + e;
}

template <typename S>
__global__ __launch_bounds__(256) void append_kernel(
    int H, int dc, int dr, int bs, const S* __restrict__ c_kv, const S* __restrict__ k_pe,
    const S* __restrict__ q_pe, const int32_t* __restrict__ seq, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ bt, int num_seqs, int max_blocks, int64_t num_blocks,
    const float* __restrict__ cosT, const float* __restrict__ sinT, int max_pos,
    S* __restrict__ pool, S* __restrict__ q_lat, uint32_t* err) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int s = seq[t];
  const int p = pos[t];
  const int half = dr >> 1;
  const int row = dc + dr;
  uint32_t bad = 0;
  if (s < 0 || s >= num_seqs) bad |= MLA_DEVERR_SEQ;
  if (p < 0 || p >= max_pos) bad |= MLA_DEVERR_POSITION;
  int64_t blk = -1;
  if (!bad) {
    if (p / bs >= max_blocks) {
      bad |= MLA_DEVERR_POSITION;
    } else {
      blk = bt[(int64_t)s * max_blocks + p / bs];
      if (blk < 0 || blk >= num_blocks) bad |= MLA_DEVERR_BLOCK;
    }
  }
  if (bad) {
    if (tid == 0 && err) atomicOr(err, bad);
    return;
  }
  const float* cr = cosT + (int64_t)p * half;
  const float* sr = sinT + (int64_t)p * half;
  S* dst = pool + (blk * bs + p % bs) * (int64_t)row;
  const S* src = c_kv + (int64_t)t * dc;
  for (int i = tid; i < dc; i += blockDim.x) dst[i] = src[i];
  const S* kp = k_pe + (int64_t)t * dr;
  for (int i = tid; i < half; i += blockDim.x) {
    float y1, y2;
    rope_pair(Storage<S>::load(kp + i), Storage<S>::load(kp + i + half), cr[i], sr[i], y1, y2);
    Storage<S>::store(dst + dc + i, y1);
    Storage<S>::store(dst + dc + i + half, y2);
  }
  if (q_pe) {
    const S* qp = q_pe + (int64_t)t * H * dr;
    S* ql = q_lat + (int64_t)t * H * row;
    for (int k = tid; k < H * half; k += blockDim.x) {
      int h = k / half, i = k - h * half;
      float y1, y2;
      rope_pair(Storage<S>::load(qp + h * dr + i), Storage<S>::load(qp + h * dr + i + half),
                cr[i], sr[i], y1, y2);
      Storage<S>::store(ql + (int64_t)h * row + dc + i, y1);
      Storage<S>::store(ql + (int64_t)h * row + dc + i + half, y2);
    }
  }
}

}  // namespace

hipError_t launch_append(const mla_config& c, int T, const void* c_kv, const void* k_pe,
                         const void* q_pe, const int32_t* seq, const int32_t* pos,
                         const int32_t* bt, int num_seqs, int max_blocks, int64_t num_blocks,
                         const float* cosT, const float* sinT, int max_pos, void* pool,
                         void* q_lat, uint32_t* err, hipStream_t st) {
  dim3 grid(T), block(256);
  if (c.dtype == MLA_BF16) {
    hipLaunchKernelGGL(append_kernel<uint16_t>, grid, block, 0, st,
        c.num_heads, c.d_latent, c.d_rope, c.block_size, (const uint16_t*)c_kv,
        (const uint16_t*)k_pe, (const uint16_t*)q_pe, seq, pos, bt, num_seqs, max_blocks,
        num_blocks, cosT, sinT, max_pos, (uint16_t*)pool, (uint16_t*)q_lat, err);
  } else {
    hipLaunchKernelGGL(append_kernel<float>, grid, block, 0, st,
        c.num_heads, c.d_latent, c.d_rope, c.block_size, (const float*)c_kv, (const float*)k_pe,
        (const float*)q_pe, seq, pos, bt, num_seqs, max_blocks, num_blocks, cosT, sinT, max_pos,
        (float*)pool, (float*)q_lat, err);
  }
  return hipGetLastError();
}

}  // namespace mla
