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
#include "rope.h"

namespace mla {
namespace {

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

// DeepSeek-V3 shapes (d_c 512, d_r 64, 128 heads), bf16: three workgroups per
// new token.  Part 0 copies c_kv into the cache row (64 threads x 16 bytes) and
// rotates k_pe into it (4 threads); parts 1 and 2, launched only when queries
// are given, rotate the RoPE columns of q_lat for heads 64*(part-1) .. +63 (4
// threads per head, each 8 rotate-half pairs i, i+32 with 16-byte loads and
// stores).  Same fp32 op order and rounding as append_kernel, so the bytes
// written are identical.  Every pointer must be 16-byte aligned.
__global__ __launch_bounds__(256) void append_v3_kernel(
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const uint16_t* __restrict__ q_pe, const int32_t* __restrict__ seq,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ bt, int num_seqs, int max_blocks,
    int64_t num_blocks, const float* __restrict__ cosT, const float* __restrict__ sinT,
    int max_pos, uint16_t* __restrict__ pool, uint16_t* __restrict__ q_lat, uint32_t* err) {
  const int t = blockIdx.y, part = blockIdx.x, tid = threadIdx.x;
  const int s = seq[t];
  const int p = pos[t];
  uint32_t bad = 0;
  if (s < 0 || s >= num_seqs) bad |= MLA_DEVERR_SEQ;
  if (p < 0 || p >= max_pos) bad |= MLA_DEVERR_POSITION;
  int64_t blk = -1;
  if (!bad) {
    if (p / 64 >= max_blocks) {
      bad |= MLA_DEVERR_POSITION;
    } else {
      blk = bt[(int64_t)s * max_blocks + p / 64];
      if (blk < 0 || blk >= num_blocks) bad |= MLA_DEVERR_BLOCK;
    }
  }
  if (bad) {
    if (part == 0 && tid == 0 && err) atomicOr(err, bad);
    return;
  }
  const float* cr = cosT + (int64_t)p * kV3Half;
  const float* sr = sinT + (int64_t)p * kV3Half;
  if (part > 0) {
    const int h = 64 * (part - 1) + (tid >> 2), i0 = (tid & 3) * 8;
    rope8_bf16(q_pe + ((int64_t)t * kV3H + h) * kV3Dr, cr, sr, i0,
               q_lat + ((int64_t)t * kV3H + h) * kV3Row + kV3Dc);
    return;
  }
  uint16_t* row = pool + (blk * 64 + p % 64) * (int64_t)kV3Row;
  if (tid < 64) {
    *(u32x4*)(row + 8 * tid) = *(const u32x4*)(c_kv + (int64_t)t * kV3Dc + 8 * tid);
  } else if (tid < 68) {
    rope8_bf16(k_pe + (int64_t)t * kV3Dr, cr, sr, (tid - 64) * 8, row + kV3Dc);
  }
}

// e4m3 cache, DeepSeek-V3 shapes: part 0 writes the 576-byte row, c_kv (64
// threads x 8 values) and the rotated k_pe (4 threads x 8 pairs), each value
// multiplied by 1/kv_scale (a power of two, so exactly) and rounded once to e4m3;
// parts 1 and 2 write the bf16 RoPE columns of q_lat exactly as append_v3_kernel.
__global__ __launch_bounds__(256) void append_fp8_kernel(
    const uint16_t* __restrict__ c_kv, const uint16_t* __restrict__ k_pe,
    const uint16_t* __restrict__ q_pe, const int32_t* __restrict__ seq,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ bt, int num_seqs, int max_blocks,
    int64_t num_blocks, const float* __restrict__ cosT, const float* __restrict__ sinT,
    int max_pos, float inv_scale, uint8_t* __restrict__ pool, uint16_t* __restrict__ q_lat,
    uint32_t* err) {
  const int t = blockIdx.y, part = blockIdx.x, tid = threadIdx.x;
  const int s = seq[t];
  const int p = pos[t];
  uint32_t bad = 0;
  if (s < 0 || s >= num_seqs) bad |= MLA_DEVERR_SEQ;
  if (p < 0 || p >= max_pos) bad |= MLA_DEVERR_POSITION;
  int64_t blk = -1;
  if (!bad) {
    if (p / 64 >= max_blocks) {
      bad |= MLA_DEVERR_POSITION;
    } else {
      blk = bt[(int64_t)s * max_blocks + p / 64];
      if (blk < 0 || blk >= num_blocks) bad |= MLA_DEVERR_BLOCK;
    }
  }
  if (bad) {
    if (part == 0 && tid == 0 && err) atomicOr(err, bad);
    return;
  }
  const float* cr = cosT + (int64_t)p * kV3Half;
  const float* sr = sinT + (int64_t)p * kV3Half;
  if (part > 0) {
    const int h = 64 * (part - 1) + (tid >> 2), i0 = (tid & 3) * 8;
    rope8_bf16(q_pe + ((int64_t)t * kV3H + h) * kV3Dr, cr, sr, i0,
               q_lat + ((int64_t)t * kV3H + h) * kV3Row + kV3Dc);
    return;
  }
  uint8_t* row = pool + (blk * 64 + p % 64) * (int64_t)kV3Row;
  auto pack8 = [&](const float* v) {
    u32x2 o = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma clang fp contract(off)
      const float y = v[j] * inv_scale;
      o[j >> 2] |= (uint32_t)f32_to_e4m3(y) << (8 * (j & 3));
    }
    return o;
  };
  if (tid < 64) {
    const u32x4 c = *(const u32x4*)(c_kv + (int64_t)t * kV3Dc + 8 * tid);
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = bf16_bits_to_f32((uint16_t)(c[j >> 1] >> (16 * (j & 1))));
    *(u32x2*)(row + 8 * tid) = pack8(v);
  } else if (tid < 68) {
    const int i0 = (tid - 64) * 8;
    float y1[8], y2[8];
    rope8_pairs(k_pe + (int64_t)t * kV3Dr, cr, sr, i0, y1, y2);
    *(u32x2*)(row + kV3Dc + i0) = pack8(y1);
    *(u32x2*)(row + kV3Dc + kV3Half + i0) = pack8(y2);
  }
}

}  // namespace

hipError_t launch_append(const mla_config& c, int T, const void* c_kv, const void* k_pe,
                         const void* q_pe, const int32_t* seq, const int32_t* pos,
                         const int32_t* bt, int num_seqs, int max_blocks, int64_t num_blocks,
                         const float* cosT, const float* sinT, int max_pos, void* pool,
                         void* q_lat, uint32_t* err, hipStream_t st) {
  const auto a16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
  if (c.dtype == MLA_BF16 && c.d_latent == kV3Dc && c.d_rope == kV3Dr && c.num_heads == kV3H &&
      c.block_size == 64 && a16(c_kv) && a16(k_pe) && a16(q_pe) && a16(q_lat) && a16(pool) &&
      a16(cosT) && a16(sinT)) {
    // parts 1 and 2 (q_lat RoPE columns) only when queries are given
    hipLaunchKernelGGL(append_v3_kernel, dim3(q_pe ? 3 : 1, T), dim3(256), 0, st,
        (const uint16_t*)c_kv, (const uint16_t*)k_pe, (const uint16_t*)q_pe, seq, pos, bt,
        num_seqs, max_blocks, num_blocks, cosT, sinT, max_pos, (uint16_t*)pool,
        (uint16_t*)q_lat, err);
    return hipGetLastError();
  }
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

hipError_t launch_append_fp8(int T, const void* c_kv, const void* k_pe, const void* q_pe,
                             const int32_t* seq, const int32_t* pos, const int32_t* bt,
                             int num_seqs, int max_blocks, int64_t num_blocks, const float* cosT,
                             const float* sinT, int max_pos, float inv_scale, void* pool,
                             void* q_lat, uint32_t* err, hipStream_t st) {
  hipLaunchKernelGGL(append_fp8_kernel, dim3(q_pe ? 3 : 1, T), dim3(256), 0, st,
                     (const uint16_t*)c_kv, (const uint16_t*)k_pe, (const uint16_t*)q_pe, seq,
                     pos, bt, num_seqs, max_blocks, num_blocks, cosT, sinT, max_pos, inv_scale,
                     (uint8_t*)pool, (uint16_t*)q_lat, err);
  return hipGetLastError();
}

}  // namespace mla
