// Internal declarations shared by the libmla translation units (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16 helpers
// fp32 -> bf16, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// two fp32 -> packed bf16 pair (low half = a), nearest even (hardware convert).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// fp32 -> e4m3 (OCP fp8: bias 7, 3 mantissa bits, largest finite 448, 0x7F NaN):
// round to nearest, ties to even; finite magnitudes >= 448 saturate to 448; NaN
// -> 0x7F.  Integer arithmetic only, so the code is the same on every device.
__device__ __host__ __forceinline__ uint8_t f32_to_e4m3(float x) {
  uint32_t u;
  __builtin_memcpy(&u, &x, 4);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7f;                  // NaN
  if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7eu);  // >= 448 (and inf)
  if (a < 0x3c800000u) {                             // below 2^-6: quantum 2^-9
    // a * 2^9 < 8 is exact in fp32; round it to an integer, ties to even
    float v;
    __builtin_memcpy(&v, &a, 4);
    v *= 512.0f;
    const uint32_t m = (uint32_t)__builtin_rintf(v);  // 0..8 (8 = smallest normal)
    return (uint8_t)(sign | m);
  }
  // normal: keep 3 of the 23 mantissa bits, ties to even; a carry moves into
  // the exponent; rebias 127 -> 7
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  uint32_t code = r - (120u << 3);
  if (code > 0x7eu) code = 0x7eu;
  return (uint8_t)(sign | code);
}

template <typename T> struct Storage;
template <> struct Storage<float> {
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Storage<uint16_t> {
  __device__ static __forceinline__ float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  __device__ static __forceinline__ void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

// ---------------------------------------------------------------- split plan
// Work is counted in "units": one unit = one cache block of one query token.
// The units of all query tokens, in token order, are split into G contiguous
// ranges, one per KV workgroup: range w = [w*U/G, (w+1)*U/G).  A token whose
// units all fall in one range is finished by that workgroup; otherwise every
// range touching it writes a partial (normalised output + log2-sum-exp) to slot
// 2w (if the token is the first one of range w) or 2w+1 (otherwise), and the
// merge kernel combines the partials in increasing w.
struct PlanArgs {
  const int32_t* q_start;  // device [B+1]
  const int32_t* kv_lens;  // device [B]
  int32_t B;
  int32_t T;
  int32_t block_size;
  int32_t causal;
  int32_t G;
  int64_t U;
};

// sum_{k=1..n} ceil(k / bs)
__device__ __host__ __forceinline__ int64_t ceil_prefix(int64_t n, int64_t bs) {
  if (n <= 0) return 0;
  int64_t q = n / bs, r = n % bs;
  return bs * q * (q + 1) / 2 + r * (q + 1);
}
// units of sequence b's query tokens j < jn
__device__ __host__ __forceinline__ int64_t seq_units_before(int64_t L, int64_t q, int64_t jn,
                                                             int64_t bs, int causal) {
  if (causal) return ceil_prefix(L - q + jn, bs) - ceil_prefix(L - q, bs);
  return jn * ((L + bs - 1) / bs);
}
// attended length of query token j of a sequence with kv length L and q new tokens
__device__ __host__ __forceinline__ int64_t attend_len(int64_t L, int64_t q, int64_t j, int causal) {
  return causal ? (L - q + j + 1) : L;
}
__device__ __host__ __forceinline__ int64_t range_start(int64_t w, int64_t U, int64_t G) {
  return (w * U) / G;
}
// workgroup whose range holds unit u
__device__ __host__ __forceinline__ int64_t range_of(int64_t u, int64_t U, int64_t G) {
  return ((u + 1) * G - 1) / U;
}

// Partial-result workspace layout for a plan with G workgroups:
//   lse  float [2G][H]          (log2-sum-exp of the scaled scores)
//   o    storage [2G][H][d_c]   (normalised partial output)
__host__ __device__ inline size_t ws_lse_bytes(int64_t G, int H) {
  return (size_t)(2 * G) * H * sizeof(float);
}
__host__ __device__ inline size_t ws_align(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------- launchers
// (defined in the kernel translation units; return hipGetLastError())
hipError_t launch_append(const mla_config& c, int T, const void* c_kv, const void* k_pe,
                         const void* q_pe, const int32_t* seq, const int32_t* pos,
                         const int32_t* bt, int num_seqs, int max_blocks, int64_t num_blocks,
                         const float* cos, const float* sin, int max_pos, void* pool,
                         void* q_lat, uint32_t* err, hipStream_t st);
size_t prefill_workspace_bytes(int B, int64_t R);
hipError_t launch_prefill(int B, int T, int64_t R, int max_qt, const int32_t* q_start,
                          const int32_t* kv_lens, const int32_t* bt, int max_blocks,
                          int64_t num_blocks, const void* q_nope, const void* q_lat,
                          const void* pool, const void* w_uk, const void* w_uv, int causal,
                          float scale, void* workspace, float* out, uint32_t* err,
                          hipStream_t st);
size_t out_fused_workspace_bytes(int T, int d_model);
hipError_t launch_absorb_q_fused(int T, int d_cq, const void* c_q, const void* w_kq, void* q_lat,
                                 hipStream_t st);
hipError_t launch_out_proj_fused(int T, int d_model, const void* o_lat, const void* w_ov,
                                 float* out, void* workspace, hipStream_t st);
size_t kv_down_workspace_bytes(int T, int d_model);
hipError_t launch_kv_down_append(int T, int d_model, const void* x, const void* w_dkv,
                                 const void* b_dkv, const void* gamma, float eps,
                                 const void* q_pe, const int32_t* seq, const int32_t* pos,
                                 const int32_t* bt, int num_seqs, int max_blocks,
                                 int64_t num_blocks, const float* cos, const float* sin,
                                 int max_pos, void* workspace, void* pool, void* q_lat,
                                 uint32_t* err, hipStream_t st);
hipError_t launch_absorb_q(const mla_config& c, int T, const void* q_nope, const void* w_uk,
                           void* q_lat, hipStream_t st);
hipError_t launch_out_proj(const mla_config& c, int T, const void* o_lat, const void* w_uv,
                           float* out, hipStream_t st);
struct DecodeArgs {
  PlanArgs plan;
  const int32_t* block_table;
  int32_t max_blocks;
  int64_t num_blocks;
  const void* q_lat;
  const void* pool;
  void* o_lat;
  float* ws_lse;
  void* ws_o;
  uint32_t* err;
  float scale_log2;  // softmax_scale * log2(e)
};
hipError_t launch_decode_generic(const mla_config& c, const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_v3(const DecodeArgs& a, hipStream_t st);
hipError_t launch_decode_fp8(const DecodeArgs& a, float kv_scale, hipStream_t st);
hipError_t launch_append_fp8(int T, const void* c_kv, const void* k_pe, const void* q_pe,
                             const int32_t* seq, const int32_t* pos, const int32_t* bt,
                             int num_seqs, int max_blocks, int64_t num_blocks, const float* cos,
                             const float* sin, int max_pos, float inv_scale, void* pool,
                             void* q_lat, uint32_t* err, hipStream_t st);
hipError_t launch_merge(const mla_config& c, const DecodeArgs& a, hipStream_t st);
hipError_t launch_merge_v3(const DecodeArgs& a, hipStream_t st);

}  // namespace mla
