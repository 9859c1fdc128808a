// RoPE of the shared key and of the queries, rotate-half pairing
// ([MLA explainer] "MLA的实现", RoPE module: y = x*cos + rotate_half(x)*sin,
// pairs (i, i + d_r/2)), with every product and sum rounded to fp32 (no fused
// multiply-add) so that cache rows are bit-exact and independent of the device.
#pragma once

#include "mla_internal.h"

namespace mla {

constexpr int kV3Dc = 512, kV3Dr = 64, kV3H = 128, kV3Row = 576, kV3Half = 32;

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

// DeepSeek-V3 RoPE width (64, 32 pairs), bf16 input: rotates the 8 pairs
// i0 .. i0+7 of x into fp32 y1[j] (element i0+j) and y2[j] (element i0+32+j)
// (16-byte loads; x 16-byte aligned).
__device__ __forceinline__ void rope8_pairs(const uint16_t* x, const float* cr, const float* sr,
                                            int i0, float* y1, float* y2) {
  const u32x4 a = *(const u32x4*)(x + i0);            // x[i0 .. i0+7]
  const u32x4 b = *(const u32x4*)(x + kV3Half + i0);  // x[i0+32 .. i0+39]
  const f32x4 c0 = *(const f32x4*)(cr + i0), c1 = *(const f32x4*)(cr + i0 + 4);
  const f32x4 s0 = *(const f32x4*)(sr + i0), s1 = *(const f32x4*)(sr + i0 + 4);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float x1 = bf16_bits_to_f32((uint16_t)(a[j >> 1] >> (16 * (j & 1))));
    const float x2 = bf16_bits_to_f32((uint16_t)(b[j >> 1] >> (16 * (j & 1))));
    const float c = j < 4 ? c0[j] : c1[j - 4];
    const float sn = j < 4 ? s0[j] : s1[j - 4];
    rope_pair(x1, x2, c, sn, y1[j], y2[j]);
  }
}

// The same rotation stored as bf16 (nearest even) at y + i0 and y + 32 + i0
// (16-byte stores; y 16-byte aligned).
__device__ __forceinline__ void rope8_bf16(const uint16_t* x, const float* cr, const float* sr,
                                           int i0, uint16_t* y) {
  float y1[8], y2[8];
  rope8_pairs(x, cr, sr, i0, y1, y2);
  uint32_t o1[4], o2[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o1[k] = (uint32_t)f32_to_bf16_bits(y1[2 * k]) | ((uint32_t)f32_to_bf16_bits(y1[2 * k + 1]) << 16);
    o2[k] = (uint32_t)f32_to_bf16_bits(y2[2 * k]) | ((uint32_t)f32_to_bf16_bits(y2[2 * k + 1]) << 16);
  }
  *(u32x4*)(y + i0) = u32x4{o1[0], o1[1], o1[2], o1[3]};
  *(u32x4*)(y + kV3Half + i0) = u32x4{o2[0], o2[1], o2[2], o2[3]};
}

}  // namespace mla
