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

// DeepSeek-V3 RoPE width (64, 32 pairs), bf16: rotates the 8 pairs i0 .. i0+7
// of x (16-byte loads and stores; x and y 16-byte aligned).
__device__ __forceinline__ void rope8_bf16(const uint16_t* x, const float* cr, const float* sr,
                                           int i0, uint16_t* y) {
  const u32x4 a = *(const u32x4*)(x + i0);            // x[i0 .. i0+7]
  const u32x4 b = *(const u32x4*)(x + kV3Half + i0);  // x[i0+32 .. i0+39]
  const f32x4 c0 = *(const f32x4*)(cr + i0), c1 = *(const f32x4*)(cr + i0 + 4);
  const f32x4 s0 = *(const f32x4*)(sr + i0), s1 = *(const f32x4*)(sr + i0 + 4);
  uint32_t o1[4], o2[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float y1[2], y2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = 2 * k + e;  // pair i0 + j
      const float x1 = bf16_bits_to_f32((uint16_t)(a[k] >> (16 * e)));
      const float x2 = bf16_bits_to_f32((uint16_t)(b[k] >> (16 * e)));
      const float c = j < 4 ? c0[j] : c1[j - 4];
      const float sn = j < 4 ? s0[j] : s1[j - 4];
      rope_pair(x1, x2, c, sn, y1[e], y2[e]);
    }
    o1[k] = (uint32_t)f32_to_bf16_bits(y1[0]) | ((uint32_t)f32_to_bf16_bits(y1[1]) << 16);
    o2[k] = (uint32_t)f32_to_bf16_bits(y2[0]) | ((uint32_t)f32_to_bf16_bits(y2[1]) << 16);
  }
  *(u32x4*)(y + i0) = u32x4{o1[0], o1[1], o1[2], o1[3]};
  *(u32x4*)(y + kV3Half + i0) = u32x4{o2[0], o2[1], o2[2], o2[3]};
}

}  // namespace mla
