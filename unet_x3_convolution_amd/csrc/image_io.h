// Per-pixel arithmetic of the input pass ([webgpu-0.6] inputShader) and the
// output pass ([webgpu-0.6] outputShader), shared by the standalone kernels
// and the convs that run them in their prologue or epilogue, so that every
// route gives the same bits.  Device code only.
#pragma once
#include <hip/hip_runtime.h>

namespace oidn {

constexpr float kFltMax = 3.402823466e+38f;

// NaN -> 0, otherwise clamp to [lo, hi] (reading of the pages' sanitize()).
__device__ __forceinline__ float sanitize(float v, float lo, float hi) {
  if (v != v) return 0.f;
  return fminf(fmaxf(v, lo), hi);
}

// Input channels: colour through the HDR log transfer of the scaled value
// (hdr) or clamped to [0, 1]; albedo clamped to [0, 1]; normals from [-1, 1]
// to [0, 1].
__device__ __forceinline__ float in_color(float v, int hdr, float input_scale) {
  return hdr ? log1pf(sanitize(v * input_scale, 0.f, kFltMax)) : sanitize(v, 0.f, 1.f);
}
__device__ __forceinline__ float in_albedo(float v) { return sanitize(v, 0.f, 1.f); }
__device__ __forceinline__ float in_normal(float v) { return sanitize(v, -1.f, 1.f) * 0.5f + 0.5f; }

// Two channels as fp16 (round to nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Two channels as bf16 (round to nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
}

// ... in the 16-bit storage type: fp16, or bf16 (BF).
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (BF)
    return pack_bf2(a, b);
  else
    return pack_h2(a, b);
}

// Network RGB -> image RGBA: sanitize, invert the HDR log transfer and the
// input scale (hdr), else clamp to [0, 1]; alpha from the input colour.
__device__ __forceinline__ float4 output_pixel(float r, float g, float b, float alpha, int hdr,
                                               float input_scale) {
  float4 o;
  if (hdr) {
    o.x = expm1f(sanitize(r, 0.f, kFltMax)) / input_scale;
    o.y = expm1f(sanitize(g, 0.f, kFltMax)) / input_scale;
    o.z = expm1f(sanitize(b, 0.f, kFltMax)) / input_scale;
  } else {
    o.x = sanitize(r, 0.f, 1.f);
    o.y = sanitize(g, 0.f, 1.f);
    o.z = sanitize(b, 0.f, 1.f);
  }
  o.w = alpha;
  return o;
}

}  // namespace oidn
