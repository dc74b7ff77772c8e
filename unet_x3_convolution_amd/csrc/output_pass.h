// Per-pixel arithmetic of the output pass ([webgpu-0.6] outputShader), shared
// by the standalone unpack kernel and the last conv's fused epilogue so both
// give the same bits.  Device code only.
#pragma once
#include <hip/hip_runtime.h>

namespace oidn {

constexpr float kFltMax = 3.402823466e+38f;

// NaN -> 0, otherwise clamp to [lo, hi] (reading of the pages' sanitize()).
__device__ __forceinline__ float sanitize(float v, float lo, float hi) {
  if (v != v) return 0.f;
  return fminf(fmaxf(v, lo), hi);
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
