// Per-pixel arithmetic of the input pass ([webgpu-0.6] inputShader) and the
// output pass ([webgpu-0.6] outputShader), shared by the standalone kernels
// and the convs that run them in their prologue or epilogue, so that every
// route gives the same bits.  Device code only.
#pragma once
#include <hip/hip_runtime.h>

namespace oidn {

constexpr float kFltMax = 3.402823466e+38f;

// NaN -> 0, otherwise clamp to [lo, hi] (reading of the pages' sanitize()).
// fmaxf returns the other operand for a NaN, so with lo = 0 the clamp alone
// maps NaN to 0; other bounds test for it.
__device__ __forceinline__ float sanitize(float v, float lo, float hi) {
  if (lo == 0.f) return fminf(fmaxf(v, 0.f), hi);
  if (v != v) return 0.f;
  return fminf(fmaxf(v, lo), hi);
}

// log(1 + x) for 0 <= x <= FLT_MAX, for results that are rounded to 16 bits
// next: the hardware base-2 logarithm of u = fl(1 + x), times ln 2, times
// x / (u - 1), which cancels the rounding of 1 + x to first order
// (D. Goldberg, "What every computer scientist should know about
// floating-point arithmetic", 1991, the ln(1 + x) theorem of section 1.4).
// A few fp32 ulps against the library log1pf's 120-odd instructions: far
// below half an ulp of fp16 or bf16, so the stored value is the correctly
// rounded one or its neighbour.  u == 1 means x < 2^-24, where log1p(x)
// rounds to x; from x = 1 on the rounding of u moves log(u) by under an
// fp32 ulp and the factor is left out (1 / (u - 1) would underflow to zero
// near FLT_MAX).
__device__ __forceinline__ float log1p_narrow(float x) {
  const float u = 1.f + x;
  const float d = u - 1.f;
  if (d == 0.f) return x;
  const float corr = x < 1.f ? x * __builtin_amdgcn_rcpf(d) : 1.f;
  return __builtin_amdgcn_logf(u) * 0.693147180559945309f * corr;
}

// Input channels: colour through the HDR log transfer of the scaled value
// (hdr) or clamped to [0, 1]; albedo clamped to [0, 1]; normals from [-1, 1]
// to [0, 1].  NARROW: the value is stored as fp16 / bf16 (log1p_narrow),
// else as fp32 (the library log1pf).
template <bool NARROW = false>
__device__ __forceinline__ float in_color(float v, int hdr, float input_scale) {
  if (!hdr) return sanitize(v, 0.f, 1.f);
  const float x = sanitize(v * input_scale, 0.f, kFltMax);
  return NARROW ? log1p_narrow(x) : log1pf(x);
}
__device__ __forceinline__ float in_albedo(float v) { return sanitize(v, 0.f, 1.f); }
__device__ __forceinline__ float in_normal(float v) { return sanitize(v, -1.f, 1.f) * 0.5f + 0.5f; }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two channels as fp16 (round to nearest even), the first in the low half:
// one packed conversion instruction.
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
}

// Two channels as bf16 (round to nearest even), the first in the low half.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// ... in the 16-bit storage type: fp16, or bf16 (BF).
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (BF)
    return pack_bf2(a, b);
  else
    return pack_h2(a, b);
}

// e^v - 1 for 0 <= v <= FLT_MAX.  Below 1/2 the Taylor series to v^9
// (truncation under 1e-9 relative, no cancellation); from 1/2 on
// 2 * 2^(t - 1) - 1 with the hardware base-2 exponential, where
// t = v log2(e) is carried as a rounded head and its tail (the exact
// rounding error of the head plus v times the tail of log2(e)), the tail
// applied to first order; the halving keeps the head finite up to the
// overflow point (e^v - 1 rounds past FLT_MAX from v = 88.72284), above
// which the result is inf.  A few fp32 ulps against the library expm1f's
// longer sequence.
__device__ __forceinline__ float expm1_fast(float v) {
  constexpr float kLog2eHi = 1.44269502162933349609375f;
  constexpr float kLog2eLo = 1.925963033500011e-08f;
  constexpr float kLn2 = 0.693147180559945309f;
  float p = 1.f / 362880.f;
  p = fmaf(p, v, 1.f / 40320.f);
  p = fmaf(p, v, 1.f / 5040.f);
  p = fmaf(p, v, 1.f / 720.f);
  p = fmaf(p, v, 1.f / 120.f);
  p = fmaf(p, v, 1.f / 24.f);
  p = fmaf(p, v, 1.f / 6.f);
  p = fmaf(p, v, 0.5f);
  const float small = fmaf(p * v, v, v);
  const float hi = v * kLog2eHi;
  const float lo = fmaf(v, kLog2eHi, -hi) + v * kLog2eLo;
  const float e = __builtin_amdgcn_exp2f(hi - 1.f);   // hi - 1 is exact for 0.72 <= hi < 2^24
  const float big = fmaf(2.f, fmaf(e, lo * kLn2, e), -1.f);
  if (v > 88.8f) return __builtin_inff();
  return v < 0.5f ? small : big;
}

// Network RGB -> image RGBA: sanitize, invert the HDR log transfer and the
// input scale (hdr), else clamp to [0, 1]; alpha from the input colour.
// The scale is undone by one reciprocal and three products.
__device__ __forceinline__ float4 output_pixel(float r, float g, float b, float alpha, int hdr,
                                               float input_scale) {
  float4 o;
  if (hdr) {
    const float rs = 1.f / input_scale;
    o.x = expm1_fast(sanitize(r, 0.f, kFltMax)) * rs;
    o.y = expm1_fast(sanitize(g, 0.f, kFltMax)) * rs;
    o.z = expm1_fast(sanitize(b, 0.f, kFltMax)) * rs;
  } else {
    o.x = sanitize(r, 0.f, 1.f);
    o.y = sanitize(g, 0.f, 1.f);
    o.z = sanitize(b, 0.f, 1.f);
  }
  o.w = alpha;
  return o;
}

}  // namespace oidn
