// fp32 3x3 convolution on the vector ALUs (fp32 storage, fp32 FMA).
//
// The arithmetic is [web-0.4] createConvShader ("oidn-web 0.3.4 -> 0.4.0",
// nativeUNet.ts): one thread owns one 4-channel output block of one output
// pixel, starts from the bias, skips taps outside the image and accumulates
// fma(x[i], w[i][0..3], acc) over taps and stored input channels.  The
// decoder form reads the upsampled source at (y >> 1, x >> 1)
// (createFusedDecoderShader); the pooled form evaluates the 2x2 window and
// keeps the max (createFusedConvPoolShader).  Weights:
// [out block][tap][stored input channel over both sources][4 out lanes].
#include "internal.h"

namespace oidn {
namespace {

constexpr int THREADS = 256;

__device__ __forceinline__ float4 conv_at(const ConvF32Args& a, bool upcat, int y, int x,
                                          int ob) {
  const int cin = a.cs0 + a.cs1;
  float4 acc = reinterpret_cast<const float4*>(a.bias)[ob];
  const float4* wob = reinterpret_cast<const float4*>(a.wt) + (size_t)ob * 9 * cin;
  for (int ky = 0; ky < 3; ++ky) {
    const int iy = y + ky - 1;
    if (iy < 0 || iy >= a.h) continue;
    for (int kx = 0; kx < 3; ++kx) {
      const int ix = x + kx - 1;
      if (ix < 0 || ix >= a.w) continue;
      const float4* wt = wob + (ky * 3 + kx) * cin;
      const float* s0 = upcat ? a.src0 + ((size_t)(iy >> 1) * (a.w >> 1) + (ix >> 1)) * a.cs0
                              : a.src0 + ((size_t)iy * a.w + ix) * a.cs0;
      for (int i = 0; i < a.cs0; ++i) {
        const float v = s0[i];
        const float4 wv = wt[i];
        acc.x = fmaf(v, wv.x, acc.x);
        acc.y = fmaf(v, wv.y, acc.y);
        acc.z = fmaf(v, wv.z, acc.z);
        acc.w = fmaf(v, wv.w, acc.w);
      }
      if (a.cs1) {
        const float* s1 = a.src1 + ((size_t)iy * a.w + ix) * a.cs1;
        for (int i = 0; i < a.cs1; ++i) {
          const float v = s1[i];
          const float4 wv = wt[a.cs0 + i];
          acc.x = fmaf(v, wv.x, acc.x);
          acc.y = fmaf(v, wv.y, acc.y);
          acc.z = fmaf(v, wv.z, acc.z);
          acc.w = fmaf(v, wv.w, acc.w);
        }
      }
    }
  }
  return acc;
}

__device__ __forceinline__ float4 relu4(float4 v) {
  return make_float4(fmaxf(v.x, 0.f), fmaxf(v.y, 0.f), fmaxf(v.z, 0.f), fmaxf(v.w, 0.f));
}

__device__ __forceinline__ float4 max4(float4 a, float4 b) {
  return make_float4(fmaxf(a.x, b.x), fmaxf(a.y, b.y), fmaxf(a.z, b.z), fmaxf(a.w, b.w));
}

__global__ __launch_bounds__(THREADS) void conv3x3_f32_direct(ConvF32Args a, int upcat, int pool,
                                                              int relu) {
  const int oblocks = a.cout_stored / 4;
  const int ow = pool ? a.w >> 1 : a.w;
  const int oh = pool ? a.h >> 1 : a.h;
  const size_t total = (size_t)ow * oh * oblocks;
  const size_t t = (size_t)blockIdx.x * THREADS + threadIdx.x;
  if (t >= total) return;
  const int ob = (int)(t % oblocks);
  const size_t pix = t / oblocks;
  const int x = (int)(pix % ow);
  const int y = (int)(pix / ow);
  float4 v;
  if (!pool) {
    v = conv_at(a, upcat, y, x, ob);
    if (relu) v = relu4(v);
  } else {
    v = make_float4(-3.402823466e+38f, -3.402823466e+38f, -3.402823466e+38f, -3.402823466e+38f);
    for (int py = 0; py < 2; ++py)
      for (int px = 0; px < 2; ++px) {
        float4 c = conv_at(a, upcat, 2 * y + py, 2 * x + px, ob);
        if (relu) c = relu4(c);
        v = max4(v, c);
      }
  }
  reinterpret_cast<float4*>(a.y)[pix * oblocks + ob] = v;
}

}  // namespace

size_t conv_f32_bytes(int cin_stored_total, int cout) {
  const int cs = stored_channels(cout);
  return align256(sizeof(float) * cs) + sizeof(float) * (size_t)(cs / 4) * 9 * cin_stored_total * 4;
}

hipError_t launch_conv_f32(const ConvF32Args& a, bool upcat, bool pool, bool relu,
                           hipStream_t stream) {
  const int ow = pool ? a.w >> 1 : a.w;
  const int oh = pool ? a.h >> 1 : a.h;
  const size_t total = (size_t)ow * oh * (a.cout_stored / 4);
  if (total == 0) return hipSuccess;
  const dim3 grid((unsigned)((total + THREADS - 1) / THREADS)), block(THREADS);
  hipLaunchKernelGGL(conv3x3_f32_direct, grid, block, 0, stream, a, (int)upcat, (int)pool,
                     (int)relu);
  return hipGetLastError();
}

}  // namespace oidn
