// Bandwidth-bound passes: input pack, output unpack, 2x2 max-pool and the
// materialised nearest-2x upsample + concat.  One thread per output pixel (or
// per 4-channel block), consecutive threads on consecutive addresses, 16-byte
// loads where the layout allows.
#include "internal.h"
#include "image_io.h"

namespace oidn {
namespace {

constexpr int THREADS = 256;


// [webgpu-0.6] inputShader ("oidn-webgpu 0.0.0-stage -> 0.6.0",
// native/denoise.ts): clamp-to-edge read, sanitize, HDR log transfer of the
// scaled colour, normals to [0, 1], channels packed densely into 4-lane
// blocks with zero lanes ([web-0.4] createInputPackShader lane rule).
// With `taps` (fp16, 16 lanes, three images) lanes 8, 9, 10 hold channel 8
// (the normal's z) of the pixels in tile columns x - 1, x, x + 1, zero
// outside the tile -- the layout the first convs read as a tap chunk.
// DT: the storage type (OIDN_F32, OIDN_F16 or OIDN_BF16).
template <int DT>
__global__ __launch_bounds__(THREADS) void pack_input_kernel(PackArgs a) {
  const int n = a.tile_w * a.tile_h;
  const int t0 = blockIdx.x * THREADS + threadIdx.x;
  // lanes past the end compute the last pixel (for the tap shuffles) and store nothing
  const int t = t0 < n ? t0 : n - 1;
  const int ty = t / a.tile_w, tx = t - ty * a.tile_w;
  const int sy = min(max(ty + a.tile_y, 0), a.img_h - 1);
  const int sx = min(max(tx + a.tile_x, 0), a.img_w - 1);
  const size_t src = (size_t)sy * a.img_w + sx;
  float ch[12];
#pragma unroll
  for (int i = 0; i < 12; ++i) ch[i] = 0.f;
  const float4 col = a.color[src];
  ch[0] = in_color(col.x, a.hdr, a.input_scale);
  ch[1] = in_color(col.y, a.hdr, a.input_scale);
  ch[2] = in_color(col.z, a.hdr, a.input_scale);
  if (a.sources > 1) {
    const float4 al = a.albedo[src];
    ch[3] = in_albedo(al.x);
    ch[4] = in_albedo(al.y);
    ch[5] = in_albedo(al.z);
  }
  if (a.sources > 2) {
    const float4 nr = a.normal[src];
    ch[6] = in_normal(nr.x);
    ch[7] = in_normal(nr.y);
    ch[8] = in_normal(nr.z);
  }
  if (a.taps && a.sources > 2) {
    // channel 8 of the row neighbours inside the tile: from the neighbouring
    // lanes (consecutive pixels of a row), read directly at a wave's edge or
    // where the neighbour lane holds another row
    const int lane = threadIdx.x & 63;
    const float c8 = ch[8];
    float left = __shfl_up(c8, 1, 64), right = __shfl_down(c8, 1, 64);
    const size_t row = (size_t)sy * a.img_w;
    if (tx > 0 && (lane == 0 || t0 >= n))
      left = in_normal(a.normal[row + min(max(tx - 1 + a.tile_x, 0), a.img_w - 1)].z);
    if (tx + 1 < a.tile_w && (lane == 63 || t0 + 1 >= n))
      right = in_normal(a.normal[row + min(max(tx + 1 + a.tile_x, 0), a.img_w - 1)].z);
    ch[8] = tx > 0 ? left : 0.f;
    ch[9] = c8;
    ch[10] = tx + 1 < a.tile_w ? right : 0.f;
  }
  if (t0 >= n) return;
  const int nblk = a.lanes / 4;   // blocks past the data (lanes 12..15) are zero
  if constexpr (DT != OIDN_F32) {
    constexpr bool BF = DT == OIDN_BF16;
    uint2* out = static_cast<uint2*>(a.packed) + (size_t)t * nblk;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (b < nblk)
        out[b] = b < 3 ? make_uint2(pack2<BF>(ch[4 * b], ch[4 * b + 1]),
                                    pack2<BF>(ch[4 * b + 2], ch[4 * b + 3]))
                       : make_uint2(0u, 0u);
  } else {
    float4* out = static_cast<float4*>(a.packed) + (size_t)t * nblk;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (b < nblk)
        out[b] = b < 3 ? make_float4(ch[4 * b], ch[4 * b + 1], ch[4 * b + 2], ch[4 * b + 3])
                       : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// [webgpu-0.6] outputShader: sanitize the network RGB, invert the transfer and
// the input scale, alpha from the input colour; only the output rectangle.
__global__ __launch_bounds__(THREADS) void unpack_output_kernel(UnpackArgs a) {
  const OutputPass& p = a.o;
  const int t = blockIdx.x * THREADS + threadIdx.x;
  if (t >= p.out_w * p.out_h) return;
  const int y = t / p.out_w, x = t - y * p.out_w;
  const float4 net = a.net[(size_t)(y + p.in_off_y) * a.tile_w + x + p.in_off_x];
  const size_t o = (size_t)(y + p.out_y) * p.img_w + x + p.out_x;
  p.out[o] = output_pixel(net.x, net.y, net.z, p.color[o].w, p.hdr, p.input_scale);
}

// [web-0.4] createMaxPoolShader / [web-0.5] coalesced "channels" pool: one
// thread per (output pixel, 4-channel block), threads of a wave walk the
// blocks of consecutive pixels.
template <int DT>
__global__ __launch_bounds__(THREADS) void pool2x2_kernel(const void* x, int h, int w, int cs,
                                                          void* y) {
  const int nb = cs / 4;
  const int ow = w >> 1, oh = h >> 1;
  const size_t t = (size_t)blockIdx.x * THREADS + threadIdx.x;
  if (t >= (size_t)ow * oh * nb) return;
  const int b = (int)(t % nb);
  const size_t pix = t / nb;
  const int ox = (int)(pix % ow), oy = (int)(pix / ow);
  const size_t i00 = ((size_t)(2 * oy) * w + 2 * ox) * nb + b;
  const size_t i01 = i00 + nb;
  const size_t i10 = i00 + (size_t)w * nb;
  const size_t i11 = i10 + nb;
  if constexpr (DT == OIDN_BF16) {
    // bf16 -> fp32 is exact (the high half of the fp32 bits)
    const uint2* in = static_cast<const uint2*>(x);
    const uint2 a0 = in[i00], a1 = in[i01], a2 = in[i10], a3 = in[i11];
    auto lo = [](uint32_t u) { return __uint_as_float(u << 16); };
    auto hi = [](uint32_t u) { return __uint_as_float(u & 0xffff0000u); };
    const float m0 = fmaxf(fmaxf(lo(a0.x), lo(a1.x)), fmaxf(lo(a2.x), lo(a3.x)));
    const float m1 = fmaxf(fmaxf(hi(a0.x), hi(a1.x)), fmaxf(hi(a2.x), hi(a3.x)));
    const float m2 = fmaxf(fmaxf(lo(a0.y), lo(a1.y)), fmaxf(lo(a2.y), lo(a3.y)));
    const float m3 = fmaxf(fmaxf(hi(a0.y), hi(a1.y)), fmaxf(hi(a2.y), hi(a3.y)));
    // exact: each maximum is one of the bf16 inputs
    static_cast<uint2*>(y)[t] = make_uint2(pack_bf2(m0, m1), pack_bf2(m2, m3));
  } else if constexpr (DT == OIDN_F16) {
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    const half4* in = static_cast<const half4*>(x);
    const half4 a0 = in[i00], a1 = in[i01], a2 = in[i10], a3 = in[i11];
    half4 m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = fmaxf(fmaxf((float)a0[i], (float)a1[i]), fmaxf((float)a2[i], (float)a3[i]));
      m[i] = (_Float16)v;  // exact: v is one of the fp16 inputs
    }
    static_cast<half4*>(y)[t] = m;
  } else {
    const float4* in = static_cast<const float4*>(x);
    const float4 a0 = in[i00], a1 = in[i01], a2 = in[i10], a3 = in[i11];
    float4 m;
    m.x = fmaxf(fmaxf(a0.x, a1.x), fmaxf(a2.x, a3.x));
    m.y = fmaxf(fmaxf(a0.y, a1.y), fmaxf(a2.y, a3.y));
    m.z = fmaxf(fmaxf(a0.z, a1.z), fmaxf(a2.z, a3.z));
    m.w = fmaxf(fmaxf(a0.w, a1.w), fmaxf(a2.w, a3.w));
    static_cast<float4*>(y)[t] = m;
  }
}

// Materialised [up(low) | skip]: one thread per (pixel, 4-channel block of
// the concat); a block is 8 bytes (fp16) or 16 bytes (fp32).
template <typename Block>
__global__ __launch_bounds__(THREADS) void upcat_kernel(const Block* low, int nb_low,
                                                        const Block* skip, int nb_skip, int h,
                                                        int w, Block* z) {
  const int nb = nb_low + nb_skip;
  const size_t t = (size_t)blockIdx.x * THREADS + threadIdx.x;
  if (t >= (size_t)h * w * nb) return;
  const int b = (int)(t % nb);
  const size_t pix = t / nb;
  const int x = (int)(pix % w), y = (int)(pix / w);
  Block v;
  if (b < nb_low)
    v = low[((size_t)(y >> 1) * (w >> 1) + (x >> 1)) * nb_low + b];
  else
    v = skip[pix * nb_skip + (b - nb_low)];
  z[t] = v;
}

inline dim3 grid_for(size_t n) { return dim3((unsigned)((n + THREADS - 1) / THREADS)); }

}  // namespace

hipError_t launch_pack(const PackArgs& a, int dtype, hipStream_t stream) {
  const size_t n = (size_t)a.tile_w * a.tile_h;
  if (n == 0) return hipSuccess;
  if (dtype == OIDN_BF16)
    hipLaunchKernelGGL(pack_input_kernel<OIDN_BF16>, grid_for(n), dim3(THREADS), 0, stream, a);
  else if (dtype == OIDN_F16)
    hipLaunchKernelGGL(pack_input_kernel<OIDN_F16>, grid_for(n), dim3(THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL(pack_input_kernel<OIDN_F32>, grid_for(n), dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_unpack(const UnpackArgs& a, hipStream_t stream) {
  const size_t n = (size_t)a.o.out_w * a.o.out_h;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(unpack_output_kernel, grid_for(n), dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_pool(const void* x, int h, int w, int cs, void* y, int dtype, hipStream_t stream) {
  const size_t n = (size_t)(w / 2) * (h / 2) * (cs / 4);
  if (n == 0) return hipSuccess;
  if (dtype == OIDN_BF16)
    hipLaunchKernelGGL(pool2x2_kernel<OIDN_BF16>, grid_for(n), dim3(THREADS), 0, stream, x, h, w, cs, y);
  else if (dtype == OIDN_F16)
    hipLaunchKernelGGL(pool2x2_kernel<OIDN_F16>, grid_for(n), dim3(THREADS), 0, stream, x, h, w, cs, y);
  else
    hipLaunchKernelGGL(pool2x2_kernel<OIDN_F32>, grid_for(n), dim3(THREADS), 0, stream, x, h, w, cs, y);
  return hipGetLastError();
}

hipError_t launch_upcat(const void* low, int cs_low, const void* skip, int cs_skip, int h, int w,
                        void* z, bool b16, hipStream_t stream) {
  const int nb = (cs_low + cs_skip) / 4;
  const size_t n = (size_t)h * w * nb;
  if (n == 0) return hipSuccess;
  if (b16)
    hipLaunchKernelGGL(upcat_kernel<uint2>, grid_for(n), dim3(THREADS), 0, stream,
                       static_cast<const uint2*>(low), cs_low / 4, static_cast<const uint2*>(skip),
                       cs_skip / 4, h, w, static_cast<uint2*>(z));
  else
    hipLaunchKernelGGL(upcat_kernel<float4>, grid_for(n), dim3(THREADS), 0, stream,
                       static_cast<const float4*>(low), cs_low / 4, static_cast<const float4*>(skip),
                       cs_skip / 4, h, w, static_cast<float4*>(z));
  return hipGetLastError();
}

}  // namespace oidn
