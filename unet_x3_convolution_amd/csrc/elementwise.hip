// Bandwidth-bound passes: input pack, output unpack, 2x2 max-pool and the
// materialised nearest-2x upsample + concat.  One thread per output pixel (or
// per 4-channel block), consecutive threads on consecutive addresses, 16-byte
// loads where the layout allows.
#include <type_traits>

#include "internal.h"
#include "image_io.h"

namespace oidn {
namespace {

constexpr int THREADS = 256;

// Streaming accesses.  Inputs that a wave reads in whole 64-byte lines and
// nothing reads again are loaded non-temporally, and the input pass, output
// pass and pool store whole-line outputs non-temporally: cold reads of a
// just-written cache then do not have to evict its dirty lines first.
// Measured on one MI355X after other work left dirty lines: the input pass
// 29.5 us instead of 44.6 with plain accesses, the pool 32.0 instead of
// 53.4, the output pass 20.1 instead of 31.2 (with clean caches plain
// accesses are 3-6% faster).  The materialised concat stores plainly, which
// is faster either way.  The input pass's 16-bit packed pixels of a whole
// wave leave through LDS as lane-contiguous 16-byte streaming stores.
// Partial-line accesses (the per-lane 8-byte channel blocks at a 24-byte
// pixel stride of a wave that reaches past the tile and of the fp32 input
// pass) stay cached, so that the neighbouring lanes' and waves' pieces of a
// line meet in L2.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float ld_stream(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream(float4* p, float4 v) {
  __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void st_stream(uint2* p, uint2 v) {
  __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}


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
  const float4 col = ld_stream(a.color + src);
  ch[0] = in_color<DT != OIDN_F32>(col.x, a.hdr, a.input_scale);
  ch[1] = in_color<DT != OIDN_F32>(col.y, a.hdr, a.input_scale);
  ch[2] = in_color<DT != OIDN_F32>(col.z, a.hdr, a.input_scale);
  if (a.sources > 1) {
    const float4 al = ld_stream(a.albedo + src);
    ch[3] = in_albedo(al.x);
    ch[4] = in_albedo(al.y);
    ch[5] = in_albedo(al.z);
  }
  if (a.sources > 2) {
    const float4 nr = ld_stream(a.normal + src);
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
  const int nblk = a.lanes / 4;   // blocks past the data (lanes 12..15) are zero
  if constexpr (DT != OIDN_F32) {
    constexpr bool BF = DT == OIDN_BF16;
    // A wave's 64 pixels are one contiguous run of 64 nblk 8-byte blocks:
    // when all of them are in the tile they go through LDS and out as
    // lane-contiguous 16-byte streaming stores (whole lines) instead of
    // nblk 8-byte stores per lane at a pixel stride.
    __shared__ __attribute__((aligned(16))) uint2 stage[THREADS * 4];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wbase = t0 - lane;                    // the wave's first pixel
    const bool whole = wbase + 64 <= n;             // wave-uniform
    uint2* wst = stage + wave * 64 * 4;
    if (whole) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (b < nblk)
          wst[lane * nblk + b] = b < 3 ? make_uint2(pack2<BF>(ch[4 * b], ch[4 * b + 1]),
                                                    pack2<BF>(ch[4 * b + 2], ch[4 * b + 3]))
                                       : make_uint2(0u, 0u);
    }
    __syncthreads();
    if (whole) {
      // 64 nblk blocks = 32 nblk 16-byte units; nblk is 3 or 4
      const uint4* src4 = reinterpret_cast<const uint4*>(wst);
      uint2* out = static_cast<uint2*>(a.packed) + (size_t)wbase * nblk;
      for (int u = lane; u < 32 * nblk; u += 64) {
        const uint4 v = src4[u];
        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(out) + u);
      }
      return;
    }
    if (t0 >= n) return;
    uint2* out = static_cast<uint2*>(a.packed) + (size_t)t * nblk;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (b < nblk)
        out[b] = b < 3 ? make_uint2(pack2<BF>(ch[4 * b], ch[4 * b + 1]),
                                    pack2<BF>(ch[4 * b + 2], ch[4 * b + 3]))
                       : make_uint2(0u, 0u);
  } else {
    if (t0 >= n) return;
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
// A block covers 2 x 256 pixels: each thread loads both of its pixels (256
// apart, so every load and store instruction stays lane-contiguous) before
// storing either.
constexpr int kUnpackPerThread = 2;
__global__ __launch_bounds__(THREADS) void unpack_output_kernel(UnpackArgs a) {
  const OutputPass& p = a.o;
  const int n = p.out_w * p.out_h;
  const int t0 = blockIdx.x * THREADS * kUnpackPerThread + threadIdx.x;
  float4 net[kUnpackPerThread];
  float alpha[kUnpackPerThread];
  size_t o[kUnpackPerThread];
#pragma unroll
  for (int k = 0; k < kUnpackPerThread; ++k) {
    const int t = t0 + k * THREADS;
    if (t >= n) break;
    const int y = t / p.out_w, x = t - y * p.out_w;
    net[k] = ld_stream(a.net + (size_t)(y + p.in_off_y) * a.tile_w + x + p.in_off_x);
    o[k] = (size_t)(y + p.out_y) * p.img_w + x + p.out_x;
    alpha[k] = ld_stream(reinterpret_cast<const float*>(p.color + o[k]) + 3);
  }
#pragma unroll
  for (int k = 0; k < kUnpackPerThread; ++k) {
    if (t0 + k * THREADS >= n) break;
    st_stream(p.out + o[k], output_pixel(net[k].x, net[k].y, net[k].z, alpha[k], p.hdr, p.input_scale));
  }
}

// [web-0.4] createMaxPoolShader / [web-0.5] coalesced "channels" pool: one
// thread per two (output pixel, 4-channel block) items of an output row,
// 256 apart (threads of a wave walk the blocks of consecutive pixels, every
// instruction stays lane-contiguous); all eight loads are issued before the
// maxima.  blockIdx.y is the output row, so the index arithmetic stays in
// 32 bits.
constexpr int kPoolPerThread = 2;
template <int DT>
__global__ __launch_bounds__(THREADS) void pool2x2_kernel(const void* x, int h, int w, int cs,
                                                          void* y) {
  // a 4-channel block: fp32 x 4, fp16 x 4, or bf16 x 4 as two 32-bit words
  typedef _Float16 half4 __attribute__((ext_vector_type(4)));
  using Blk = std::conditional_t<DT == OIDN_F32, float4,
                                 std::conditional_t<DT == OIDN_F16, half4, uint2>>;
  const Blk* in = static_cast<const Blk*>(x);
  Blk* out = static_cast<Blk*>(y);
  const int nb = cs / 4;
  const int ow = w >> 1, oh = h >> 1;
  const int r0 = blockIdx.x * THREADS * kPoolPerThread + threadIdx.x;
  for (int oy = blockIdx.y; oy < oh; oy += gridDim.y) {
    Blk v[kPoolPerThread][4];
    size_t t[kPoolPerThread];
#pragma unroll
    for (int k = 0; k < kPoolPerThread; ++k) {
      const int r = r0 + k * THREADS;   // (pixel, block) within the row
      if (r >= ow * nb) break;
      const int ox = r / nb, b = r - ox * nb;
      t[k] = (size_t)oy * ow * nb + r;
      const size_t i00 = ((size_t)(2 * oy) * w + 2 * ox) * nb + b;
      const size_t i10 = i00 + (size_t)w * nb;
      if constexpr (DT == OIDN_F16) {
        v[k][0] = __builtin_nontemporal_load(in + i00);
        v[k][1] = __builtin_nontemporal_load(in + i00 + nb);
        v[k][2] = __builtin_nontemporal_load(in + i10);
        v[k][3] = __builtin_nontemporal_load(in + i10 + nb);
      } else {
        v[k][0] = ld_stream(in + i00);
        v[k][1] = ld_stream(in + i00 + nb);
        v[k][2] = ld_stream(in + i10);
        v[k][3] = ld_stream(in + i10 + nb);
      }
    }
#pragma unroll
    for (int k = 0; k < kPoolPerThread; ++k) {
      if (r0 + k * THREADS >= ow * nb) break;
      const Blk* a = v[k];
      if constexpr (DT == OIDN_F32) {
        float4 m;
        m.x = fmaxf(fmaxf(a[0].x, a[1].x), fmaxf(a[2].x, a[3].x));
        m.y = fmaxf(fmaxf(a[0].y, a[1].y), fmaxf(a[2].y, a[3].y));
        m.z = fmaxf(fmaxf(a[0].z, a[1].z), fmaxf(a[2].z, a[3].z));
        m.w = fmaxf(fmaxf(a[0].w, a[1].w), fmaxf(a[2].w, a[3].w));
        st_stream(out + t[k], m);
      } else if constexpr (DT == OIDN_F16) {
        half4 m;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float mv = fmaxf(fmaxf((float)a[0][i], (float)a[1][i]), fmaxf((float)a[2][i], (float)a[3][i]));
          m[i] = (_Float16)mv;   // exact: mv is one of the fp16 inputs
        }
        __builtin_nontemporal_store(m, out + t[k]);
      } else {
        // bf16 -> fp32 is exact (the high half of the fp32 bits); the maximum
        // is one of the inputs, so converting it back is exact too
        auto lo = [](uint32_t u) { return __uint_as_float(u << 16); };
        auto hi = [](uint32_t u) { return __uint_as_float(u & 0xffff0000u); };
        float m[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint32_t w0 = i ? a[0].y : a[0].x, w1 = i ? a[1].y : a[1].x;
          const uint32_t w2 = i ? a[2].y : a[2].x, w3 = i ? a[3].y : a[3].x;
          m[2 * i] = fmaxf(fmaxf(lo(w0), lo(w1)), fmaxf(lo(w2), lo(w3)));
          m[2 * i + 1] = fmaxf(fmaxf(hi(w0), hi(w1)), fmaxf(hi(w2), hi(w3)));
        }
        st_stream(out + t[k], make_uint2(pack_bf2(m[0], m[1]), pack_bf2(m[2], m[3])));
      }
    }
  }
}

// Materialised [up(low) | skip] in 8-byte words (a 4-channel block of fp16
// or bf16, half a block of fp32): lw / sw words per pixel of the
// low-resolution and skip sources, pw = lw + sw per output pixel.  A
// workgroup writes output rows 2 ly and 2 ly + 1 over the pixel span
// [x0, x0 + n) (x0 and n even): it copies the low-resolution span and both
// skip-row spans into LDS with consecutive-lane loads, then writes each
// output row span as consecutive 16-byte units gathered from LDS (a unit
// may straddle the low/skip boundary or two pixels).  `magic` is
// ceil(2^32 / pw): floor(word / pw) = umulhi(word, magic) for the span's
// word indices (below 2^16).
__global__ __launch_bounds__(THREADS) void upcat_kernel(const uint2* __restrict__ low, int lw,
                                                        const uint2* __restrict__ skip, int sw,
                                                        int h, int w, int seg, unsigned magic,
                                                        uint4* __restrict__ z) {
  extern __shared__ uint2 sm[];
  const int tid = threadIdx.x;
  const int pw = lw + sw;
  const int x0 = blockIdx.x * seg;
  const int n = min(seg, w - x0);
  uint2* const slow = sm;
  uint2* const sskip = sm + (n >> 1) * lw;
  const int nlow = (n >> 1) * lw, nskip = n * sw;
  const int units = (n * pw) >> 1;                 // 16-byte units per output row span
  for (int ly = blockIdx.y; ly < (h >> 1); ly += gridDim.y) {
    const size_t lbase = ((size_t)ly * (w >> 1) + (x0 >> 1)) * lw;
    for (int i = tid; i < nlow; i += THREADS) slow[i] = ld_stream(low + lbase + i);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const size_t sbase = ((size_t)(2 * ly + r) * w + x0) * sw;
      for (int i = tid; i < nskip; i += THREADS) sskip[r * nskip + i] = ld_stream(skip + sbase + i);
    }
    __syncthreads();
    for (int u = tid; u < 2 * units; u += THREADS) {
      const int r = u >= units ? 1 : 0;
      const int uu = u - r * units;
      uint2 v[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const unsigned word = 2 * uu + k;
        const int p = (int)__umulhi(word, magic);
        const int off = (int)word - p * pw;
        v[k] = off < lw ? slow[(p >> 1) * lw + off] : sskip[r * nskip + p * sw + (off - lw)];
      }
      // a plain store: kept in the caches, the concat's lines are written
      // back whole (streaming stores measured 10% slower here, with the
      // caches clean or dirty)
      const size_t zo = (((size_t)(2 * ly + r) * w + x0) * pw >> 1) + uu;
      z[zo] = make_uint4(v[0].x, v[0].y, v[1].x, v[1].y);
    }
    __syncthreads();
  }
}

inline dim3 grid_for(size_t n) { return dim3((unsigned)((n + THREADS - 1) / THREADS)); }
// Rows per launch of the row-indexed kernels (grid y); they step over the rest.
constexpr int kMaxGridRows = 32768;
inline unsigned grid_rows(int rows) { return (unsigned)(rows < kMaxGridRows ? rows : kMaxGridRows); }

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
  hipLaunchKernelGGL(unpack_output_kernel, grid_for((n + kUnpackPerThread - 1) / kUnpackPerThread),
                     dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_pool(const void* x, int h, int w, int cs, void* y, int dtype, hipStream_t stream) {
  const size_t row = (size_t)(w / 2) * (cs / 4);   // items per output row
  if (row == 0 || h / 2 == 0) return hipSuccess;
  const dim3 grid(grid_for((row + kPoolPerThread - 1) / kPoolPerThread).x, grid_rows(h / 2));
  if (dtype == OIDN_BF16)
    hipLaunchKernelGGL(pool2x2_kernel<OIDN_BF16>, grid, dim3(THREADS), 0, stream, x, h, w, cs, y);
  else if (dtype == OIDN_F16)
    hipLaunchKernelGGL(pool2x2_kernel<OIDN_F16>, grid, dim3(THREADS), 0, stream, x, h, w, cs, y);
  else
    hipLaunchKernelGGL(pool2x2_kernel<OIDN_F32>, grid, dim3(THREADS), 0, stream, x, h, w, cs, y);
  return hipGetLastError();
}

hipError_t launch_upcat(const void* low, int cs_low, const void* skip, int cs_skip, int h, int w,
                        void* z, bool b16, hipStream_t stream) {
  // 8-byte words per pixel: a 4-channel block is one word in 16 bits, two in fp32
  const int lw = (cs_low / 4) * (b16 ? 1 : 2), sw = (cs_skip / 4) * (b16 ? 1 : 2);
  if (w < 2 || h < 2) return hipSuccess;
  // span: even, at most 256 pixels, LDS (half a span of low pixels and two
  // rows of skip pixels) within 16 KB.  Measured at 960x544x64 + 1920x1088x12
  // fp16 (event-timed, clean / dirty caches): 16 KB 76 / 89 us, 14 KB
  // 81 / 83, 20 KB 83 / 86, 24 KB 88 / 91.
  const int per_px = 4 * lw + 16 * sw;             // bytes of LDS per span pixel
  int seg = 16 * 1024 / per_px;
  seg = seg > 256 ? 256 : seg < 2 ? 2 : seg;
  seg &= ~1;
  if (seg > w) seg = w;
  const int pw = lw + sw;
  const unsigned magic = (unsigned)((0x100000000ull + pw - 1) / pw);
  const size_t lds = (size_t)((seg >> 1) * lw + 2 * seg * sw) * 8;
  const dim3 grid(cdiv(w, seg), grid_rows(h / 2));
  hipLaunchKernelGGL(upcat_kernel, grid, dim3(THREADS), lds, stream, static_cast<const uint2*>(low),
                     lw, static_cast<const uint2*>(skip), sw, h, w, seg, magic, static_cast<uint4*>(z));
  return hipGetLastError();
}

}  // namespace oidn
