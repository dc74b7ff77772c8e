// 3x3 convolution as an fp16 MFMA implicit GEMM with fp32 accumulation
// (gfx950, v_mfma_f32_16x16x32_f16), persistent and software-pipelined.
//
// What it computes is [web-0.4] createConvShader / createTiledConvShader /
// createTiledDecoderShader / createFusedConvPoolShader ("oidn-web 0.3.4 ->
// 0.4.0", nativeUNet.ts): y = act(b + sum over taps and input channels of
// W * x) with zero padding, optionally over [nearest-2x-upsampled source,
// skip] and optionally followed by a 2x2 max-pool.  The tiling is our own:
//
//  * GEMM roles: D[cout][pixel] = A[cout][k] * B[k][pixel].  A holds packed
//    weights (global memory, L2/L1 resident), B is read straight from an LDS
//    halo patch (no im2col), so each lane of a 16x16 accumulator owns 4
//    consecutive output channels of one pixel -- a whole 4-lane channel
//    block, stored with one 8-byte write.
//  * A workgroup of 4 waves computes (4 R) x 16 pixel tiles for NFW of the
//    nf output fragments; wave w owns R consecutive rows of a tile, one
//    16-pixel B fragment per row.
//  * K order: chunk (32 channels of one source) -> column group kx (the four
//    8-channel groups of the chunk, one per 16-lane group) -> ky.  All lanes
//    of a column group read the same patch row, so the B fragment of patch
//    row p serves output rows p, p - 1 and p - 2 with the weights of
//    ky = 0, 1, 2: R + 2 fragment loads per column group instead of 3 R.
//  * Pipeline.  Workgroups are persistent: each walks a list of (tile,
//    chunk) items.  While item k computes from one LDS patch buffer, the halo
//    patch and the weight fragments of item k + 1 are already in flight into
//    the other pair of buffers by direct global -> LDS loads
//    (global_load_lds: no registers, one copy of the weights per workgroup).
//    Nothing inside the MFMA phase waits on them; the one barrier per item
//    drains them.  The buffer pairs are distinct arrays selected at compile
//    time (the item loop is unrolled by two) so the compiler can see that
//    reads of one never alias the loads into the other.
//  * The decoder's upsampled source is gathered at (y >> 1, x >> 1) by the
//    patch loads; the skip follows as further chunks (concat order [up, skip]).
//    Channels past a source's stored count, and pixels outside the image,
//    load from a 16-byte zero block, which gives the zero padding.
//  * Epilogue: bias, ReLU, then the store or the fused 2x2 pool: the vertical
//    pair sits in two rows held by the same lane, the horizontal pair in
//    neighbouring lanes (one DPP swap).  Max is taken in fp32 before the
//    single fp16 rounding; RNE is monotone, so this equals pooling the
//    rounded conv output.
//  * Tiles are dealt so that each of the 8 XCDs walks a contiguous band of
//    tiles (halo rows shared through its own L2).
//
// The per-pixel reduction order depends only on the channel layout, never on
// the pixel position or the image size, so tiled and untiled runs agree bit
// for bit wherever their inputs agree.
#include "internal.h"

namespace oidn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int TW = 16;                 // tile width (one B fragment)
constexpr int PW = TW + 2;             // patch width
constexpr int SLOT_HALVES = 8;         // one 16-byte LDS slot
constexpr int PIX_SLOTS = 5;           // per patch pixel: 4 channel groups + 1 pad (80 B stride,
                                       // conflict-free 16-byte fragment reads)
constexpr int PIX_HALVES = PIX_SLOTS * SLOT_HALVES;
constexpr int THREADS = 256;
constexpr int kXcds = 8;
constexpr int kCUs = 256;

// Zero block that padding lanes of the patch loads read from.
__device__ __attribute__((aligned(16))) unsigned int g_zero16[4] = {0u, 0u, 0u, 0u};

template <int R>
struct Tile {
  static constexpr int TH = 4 * R;
  static constexpr int PH = TH + 2;
  static constexpr int PIX = PH * PW;
  static constexpr int SLOTS = PIX * PIX_SLOTS;
  static constexpr int LOADS16 = (SLOTS + 63) / 64;       // 16-byte-per-lane wave loads
  static constexpr int LOADS4 = (SLOTS * 4 + 63) / 64;    // 4-byte-per-lane wave loads
  static constexpr int BUF_SLOTS = LOADS16 * 64;          // >= LOADS4 * 16
};

__device__ __forceinline__ half8 as_half8(uint4 v) { return __builtin_bit_cast(half8, v); }

// Global -> LDS loads of one chunk's halo patch into `buf` (BUF_SLOTS slots).
// Wave load k fills slots [64 k, 64 k + 64); slot s is pixel s / 5, channel
// group s % 5 (group 4 is the pad slot).  Sources whose stored channel count
// is a multiple of 8 move 16 bytes per lane; others (the 12-channel network
// input) move 4 bytes per lane.
template <int R>
__device__ __forceinline__ void load_patch(uint4* buf, const _Float16* src, int cs, int coff,
                                           bool up, int h, int w, int y0, int x0, int wave,
                                           int lane) {
  using T = Tile<R>;
  const int sw = up ? (w >> 1) : w;
  if ((cs & 7) == 0) {
    for (int k = wave; k < T::LOADS16; k += 4) {
      const int s = k * 64 + lane;
      const int p = s / PIX_SLOTS;
      const int u = s - p * PIX_SLOTS;
      const void* gp = g_zero16;
      if (u < 4 && p < T::PIX) {
        const int py = p / PW;
        const int iy = y0 - 1 + py;
        const int ix = x0 - 1 + (p - py * PW);
        const int c = coff + 8 * u;
        if (iy >= 0 && iy < h && ix >= 0 && ix < w && c < cs) {
          const int sy = up ? (iy >> 1) : iy;
          const int sx = up ? (ix >> 1) : ix;
          gp = src + ((size_t)sy * sw + sx) * cs + c;
        }
      }
      __builtin_amdgcn_global_load_lds(gp, buf + k * 64, 16, 0, 0);
    }
  } else {
    for (int k = wave; k < T::LOADS4; k += 4) {
      const int d = k * 64 + lane;          // dword index
      const int s = d >> 2;
      const int p = s / PIX_SLOTS;
      const int u = s - p * PIX_SLOTS;
      const void* gp = g_zero16;
      if (u < 4 && p < T::PIX) {
        const int py = p / PW;
        const int iy = y0 - 1 + py;
        const int ix = x0 - 1 + (p - py * PW);
        const int c = coff + 8 * u + 2 * (d & 3);
        if (iy >= 0 && iy < h && ix >= 0 && ix < w && c < cs) {
          const int sy = up ? (iy >> 1) : iy;
          const int sx = up ? (ix >> 1) : ix;
          gp = src + ((size_t)sy * sw + sx) * cs + c;
        }
      }
      __builtin_amdgcn_global_load_lds(gp, reinterpret_cast<uint32_t*>(buf) + k * 64, 4, 0, 0);
    }
  }
}

// Global -> LDS loads of one chunk's weights for output fragments
// [q0, q0 + NFW) (wchunk already offset by q0): LDS fragment (3 j + ky) * NFW + q
// is global fragment chunk.wfrag + (3 j + ky) * nf + q, one 1 KB wave load each.
template <int NFW>
__device__ __forceinline__ void load_weights(uint4* abuf, const uint4* wchunk, int nf, int wave) {
  for (int i = wave; i < 9 * NFW; i += 4) {
    const int jk = i / NFW;
    __builtin_amdgcn_global_load_lds(wchunk + (jk * nf + (i - jk * NFW)) * 64, abuf + i * 64, 16,
                                     0, 0);
  }
}

template <int NFW, int R>
__device__ __forceinline__ void mma_chunk(floatx4 (&acc)[R][NFW], const uint4* abuf,
                                          const uint4* buf, int wave, int g, int c, int lane) {
  const _Float16* patch = reinterpret_cast<const _Float16*>(buf);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    uint4 a[3][NFW];
#pragma unroll
    for (int ky = 0; ky < 3; ++ky)
#pragma unroll
      for (int q = 0; q < NFW; ++q) a[ky][q] = abuf[((3 * j + ky) * NFW + q) * 64 + lane];
    const int base = ((R * wave) * PW + c + j) * PIX_HALVES + SLOT_HALVES * g;
#pragma unroll
    for (int p = 0; p < R + 2; ++p) {
      const half8 b = *reinterpret_cast<const half8*>(patch + base + p * PW * PIX_HALVES);
#pragma unroll
      for (int ky = 0; ky < 3; ++ky) {
        const int r = p - ky;
        if (r >= 0 && r < R) {
#pragma unroll
          for (int q = 0; q < NFW; ++q)
            acc[r][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(a[ky][q]), b,
                                                               acc[r][q], 0, 0, 0);
        }
      }
    }
  }
}

__device__ __forceinline__ float act(float v, int relu) { return relu ? fmaxf(v, 0.f) : v; }

__device__ __forceinline__ float swap_pair(float v) {
  // DPP quad_perm [1, 0, 3, 2]: exchange with the neighbouring lane.
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

template <bool OUTF32>
__device__ __forceinline__ void store4(void* y, size_t idx, float v0, float v1, float v2, float v3) {
  if constexpr (OUTF32) {
    *reinterpret_cast<float4*>(static_cast<float*>(y) + idx) = make_float4(v0, v1, v2, v3);
  } else {
    const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1, h2 = (_Float16)v2, h3 = (_Float16)v3;
    uint2 p;
    p.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    p.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
    *reinterpret_cast<uint2*>(static_cast<_Float16*>(y) + idx) = p;
  }
}

// Bias, ReLU, optional 2x2 pool, store; then clear the accumulators.
template <int NFW, int R, bool OUTF32>
__device__ __forceinline__ void epilogue(floatx4 (&acc)[R][NFW], const ConvF16Args& a, int q0,
                                         int y0, int x0, int wave, int g, int c, int pool,
                                         int relu) {
  const int cbase = 4 * a.nf * g + 4 * q0;
  float bv[NFW][4];
#pragma unroll
  for (int q = 0; q < NFW; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) bv[q][i] = a.bias[cbase + 4 * q + i];
  const int x = x0 + c;
  const int yb = y0 + R * wave;
  if (!pool) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int yy = yb + r;
      if (yy < a.h && x < a.w) {
        const size_t base = ((size_t)yy * a.w + x) * a.cout_stored + cbase;
#pragma unroll
        for (int q = 0; q < NFW; ++q)
          if (cbase + 4 * q < a.cout_stored)
            store4<OUTF32>(a.y, base + 4 * q, act(acc[r][q][0] + bv[q][0], relu),
                           act(acc[r][q][1] + bv[q][1], relu), act(acc[r][q][2] + bv[q][2], relu),
                           act(acc[r][q][3] + bv[q][3], relu));
      }
    }
  } else {
    const int ow = a.w >> 1;
#pragma unroll
    for (int rp = 0; rp < R / 2; ++rp) {
      float m[NFW][4];
#pragma unroll
      for (int q = 0; q < NFW; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = act(fmaxf(acc[2 * rp][q][i], acc[2 * rp + 1][q][i]) + bv[q][i], relu);
          m[q][i] = fmaxf(v, swap_pair(v));
        }
      const int yy = yb + 2 * rp;
      if ((c & 1) == 0 && yy < a.h && x < a.w) {
        const size_t base = ((size_t)(yy >> 1) * ow + (x >> 1)) * a.cout_stored + cbase;
#pragma unroll
        for (int q = 0; q < NFW; ++q)
          if (cbase + 4 * q < a.cout_stored)
            store4<OUTF32>(a.y, base + 4 * q, m[q][0], m[q][1], m[q][2], m[q][3]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int q = 0; q < NFW; ++q) acc[r][q] = floatx4{0.f, 0.f, 0.f, 0.f};
}

template <int NFW, int R, bool OUTF32>
__global__ __launch_bounds__(THREADS, 1) void conv3x3_f16_mfma(ConvF16Args a, int upcat, int pool,
                                                                int relu) {
  using T = Tile<R>;
  __shared__ __attribute__((aligned(16))) uint4 buf0[T::BUF_SLOTS];
  __shared__ __attribute__((aligned(16))) uint4 buf1[T::BUF_SLOTS];
  __shared__ __attribute__((aligned(16))) uint4 wbuf0[9 * NFW * 64];
  __shared__ __attribute__((aligned(16))) uint4 wbuf1[9 * NFW * 64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int nf = a.nf;
  const int q0 = blockIdx.y * NFW;

  // Items: workgroup bx runs on XCD bx % 8; XCD x owns tiles
  // [x * per, (x + 1) * per), taken round robin by its gridDim.x / 8
  // workgroups.  Item k is chunk k % nch of this workgroup's (k / nch)-th tile.
  const int ntiles = a.tiles_x * a.tiles_y;
  const int per = (ntiles + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds;
  const int first = blockIdx.x / kXcds;
  const int stride = gridDim.x / kXcds;
  const int nch = a.nchunks;
  auto item_valid = [&](int k) {
    const int local = first + (k / nch) * stride;
    return local < per && xcd * per + local < ntiles;
  };
  auto item_tile = [&](int k) { return xcd * per + first + (k / nch) * stride; };

  if (!item_valid(0)) return;

  auto issue = [&](int k, uint4* wdst, uint4* dst) {
    const ConvChunk ch = a.chunk[k % nch];
    const int t = item_tile(k);
    const int ty = t / a.tiles_x;
    const int tx = t - ty * a.tiles_x;
    load_weights<NFW>(wdst, static_cast<const uint4*>(a.wfrag) + ((size_t)ch.wfrag + q0) * 64, nf,
                      wave);
    load_patch<R>(dst, static_cast<const _Float16*>(ch.src ? a.src1 : a.src0),
                  ch.src ? a.cs1 : a.cs0, ch.coff, upcat && ch.src == 0, a.h, a.w, ty * T::TH,
                  tx * TW, wave, lane);
  };

  floatx4 acc[R][NFW];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int q = 0; q < NFW; ++q) acc[r][q] = floatx4{0.f, 0.f, 0.f, 0.f};

  issue(0, wbuf0, buf0);

  // One pipeline step: wait for item k's loads, start item k + 1's, compute k.
  auto step = [&](int k, const uint4* wcur, uint4* wnxt, const uint4* cur, uint4* nxt) -> bool {
    __syncthreads();
    const bool more = item_valid(k + 1);
    if (more) issue(k + 1, wnxt, nxt);
    mma_chunk<NFW, R>(acc, wcur, cur, wave, g, c, lane);
    if (k % nch == nch - 1) {
      const int t = item_tile(k);
      const int ty = t / a.tiles_x;
      epilogue<NFW, R, OUTF32>(acc, a, q0, ty * T::TH, (t - ty * a.tiles_x) * TW, wave, g, c,
                               pool, relu);
    }
    return more;
  };
#pragma unroll 1
  for (int k = 0;; k += 2) {
    if (!step(k, wbuf0, wbuf1, buf0, buf1)) break;
    if (!step(k + 1, wbuf1, wbuf0, buf1, buf0)) break;
  }
}

template <int NFW, int R>
hipError_t launch_shape(ConvF16Args a, int nsplit, bool upcat, bool pool, bool relu,
                        bool out_f32, hipStream_t stream) {
  a.tiles_x = cdiv(a.w, TW);
  a.tiles_y = cdiv(a.h, Tile<R>::TH);
  const int ntiles = a.tiles_x * a.tiles_y;
  // one resident workgroup per CU over all splits, at most one per tile
  int gx = cdiv(cdiv(kCUs, nsplit), kXcds) * kXcds;
  const int gmax = cdiv(ntiles, kXcds) * kXcds;
  if (gx > gmax) gx = gmax;
  const dim3 grid(gx, nsplit), block(THREADS);
  if (out_f32)
    hipLaunchKernelGGL((conv3x3_f16_mfma<NFW, R, true>), grid, block, 0, stream, a, (int)upcat,
                       (int)pool, (int)relu);
  else
    hipLaunchKernelGGL((conv3x3_f16_mfma<NFW, R, false>), grid, block, 0, stream, a, (int)upcat,
                       (int)pool, (int)relu);
  return hipGetLastError();
}

template <int NFW>
hipError_t launch_rows(const ConvF16Args& a, int rows, int nsplit, bool upcat, bool pool,
                       bool relu, bool out_f32, hipStream_t stream) {
  if constexpr (NFW <= 3) {
    if (rows == 8) return launch_shape<NFW, 8>(a, nsplit, upcat, pool, relu, out_f32, stream);
  }
  if (rows == 2) return launch_shape<NFW, 2>(a, nsplit, upcat, pool, relu, out_f32, stream);
  return launch_shape<NFW, 4>(a, nsplit, upcat, pool, relu, out_f32, stream);
}

}  // namespace

// Work decomposition: tile height 4 * rows and NFW (<= 4) of the nf output
// fragments per workgroup, nf / NFW workgroups sharing each tile.  Tiles as
// tall as possible while every CU still gets four or more items (32-row
// tiles only up to NFW = 3, whose two patch and weight buffers fit in LDS).
void conv_f16_plan(int h, int w, int nf, int* rows, int* nfw) {
  int width = nf;
  if (nf > 4) width = nf % 4 == 0 ? 4 : (nf % 3 == 0 ? 3 : (nf % 2 == 0 ? 2 : 1));
  const int split = nf / width;
  *nfw = width;
  for (int r : {8, 4}) {
    if (r == 8 && width > 3) continue;   // LDS: 2 x (49 KB patch + 9 NFW KB weights)
    const long items = (long)cdiv(w, TW) * cdiv(h, 4 * r) * split;
    if (items >= 4L * kCUs) {
      *rows = r;
      return;
    }
  }
  *rows = 2;
}

// Grid of the conv launch (for reporting).
int conv_f16_blocks(int h, int w, int nf) {
  int rows, nfw;
  conv_f16_plan(h, w, nf, &rows, &nfw);
  const int nsplit = nf / nfw;
  const int ntiles = cdiv(w, TW) * cdiv(h, 4 * rows);
  int gx = cdiv(cdiv(kCUs, nsplit), kXcds) * kXcds;
  const int gmax = cdiv(ntiles, kXcds) * kXcds;
  return (gx > gmax ? gmax : gx) * nsplit;
}

bool conv_f16_layout(int cin0_stored, int cin1_stored, int cout, ConvLayout* out) {
  ConvLayout L{};
  L.nf = cdiv(stored_channels(cout), 16);
  if (L.nf < 1 || L.nf > 8) return false;
  // Chunks of 32 channels per source, the last one zero-filled past the
  // source's stored channels; a chunk is 3 column groups x 3 ky x nf
  // fragments.
  int frag = 0, n = 0;
  const int cs[2] = {cin0_stored, cin1_stored};
  for (int s = 0; s < 2; ++s)
    for (int off = 0; off < cs[s]; off += kChunkChannels) {
      if (n >= kMaxChunks) return false;
      ConvChunk& ch = L.chunk[n++];
      ch.src = s;
      ch.coff = off;
      ch.cg = 4;
      ch.ncg = 3;
      ch.wfrag = frag;
      frag += ch.ncg * 3 * L.nf;
    }
  L.nchunks = n;
  L.nchunks4 = n;
  L.total_frags = frag;
  L.bias_bytes = align256(sizeof(float) * 16 * L.nf);
  L.bytes = L.bias_bytes + (size_t)frag * kFragBytes;
  *out = L;
  return true;
}

hipError_t launch_conv_f16(const ConvF16Args& a, int nf, bool upcat, bool pool, bool relu,
                           bool out_f32, hipStream_t stream) {
  int rows = 4, nfw = nf;
  conv_f16_plan(a.h, a.w, nf, &rows, &nfw);
  ConvF16Args b = a;
  b.nf = nf;
  const int nsplit = nf / nfw;
  switch (nfw) {
    case 1: return launch_rows<1>(b, rows, nsplit, upcat, pool, relu, out_f32, stream);
    case 2: return launch_rows<2>(b, rows, nsplit, upcat, pool, relu, out_f32, stream);
    case 3: return launch_rows<3>(b, rows, nsplit, upcat, pool, relu, out_f32, stream);
    case 4: return launch_rows<4>(b, rows, nsplit, upcat, pool, relu, out_f32, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oidn
