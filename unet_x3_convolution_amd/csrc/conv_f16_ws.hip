// Weight-stationary variant of the fp16 MFMA implicit-GEMM 3x3 conv (gfx950,
// v_mfma_f32_16x16x32_f16) for the large, shallow layers of the network.
//
// Same arithmetic, fragment layout, K order and epilogue as conv_f16.hip
// (see there; [web-0.4] createConvShader / createTiledDecoderShader /
// createFusedConvPoolShader, "oidn-web 0.3.4 -> 0.4.0", nativeUNet.ts), but
// organised so that no global load sits inside the matrix work:
//
//  * Workgroups are persistent (one per CU).  Every wave loads the layer's
//    whole weight set for its NFW output fragments into registers once
//    (e.g. 48 fragments = 192 VGPRs for half the outputs of a 64 + 16 -> 64
//    decoder conv).
//  * Only the halo patches stream: a tile's patches for all input chunks are
//    loaded global -> LDS directly (global_load_lds, no registers) into one of
//    two buffer sets while the previous tile computes from the other.  One
//    barrier per tile is the only wait; a tile's MFMA work (several
//    microseconds) covers the load latency.  The two buffer sets are distinct
//    arrays used at compile-time positions (the tile loop is unrolled by two)
//    so the compiler never makes reads of one wait for loads into the other.
//  * The chunk structure (N4 chunks of 32 channels, then N2 chunks of 16) is
//    a template parameter, so the weight registers are indexed statically.
//
// The per-pixel reduction order is the same as conv_f16.hip's (chunks in
// layout order, then column group, then ky), independent of position.
#include "internal.h"

namespace oidn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int TW = 16;
constexpr int PW = TW + 2;
constexpr int SLOT_HALVES = 8;
constexpr int PIX_SLOTS = 5;           // 4 channel groups + 1 pad: 80-byte pixel stride
constexpr int PIX_HALVES = PIX_SLOTS * SLOT_HALVES;
constexpr int THREADS = 256;
constexpr int kXcds = 8;
constexpr int kCUs = 256;
constexpr int kLdsBytes = 160 * 1024;
constexpr int kWeightRegBudget = 400;  // weight + accumulator registers per lane (no spills)

// Zero block that padding lanes of the patch loads read from.
__device__ __attribute__((aligned(16))) unsigned int g_ws_zero16[4] = {0u, 0u, 0u, 0u};

template <int R>
struct Tile {
  static constexpr int TH = 4 * R;
  static constexpr int PH = TH + 2;
  static constexpr int PIX = PH * PW;
  static constexpr int SLOTS = PIX * PIX_SLOTS;
  static constexpr int LOADS16 = (SLOTS + 63) / 64;
  static constexpr int LOADS4 = (SLOTS * 4 + 63) / 64;
  static constexpr int BUF_SLOTS = LOADS16 * 64;
};

constexpr int buf_slots(int r) { return ((((4 * r + 2) * PW * PIX_SLOTS) + 63) / 64) * 64; }

__device__ __forceinline__ half8 as_half8(uint4 v) { return __builtin_bit_cast(half8, v); }

// Global -> LDS loads of one chunk's halo patch (slot s of `buf` is pixel
// s / 5, channel group s % 5, group 4 = pad).  16 bytes per lane when the
// source's stored channel count is a multiple of 8, else 4 bytes per lane.
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
      const void* gp = g_ws_zero16;
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
      const int d = k * 64 + lane;
      const int s = d >> 2;
      const int p = s / PIX_SLOTS;
      const int u = s - p * PIX_SLOTS;
      const void* gp = g_ws_zero16;
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

// MFMAs of one chunk (CG = 4 or 2 groups of 8 channels) for one wave's R rows,
// weights w[j][ky][q] of its column groups j.
template <int NFW, int R, int CG, int NCGC>
__device__ __forceinline__ void mma_chunk(floatx4 (&acc)[R][NFW], const uint4 (*w)[3][NFW],
                                          const uint4* buf, const uint4* zero, int wave, int g,
                                          int c) {
  const _Float16* patch = reinterpret_cast<const _Float16*>(buf);
#pragma unroll
  for (int j = 0; j < NCGC; ++j) {
    const int slot = 4 * j + g;
    const _Float16* bp = reinterpret_cast<const _Float16*>(zero);
    int rstride = 0;
    if (slot < 3 * CG) {
      const int kx = slot / CG;
      const int grp = slot - kx * CG;
      bp = patch + ((R * wave) * PW + c + kx) * PIX_HALVES + SLOT_HALVES * grp;
      rstride = PW * PIX_HALVES;
    }
#pragma unroll
    for (int p = 0; p < R + 2; ++p) {
      const half8 b = *reinterpret_cast<const half8*>(bp + p * rstride);
#pragma unroll
      for (int ky = 0; ky < 3; ++ky) {
        const int r = p - ky;
        if (r >= 0 && r < R) {
#pragma unroll
          for (int q = 0; q < NFW; ++q)
            acc[r][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(w[j][ky][q]), b, acc[r][q],
                                                               0, 0, 0);
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
__device__ __forceinline__ void epilogue(floatx4 (&acc)[R][NFW], const float (&bv)[NFW][4],
                                         const ConvF16Args& a, int cbase, int y0, int x0, int wave,
                                         int c, int pool, int relu) {
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

template <int NFW, int R, int N4, int N2, bool OUTF32>
__global__ __launch_bounds__(THREADS, 1) void conv3x3_f16_ws(ConvF16Args a, int upcat, int pool,
                                                              int relu) {
  using T = Tile<R>;
  constexpr int NCH = N4 + N2;
  constexpr int NCG = 3 * N4 + 2 * N2;
  __shared__ __attribute__((aligned(16))) uint4 bufA[NCH * T::BUF_SLOTS];
  __shared__ __attribute__((aligned(16))) uint4 bufB[NCH * T::BUF_SLOTS];
  __shared__ __attribute__((aligned(16))) uint4 zero[1];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int nf = a.nf;
  const int q0 = blockIdx.y * NFW;

  // Tiles of this workgroup: XCD x = blockIdx.x % 8 owns tiles
  // [x * per, (x + 1) * per), taken round robin by its gridDim.x / 8 groups.
  const int ntiles = a.tiles_x * a.tiles_y;
  const int per = (ntiles + kXcds - 1) / kXcds;
  const int xcd = blockIdx.x % kXcds;
  const int first = blockIdx.x / kXcds;
  const int stride = gridDim.x / kXcds;
  auto tile_valid = [&](int m) {
    const int local = first + m * stride;
    return local < per && xcd * per + local < ntiles;
  };
  if (!tile_valid(0)) return;

  // Weights of all chunks, this block's fragments, into registers.
  uint4 w[NCG][3][NFW];
  {
    const uint4* wf = static_cast<const uint4*>(a.wfrag) + lane + q0 * 64;
#pragma unroll
    for (int ci = 0; ci < NCH; ++ci) {
      constexpr int dummy = 0;
      (void)dummy;
      const int ncg = ci < N4 ? 3 : 2;
      const int cg0 = ci < N4 ? 3 * ci : 3 * N4 + 2 * (ci - N4);
      const uint4* wc = wf + (size_t)a.chunk[ci].wfrag * 64;
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < ncg)
#pragma unroll
          for (int ky = 0; ky < 3; ++ky)
#pragma unroll
            for (int q = 0; q < NFW; ++q) w[cg0 + j][ky][q] = wc[((3 * j + ky) * nf + q) * 64];
    }
  }
  const int cbase = 4 * nf * g + 4 * q0;
  float bv[NFW][4];
#pragma unroll
  for (int q = 0; q < NFW; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) bv[q][i] = a.bias[cbase + 4 * q + i];
  if (tid == 0) zero[0] = make_uint4(0u, 0u, 0u, 0u);

  auto issue = [&](int m, uint4* dst) {
    const int t = xcd * per + first + m * stride;
    const int ty = t / a.tiles_x;
    const int tx = t - ty * a.tiles_x;
#pragma unroll
    for (int ci = 0; ci < NCH; ++ci) {
      const ConvChunk ch = a.chunk[ci];
      load_patch<R>(dst + ci * T::BUF_SLOTS, static_cast<const _Float16*>(ch.src ? a.src1 : a.src0),
                    ch.src ? a.cs1 : a.cs0, ch.coff, upcat && ch.src == 0, a.h, a.w, ty * T::TH,
                    tx * TW, wave, lane);
    }
  };

  floatx4 acc[R][NFW];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int q = 0; q < NFW; ++q) acc[r][q] = floatx4{0.f, 0.f, 0.f, 0.f};

  issue(0, bufA);
  auto step = [&](int m, const uint4* cur, uint4* nxt) -> bool {
    __syncthreads();
    const bool more = tile_valid(m + 1);
    if (more) issue(m + 1, nxt);
#pragma unroll
    for (int ci = 0; ci < NCH; ++ci) {
      if (ci < N4)
        mma_chunk<NFW, R, 4, 3>(acc, &w[3 * ci], cur + ci * T::BUF_SLOTS, zero, wave, g, c);
      else
        mma_chunk<NFW, R, 2, 2>(acc, &w[3 * N4 + 2 * (ci - N4)], cur + ci * T::BUF_SLOTS, zero,
                                wave, g, c);
    }
    const int t = xcd * per + first + m * stride;
    const int ty = t / a.tiles_x;
    epilogue<NFW, R, OUTF32>(acc, bv, a, cbase, ty * T::TH, (t - ty * a.tiles_x) * TW, wave, c,
                             pool, relu);
    return more;
  };
#pragma unroll 1
  for (int m = 0;; m += 2) {
    if (!step(m, bufA, bufB)) break;
    if (!step(m + 1, bufB, bufA)) break;
  }
}

template <int NFW, int R, int N4, int N2, bool OUTF32>
hipError_t launch(ConvF16Args a, int nsplit, bool upcat, bool pool, bool relu,
                  hipStream_t stream) {
  static_assert(2 * (N4 + N2) * Tile<R>::BUF_SLOTS * 16 + 16 <= kLdsBytes, "LDS");
  a.tiles_x = cdiv(a.w, TW);
  a.tiles_y = cdiv(a.h, Tile<R>::TH);
  const int ntiles = a.tiles_x * a.tiles_y;
  int gx = cdiv(cdiv(kCUs, nsplit), kXcds) * kXcds;
  const int gmax = cdiv(ntiles, kXcds) * kXcds;
  if (gx > gmax) gx = gmax;
  hipLaunchKernelGGL((conv3x3_f16_ws<NFW, R, N4, N2, OUTF32>), dim3(gx, nsplit), dim3(THREADS),
                     0, stream, a, (int)upcat, (int)pool, (int)relu);
  return hipGetLastError();
}

}  // namespace

// Picks NFW (output fragments per workgroup) and R (tile height 4 R) for the
// weight-stationary kernel, or returns false if no instantiated shape fits:
// weights + accumulators within the register budget, two patch sets within
// LDS, and at least four tiles (times output splits) per CU.
bool conv_f16_ws_plan(int h, int w, int nf, int n4, int n2, bool out_f32, int* rows, int* nfw) {
  const int ncg = 3 * n4 + 2 * n2, nch = n4 + n2;
  for (int width = nf < 4 ? nf : 4; width >= 1; --width) {
    if (nf % width) continue;
    for (int r : {8, 4, 2}) {
      const int regs = ncg * 3 * width * 4 + 4 * r * width;
      const int lds = 2 * nch * buf_slots(r) * 16 + 16;
      const long items = (long)cdiv(w, TW) * cdiv(h, 4 * r) * (nf / width);
      if (regs > kWeightRegBudget || lds > kLdsBytes || items < 4L * kCUs) continue;
      // instantiated shapes (the network's large layers)
      const bool have =
          (!out_f32 && ((width == 2 && r == 8 && n4 == 0 && n2 == 1) ||
                        (width == 2 && r == 8 && n4 == 1 && n2 == 0) ||
                        (width == 3 && r == 4 && n4 == 1 && n2 == 0) ||
                        (width == 2 && r == 2 && n4 == 4 && n2 == 0) ||
                        (width == 4 && r == 4 && n4 == 2 && n2 == 0) ||
                        (width == 2 && r == 4 && n4 == 2 && n2 == 1) ||
                        (width == 2 && r == 4 && n4 == 2 && n2 == 0))) ||
          (out_f32 && width == 1 && r == 8 && n4 == 1 && n2 == 0);
      if (!have) continue;
      *rows = r;
      *nfw = width;
      return true;
    }
  }
  return false;
}

int conv_f16_ws_blocks(int h, int w, int nf, int rows, int nfw) {
  const int ntiles = cdiv(w, TW) * cdiv(h, 4 * rows);
  const int nsplit = nf / nfw;
  int gx = cdiv(cdiv(kCUs, nsplit), kXcds) * kXcds;
  const int gmax = cdiv(ntiles, kXcds) * kXcds;
  return (gx > gmax ? gmax : gx) * nsplit;
}

hipError_t launch_conv_f16_ws(const ConvF16Args& a, int rows, int nfw, int n4, int n2, bool upcat,
                              bool pool, bool relu, bool out_f32, hipStream_t stream) {
  const int nsplit = a.nf / nfw;
#define OIDN_WS(W, R, A, B, F)                                                   \
  if (nfw == W && rows == R && n4 == A && n2 == B && out_f32 == F)               \
    return launch<W, R, A, B, F>(a, nsplit, upcat, pool, relu, stream);
  OIDN_WS(2, 8, 0, 1, false)
  OIDN_WS(2, 8, 1, 0, false)
  OIDN_WS(3, 4, 1, 0, false)
  OIDN_WS(2, 2, 4, 0, false)
  OIDN_WS(4, 4, 2, 0, false)
  OIDN_WS(2, 4, 2, 1, false)
  OIDN_WS(2, 4, 2, 0, false)
  OIDN_WS(1, 8, 1, 0, true)
#undef OIDN_WS
  return hipErrorInvalidValue;
}

}  // namespace oidn
