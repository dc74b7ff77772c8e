// 3x3 convolution as an fp16 MFMA implicit GEMM with fp32 accumulation
// (gfx950, v_mfma_f32_16x16x32_f16).
//
// What it computes is [web-0.4] createConvShader / createTiledConvShader /
// createTiledDecoderShader / createFusedConvPoolShader ("oidn-web 0.3.4 ->
// 0.4.0", nativeUNet.ts): y = act(b + sum over taps and input channels of
// W * x) with zero padding, optionally over [nearest-2x-upsampled source,
// skip] and optionally followed by a 2x2 max-pool.  The tiling is our own:
//
//  * GEMM roles: D[cout][pixel] = A[cout][k] * B[k][pixel].  A holds packed
//    weights, B is read straight from an LDS halo patch (no im2col), so each
//    lane of the 16x16 accumulator owns 4 consecutive output channels of one
//    pixel (a whole 4-lane channel block, stored with one 8-byte write).
//  * K is (input chunk of <= 32 channels) x (tap) x (8-channel group).  One
//    MFMA step eats four (tap, group) pairs, one per 16-lane group, so thin
//    inputs (12 channels) fold several taps into one instruction instead of
//    zero-padding channels to 32.
//  * A workgroup of 4 waves computes a 16 x 16 pixel tile for all output
//    channels; wave w owns rows 4w..4w+3 (one 16-pixel B fragment per row).
//    Per chunk, the (16 + 2) x (16 + 2) halo patch is staged in LDS once
//    (80-byte pixel stride: conflict-free 16-byte fragment reads); the
//    decoder's upsampled source is gathered at (y >> 1, x >> 1) while staging.
//  * Epilogue: bias, ReLU, then either the store or the fused 2x2 pool: the
//    vertical pair sits in two rows held by the same lane, the horizontal pair
//    in neighbouring lanes (one DPP swap).  Max is taken in fp32 before the
//    single fp16 rounding; RNE is monotone, so this equals pooling the rounded
//    conv output.
#include "internal.h"

namespace oidn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int TH = 16, TW = 16;               // output tile
constexpr int PH = TH + 2, PW = TW + 2;       // halo patch
constexpr int PSTR = 40;                      // halves per patch pixel (32 + 8 pad)
constexpr int PATCH_HALVES = PH * PW * PSTR;
constexpr int ZERO_OFF = PATCH_HALVES;        // 8 zero halves: B operand of padding K slots
constexpr int THREADS = 256;

__device__ __forceinline__ half8 as_half8(uint4 v) {
  return __builtin_bit_cast(half8, v);
}

// Stage the chunk's halo patch: CG groups of 8 channels per pixel, moved in
// 4-channel (8-byte) units; channels past the source's stored count and
// pixels outside the image are zero.
template <int CG>
__device__ __forceinline__ void stage_patch(_Float16* lds, const _Float16* src, int cs, int coff,
                                            bool up, int h, int w, int y0, int x0, int tid) {
  constexpr int UNITS = 2 * CG;
  constexpr int TOTAL = PH * PW * UNITS;
  const int sw = up ? (w >> 1) : w;
  for (int u = tid; u < TOTAL; u += THREADS) {
    const int pp = u / UNITS;
    const int q4 = u - pp * UNITS;
    const int py = pp / PW;
    const int px = pp - py * PW;
    const int iy = y0 - 1 + py;
    const int ix = x0 - 1 + px;
    const int c4 = coff + 4 * q4;
    uint2 v = make_uint2(0u, 0u);
    if (iy >= 0 && iy < h && ix >= 0 && ix < w && c4 < cs) {
      const int sy = up ? (iy >> 1) : iy;
      const int sx = up ? (ix >> 1) : ix;
      v = *reinterpret_cast<const uint2*>(src + ((size_t)sy * sw + sx) * cs + c4);
    }
    *reinterpret_cast<uint2*>(lds + pp * PSTR + 4 * q4) = v;
  }
}

template <int NF, int CG>
__device__ __forceinline__ void mma_chunk(floatx4 (&acc)[4][NF], const _Float16* lds,
                                          const uint4* wchunk, int wave, int g, int c) {
  constexpr int STEPS = (9 * CG + 3) / 4;
  uint4 afr[NF];
#pragma unroll
  for (int q = 0; q < NF; ++q) afr[q] = wchunk[q * 64];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    uint4 anext[NF];
    if (s + 1 < STEPS) {
#pragma unroll
      for (int q = 0; q < NF; ++q) anext[q] = wchunk[((s + 1) * NF + q) * 64];
    }
    const int kg = 4 * s + g;
    int boff = ZERO_OFF, rstride = 0;
    if (kg < 9 * CG) {
      const int tap = kg / CG;
      const int grp = kg - tap * CG;
      const int ky = tap / 3;
      const int kx = tap - 3 * ky;
      boff = ((4 * wave + ky) * PW + c + kx) * PSTR + 8 * grp;
      rstride = PW * PSTR;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const half8 b = *reinterpret_cast<const half8*>(lds + boff + r * rstride);
#pragma unroll
      for (int q = 0; q < NF; ++q)
        acc[r][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(afr[q]), b, acc[r][q], 0, 0, 0);
    }
    if (s + 1 < STEPS) {
#pragma unroll
      for (int q = 0; q < NF; ++q) afr[q] = anext[q];
    }
  }
}

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

template <int NF, bool OUTF32>
__global__ __launch_bounds__(THREADS) void conv3x3_f16_mfma(ConvF16Args a, int upcat, int pool,
                                                             int relu) {
  __shared__ __attribute__((aligned(16))) _Float16 lds[PATCH_HALVES + 8];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int tile = blockIdx.x;
  const int ty = tile / a.tiles_x;
  const int tx = tile - ty * a.tiles_x;
  const int y0 = ty * TH, x0 = tx * TW;

  if (tid < 2) reinterpret_cast<uint2*>(lds + ZERO_OFF)[tid] = make_uint2(0u, 0u);

  floatx4 acc[4][NF];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < NF; ++q) acc[r][q] = floatx4{0.f, 0.f, 0.f, 0.f};

  const uint4* wf = static_cast<const uint4*>(a.wfrag);
  for (int ci = 0; ci < a.nchunks; ++ci) {
    const ConvChunk ch = a.chunk[ci];
    const _Float16* src = static_cast<const _Float16*>(ch.src ? a.src1 : a.src0);
    const int cs = ch.src ? a.cs1 : a.cs0;
    const bool up = upcat && ch.src == 0;
    __syncthreads();
    switch (ch.cg) {
      case 1: stage_patch<1>(lds, src, cs, ch.coff, up, a.h, a.w, y0, x0, tid); break;
      case 2: stage_patch<2>(lds, src, cs, ch.coff, up, a.h, a.w, y0, x0, tid); break;
      case 3: stage_patch<3>(lds, src, cs, ch.coff, up, a.h, a.w, y0, x0, tid); break;
      default: stage_patch<4>(lds, src, cs, ch.coff, up, a.h, a.w, y0, x0, tid); break;
    }
    __syncthreads();
    const uint4* wchunk = wf + (size_t)ch.wfrag * 64 + lane;
    switch (ch.cg) {
      case 1: mma_chunk<NF, 1>(acc, lds, wchunk, wave, g, c); break;
      case 2: mma_chunk<NF, 2>(acc, lds, wchunk, wave, g, c); break;
      case 3: mma_chunk<NF, 3>(acc, lds, wchunk, wave, g, c); break;
      default: mma_chunk<NF, 4>(acc, lds, wchunk, wave, g, c); break;
    }
  }

  // Epilogue.  Lane (g, c) holds rows 4g..4g+3 of every fragment: output
  // channels cbase + 4q + i with cbase = 4 * NF * g, for pixel column c.
  const int cbase = 4 * NF * g;
  float bv[NF][4];
#pragma unroll
  for (int q = 0; q < NF; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) bv[q][i] = a.bias[cbase + 4 * q + i];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int q = 0; q < NF; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[r][q][i] + bv[q][i];
        acc[r][q][i] = relu ? fmaxf(v, 0.f) : v;
      }

  const int x = x0 + c;
  if (!pool) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int yy = y0 + 4 * wave + r;
      if (yy < a.h && x < a.w) {
        const size_t base = ((size_t)yy * a.w + x) * a.cout_stored + cbase;
#pragma unroll
        for (int q = 0; q < NF; ++q)
          if (cbase + 4 * q < a.cout_stored)
            store4<OUTF32>(a.y, base + 4 * q, acc[r][q][0], acc[r][q][1], acc[r][q][2],
                           acc[r][q][3]);
      }
    }
  } else {
    const int ow = a.w >> 1;
#pragma unroll
    for (int rp = 0; rp < 2; ++rp) {
      float m[NF][4];
#pragma unroll
      for (int q = 0; q < NF; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = fmaxf(acc[2 * rp][q][i], acc[2 * rp + 1][q][i]);
          m[q][i] = fmaxf(v, swap_pair(v));
        }
      const int yy = y0 + 4 * wave + 2 * rp;
      if ((c & 1) == 0 && yy < a.h && x < a.w) {
        const size_t base = ((size_t)(yy >> 1) * ow + (x >> 1)) * a.cout_stored + cbase;
#pragma unroll
        for (int q = 0; q < NF; ++q)
          if (cbase + 4 * q < a.cout_stored)
            store4<OUTF32>(a.y, base + 4 * q, m[q][0], m[q][1], m[q][2], m[q][3]);
      }
    }
  }
}

template <int NF>
hipError_t launch_nf(const ConvF16Args& a, bool upcat, bool pool, bool relu, bool out_f32,
                     hipStream_t stream) {
  const dim3 grid(a.tiles_x * a.tiles_y), block(THREADS);
  if (out_f32)
    hipLaunchKernelGGL((conv3x3_f16_mfma<NF, true>), grid, block, 0, stream, a, (int)upcat,
                       (int)pool, (int)relu);
  else
    hipLaunchKernelGGL((conv3x3_f16_mfma<NF, false>), grid, block, 0, stream, a, (int)upcat,
                       (int)pool, (int)relu);
  return hipGetLastError();
}

}  // namespace

bool conv_f16_layout(int cin0_stored, int cin1_stored, int cout, ConvLayout* out) {
  ConvLayout L{};
  L.nf = cdiv(stored_channels(cout), 16);
  if (L.nf < 1 || L.nf > 8) return false;
  int frag = 0, steps_total = 0, n = 0;
  const int cs[2] = {cin0_stored, cin1_stored};
  for (int s = 0; s < 2; ++s) {
    for (int off = 0; off < cs[s]; off += kChunkChannels) {
      if (n >= kMaxChunks) return false;
      ConvChunk& ch = L.chunk[n++];
      ch.src = s;
      ch.coff = off;
      const int rem = cs[s] - off < kChunkChannels ? cs[s] - off : kChunkChannels;
      ch.cg = cdiv(rem, 8);
      ch.steps = cdiv(9 * ch.cg, 4);
      ch.wfrag = frag;
      frag += ch.steps * L.nf;
      steps_total += ch.steps;
    }
  }
  L.nchunks = n;
  L.total_steps = steps_total;
  L.bias_bytes = align256(sizeof(float) * 16 * L.nf);
  L.bytes = L.bias_bytes + (size_t)frag * kFragBytes;
  *out = L;
  return true;
}

hipError_t launch_conv_f16(const ConvF16Args& a, int nf, bool upcat, bool pool, bool relu,
                           bool out_f32, hipStream_t stream) {
  switch (nf) {
    case 1: return launch_nf<1>(a, upcat, pool, relu, out_f32, stream);
    case 2: return launch_nf<2>(a, upcat, pool, relu, out_f32, stream);
    case 3: return launch_nf<3>(a, upcat, pool, relu, out_f32, stream);
    case 4: return launch_nf<4>(a, upcat, pool, relu, out_f32, stream);
    case 5: return launch_nf<5>(a, upcat, pool, relu, out_f32, stream);
    case 6: return launch_nf<6>(a, upcat, pool, relu, out_f32, stream);
    case 7: return launch_nf<7>(a, upcat, pool, relu, out_f32, stream);
    case 8: return launch_nf<8>(a, upcat, pool, relu, out_f32, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oidn
