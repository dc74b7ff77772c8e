// fp32 3x3 convolution on the matrix cores (fp32 storage, v_mfma_f32_16x16x4
// with fp32 products and accumulation).
//
// The operation is [web-0.4] createConvShader ("oidn-web 0.3.4 -> 0.4.0",
// nativeUNet.ts): bias plus the sum over the nine taps and every stored
// input channel, taps outside the image reading zero; the decoder form reads
// the upsampled source at (y >> 1, x >> 1) (createFusedDecoderShader) and
// the pooled form keeps the max of the 2x2 window (createFusedConvPoolShader).
//
// Implicit GEMM: a workgroup of four waves covers a 16 x 16 output tile for
// up to four 16-channel output fragments (grid y walks the fragment groups).
// The input is taken 32 stored channels at a time (a chunk, over both
// sources): its 18 x 18 halo patch is staged in LDS once and every wave reads
// its B operands there; A operands (weights) come from global memory in the
// lane order of the MFMA, reused over the wave's four output rows.  Within a
// chunk, K step j of lane group g is channel 8 g + j, so one 16-byte LDS read
// gives a lane four consecutive K steps.
#include "internal.h"

namespace oidn {
namespace {

constexpr int THREADS = 256;
constexpr int TW = 16;                   // output tile width
constexpr int PW = TW + 2;               // patch width
constexpr int CCH = 32;                  // input channels per chunk
constexpr int PSTR = CCH + 4;            // floats per patch pixel (padded against bank conflicts)

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// One chunk's patch: pixel (py, px) of the PH x PW window at (y0 - 1,
// x0 - 1), the chunk's eight 4-channel blocks, zero outside the image and
// past the stored channels.
template <int PH>
__device__ __forceinline__ void stage_chunk(float* lds, const ConvF32Args& a, bool upcat, int k,
                                            int y0, int x0, int tid) {
  const int cst = a.cs0 + a.cs1;
  for (int u = tid; u < PH * PW * (CCH / 4); u += THREADS) {
    const int pp = u >> 3, b = u & 7;
    const int py = pp / PW, px = pp - py * PW;
    const int iy = y0 - 1 + py, ix = x0 - 1 + px;
    const int c = k * CCH + 4 * b;        // first stored channel of the block
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (iy >= 0 && iy < a.h && ix >= 0 && ix < a.w && c < cst) {
      if (c < a.cs0) {
        const size_t pix = upcat ? (size_t)(iy >> 1) * (a.w >> 1) + (ix >> 1) : (size_t)iy * a.w + ix;
        v = *reinterpret_cast<const float4*>(a.src0 + pix * a.cs0 + c);
      } else {
        v = *reinterpret_cast<const float4*>(a.src1 + ((size_t)iy * a.w + ix) * a.cs1 + (c - a.cs0));
      }
    }
    *reinterpret_cast<float4*>(lds + pp * PSTR + 4 * b) = v;
  }
}

// ROWS output rows per wave (tile height 4 ROWS), up to MAXF output
// fragments per workgroup.
template <int ROWS, int MAXF>
__global__ __launch_bounds__(THREADS) void conv3x3_f32_mfma(ConvF32Args a, int upcat, int pool,
                                                            int relu) {
  static_assert(ROWS % 2 == 0 || ROWS == 1, "pooled rows come in pairs");
  constexpr int TH = 4 * ROWS, PH = TH + 2;
  __shared__ __attribute__((aligned(16))) float lds[PH * PW * PSTR];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int tiles_x = (a.w + TW - 1) / TW;
  const int ty = blockIdx.x / tiles_x, tx = blockIdx.x - ty * tiles_x;
  const int y0 = ty * TH, x0 = tx * TW;
  const int nfrag = (a.cout_stored + 15) / 16;
  const int f0 = blockIdx.y * MAXF;
  const int nfh = min(MAXF, nfrag - f0);
  const int cst = a.cs0 + a.cs1;
  const int nck = (cst + CCH - 1) / CCH;

  floatx4 acc[ROWS][MAXF];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int q = 0; q < MAXF; ++q) acc[r][q] = floatx4{0.f, 0.f, 0.f, 0.f};

  // weights: [fragment][tap][chunk][lane][8]
  const float4* wl = reinterpret_cast<const float4*>(a.wt) + lane * 2;
#pragma unroll 1
  for (int k = 0; k < nck; ++k) {
    __syncthreads();
    stage_chunk<PH>(lds, a, upcat, k, y0, x0, tid);
    __syncthreads();
#pragma unroll 1
    for (int t = 0; t < 9; ++t) {
      const int ky = t / 3, kx = t - 3 * ky;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float4 bv[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
          bv[r] = *reinterpret_cast<const float4*>(
              lds + ((ROWS * wave + r + ky) * PW + c + kx) * PSTR + 8 * g + 4 * m);
        float4 av[MAXF];
#pragma unroll
        for (int q = 0; q < MAXF; ++q)
          av[q] = q < nfh ? wl[((size_t)((f0 + q) * 9 + t) * nck + k) * 128 + m]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < MAXF; ++q) {
          if (q >= nfh) continue;
#pragma unroll
          for (int r = 0; r < ROWS; ++r) {
            acc[r][q] = mfma4(av[q].x, bv[r].x, acc[r][q]);
            acc[r][q] = mfma4(av[q].y, bv[r].y, acc[r][q]);
            acc[r][q] = mfma4(av[q].z, bv[r].z, acc[r][q]);
            acc[r][q] = mfma4(av[q].w, bv[r].w, acc[r][q]);
          }
        }
      }
    }
  }

  // epilogue: lane (g, c) holds channels 4 g .. 4 g + 3 of each fragment for
  // pixel column x0 + c of the wave's rows
  const int x = x0 + c;
#pragma unroll
  for (int q = 0; q < MAXF; ++q) {
    if (q >= nfh) continue;
    const int ch = 16 * (f0 + q) + 4 * g;
    float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ch < a.cout_stored) b = *reinterpret_cast<const float4*>(a.bias + ch);
    if (!pool) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const int y = y0 + ROWS * wave + r;
        float4 v = make_float4(acc[r][q][0] + b.x, acc[r][q][1] + b.y, acc[r][q][2] + b.z,
                               acc[r][q][3] + b.w);
        if (relu) v = make_float4(fmaxf(v.x, 0.f), fmaxf(v.y, 0.f), fmaxf(v.z, 0.f), fmaxf(v.w, 0.f));
        if (y < a.h && x < a.w && ch < a.cout_stored)
          *reinterpret_cast<float4*>(a.y + ((size_t)y * a.w + x) * a.cout_stored + ch) = v;
      }
    } else {
      const int ow = a.w >> 1, oh = a.h >> 1;
#pragma unroll
      for (int rp = 0; rp < ROWS / 2; ++rp) {
        float m4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float bi = i == 0 ? b.x : i == 1 ? b.y : i == 2 ? b.z : b.w;
          float v0 = acc[2 * rp][q][i] + bi, v1 = acc[2 * rp + 1][q][i] + bi;
          if (relu) {
            v0 = fmaxf(v0, 0.f);
            v1 = fmaxf(v1, 0.f);
          }
          const float v = fmaxf(v0, v1);
          const float s = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
          m4[i] = fmaxf(v, s);
        }
        const int py = (y0 + ROWS * wave + 2 * rp) >> 1, px = x >> 1;
        if ((c & 1) == 0 && py < oh && px < ow && ch < a.cout_stored)
          *reinterpret_cast<float4*>(a.y + ((size_t)py * ow + px) * a.cout_stored + ch) =
              make_float4(m4[0], m4[1], m4[2], m4[3]);
      }
    }
  }
}

}  // namespace

int conv_f32_chunks(int cin_stored_total) { return cdiv(cin_stored_total, CCH); }

size_t conv_f32_bytes(int cin_stored_total, int cout) {
  const int cs = stored_channels(cout);
  return align256(sizeof(float) * cs) +
         sizeof(float) * (size_t)cdiv(cs, 16) * 9 * conv_f32_chunks(cin_stored_total) * 64 * 8;
}

size_t conv_f32_weight_index(int o, int tap, int c, int cin_stored_total) {
  const int k = c / CCH, cc = c - k * CCH;
  const int lane = (cc / 8) * 16 + (o & 15), j = cc & 7;
  return ((((size_t)(o / 16) * 9 + tap) * conv_f32_chunks(cin_stored_total) + k) * 64 + lane) * 8 + j;
}

// Two shapes: 16 x 16 tiles with four fragments per workgroup (operands
// reused over four rows and four fragments), or, where that gives fewer
// workgroups than kSmallBelow, 8 x 16 tiles with one fragment each.
constexpr int kSmallBelow = 512;

bool conv_f32_small(int h, int w, int cout) {
  return (long)cdiv(w, TW) * cdiv(h, 16) * cdiv(cdiv(stored_channels(cout), 16), 4) < kSmallBelow;
}

int conv_f32_blocks(int h, int w, int cout) {
  const int nfrag = cdiv(stored_channels(cout), 16);
  return conv_f32_small(h, w, cout) ? cdiv(w, TW) * cdiv(h, 8) * nfrag
                                    : cdiv(w, TW) * cdiv(h, 16) * cdiv(nfrag, 4);
}

const char* conv_f32_kernel_name(int h, int w, int cout) {
  return conv_f32_small(h, w, cout) ? "conv3x3_f32_mfma<2, 1>" : "conv3x3_f32_mfma<4, 4>";
}

hipError_t launch_conv_f32(const ConvF32Args& a, bool upcat, bool pool, bool relu,
                           hipStream_t stream) {
  if (a.h <= 0 || a.w <= 0) return hipSuccess;
  const int nfrag = cdiv(a.cout_stored, 16);
  if (conv_f32_small(a.h, a.w, a.cout_stored)) {
    const dim3 grid(cdiv(a.w, TW) * cdiv(a.h, 8), nfrag);
    hipLaunchKernelGGL((conv3x3_f32_mfma<2, 1>), grid, dim3(THREADS), 0, stream, a, (int)upcat,
                       (int)pool, (int)relu);
  } else {
    const dim3 grid(cdiv(a.w, TW) * cdiv(a.h, 16), cdiv(nfrag, 4));
    hipLaunchKernelGGL((conv3x3_f32_mfma<4, 4>), grid, dim3(THREADS), 0, stream, a, (int)upcat,
                       (int)pool, (int)relu);
  }
  return hipGetLastError();
}

}  // namespace oidn
