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
//    weights (read from global memory, L2/L1 resident), B is read straight
//    from an LDS halo patch (no im2col), so each lane of a 16x16 accumulator
//    owns 4 consecutive output channels of one pixel -- a whole 4-lane channel
//    block, stored with one 8-byte write.
//  * A workgroup of 4 waves computes a (4 R) x 16 pixel tile for all output
//    channels; wave w owns R consecutive rows, one 16-pixel B fragment each.
//  * K order: chunk (<= 32 channels of one source, staged in LDS once) ->
//    column group (four (kx, 8-channel group) slots, one per 16-lane group)
//    -> ky.  All lanes of a column group read the same patch row, so the B
//    fragment of patch row p serves output rows p, p - 1 and p - 2 with the
//    weights of ky = 0, 1, 2: R + 2 fragment loads per column group instead
//    of 3 R.  Thin inputs (12 channels) put two kx columns in one MFMA
//    instead of padding channels to 32.
//  * The decoder's upsampled source is gathered at (y >> 1, x >> 1) while
//    staging; the skip follows as further chunks (concat order [up, skip]).
//  * Epilogue: bias, ReLU, then the store or the fused 2x2 pool: the vertical
//    pair sits in two rows held by the same lane, the horizontal pair in
//    neighbouring lanes (one DPP swap).  Max is taken in fp32 before the
//    single fp16 rounding; RNE is monotone, so this equals pooling the
//    rounded conv output.
//  * Tiles are dealt to blocks in 8 x 8-tile super-tiles, each of the 8 XCDs
//    taking a contiguous range of them (halos shared through its own L2).
//
// The per-pixel reduction order depends only on the channel layout, never on
// the pixel position or the image size, so tiled and untiled runs agree bit
// for bit wherever their inputs agree.
#include <atomic>
#include <cstdio>
#include <type_traits>

#include "internal.h"
#include "image_io.h"
#include "mfma_common.h"

namespace oidn {
namespace {

// Stage one chunk's halo patch.  Full resolution: (TH + 2) x 18 pixels at
// (y0 - 1, x0 - 1).  UP (the decoder's upsampled source): the same window
// at half resolution, (TH / 2 + 2) x 10 low-resolution pixels at
// (y0 / 2 - 1, x0 / 2 - 1) -- nearest upsampling repeats each of them 2 x 2
// times, so staging them once cuts the staged bytes about four-fold.
// VEC16: channels move in 8-channel (16 B) units, else in 4-channel (8 B)
// units.  Channels past the source's stored count and pixels outside the
// image are zero.
// Direct global -> LDS staging of the same patch for sources whose stored
// channel count is a multiple of 8: wave load k fills LDS slots
// [64 k, 64 k + 64); slot s is patch pixel s / SPP, position s % SPP
// (padded layout: channel group s % SPP, the last slot of a pixel is the
// pad, which no lane loads; swizzled: the group gslot maps to it).  Every load of
// the chunk is issued back to back (nothing waits on registers); the barrier
// that follows drains them.  Slots with no data (channel groups past the
// source, pixels outside the image) load the zero block.
// TH: tile height; NW: waves sharing the work; CAP: buffer capacity in slots.
template <int TH, int NW, int CAP, int CG, bool UP, bool SW = false, bool ASM = false>
__device__ __forceinline__ void stage_patch_direct(uint4* slots, const _Float16* src, int cs,
                                                   int coff, int h, int w, int y0, int x0,
                                                   int wave, int lane) {
  constexpr int PH = UP ? TH / 2 + 2 : TH + 2;
  constexpr int PWD = UP ? LPW : PW;
  constexpr int NPIX = PH * PWD;
  constexpr int SPP = pstride<CG, SW>() / 8;    // 16-byte slots per pixel
  constexpr int NLOAD = (NPIX * SPP + 63) / 64;
  static_assert(NLOAD * 64 <= CAP, "patch buffer");
  const int sh = UP ? (h >> 1) : h, sw = UP ? (w >> 1) : w;
  const int oy = UP ? (y0 >> 1) - 1 : y0 - 1, ox = UP ? (x0 >> 1) - 1 : x0 - 1;
#pragma unroll
  for (int i = 0; i < (NLOAD + NW - 1) / NW; ++i) {
    const int k = wave + NW * i;
    if (k >= NLOAD) break;
    const int sl = k * 64 + lane;
    const int pp = sl / SPP;
    const int u = sl - pp * SPP;
    if (u < CG && pp < NPIX) {   // pad slots are never read: those lanes stay idle
      const int py = pp / PWD;
      const int px = pp - py * PWD;
      const int iy = oy + py;
      const int ix = ox + px;
      const int c = coff + 8 * gslot<CG, SW>(px, u);   // gslot is its own inverse
      const void* gp = g_zero16;
      if (iy >= 0 && iy < sh && ix >= 0 && ix < sw && c < cs)
        gp = src + ((size_t)iy * sw + ix) * cs + c;
      dma16<ASM>(gp, slots + k * 64);
    }
  }
}

template <int TH, int CG, bool VEC16, bool UP, bool SW = false>
__device__ __forceinline__ void stage_patch(_Float16* lds, const _Float16* src, int cs, int coff,
                                            int h, int w, int y0, int x0, int tid) {
  constexpr int PH = UP ? Tile<TH>::LPH : Tile<TH>::PH;
  constexpr int PWD = UP ? LPW : PW;
  constexpr int UNITS = VEC16 ? CG : 2 * CG;
  constexpr int UCH = VEC16 ? 8 : 4;
  constexpr int TOTAL = PH * PWD * UNITS;
  const int sh = UP ? (h >> 1) : h, sw = UP ? (w >> 1) : w;
  const int oy = UP ? (y0 >> 1) - 1 : y0 - 1, ox = UP ? (x0 >> 1) - 1 : x0 - 1;
#pragma unroll 4
  for (int u = tid; u < TOTAL; u += THREADS) {
    const int pp = u / UNITS;
    const int q = u - pp * UNITS;
    const int py = pp / PWD;
    const int px = pp - py * PWD;
    const int iy = oy + py;
    const int ix = ox + px;
    const int c = coff + UCH * q;
    const bool inside = iy >= 0 && iy < sh && ix >= 0 && ix < sw && c < cs;
    const _Float16* p = src + ((size_t)iy * sw + ix) * cs + c;
    if constexpr (VEC16) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (inside) v = *reinterpret_cast<const uint4*>(p);
      *reinterpret_cast<uint4*>(lds + pp * pstride<CG, SW>() + 8 * gslot<CG, SW>(px, q)) = v;
    } else {
      uint2 v = make_uint2(0u, 0u);
      if (inside) v = *reinterpret_cast<const uint2*>(p);
      *reinterpret_cast<uint2*>(lds + pp * pstride<CG, SW>() + 8 * gslot<CG, SW>(px, q >> 1) +
                                4 * (q & 1)) = v;
    }
  }
}

// MFMAs of one chunk for one wave: rows [R * rg, R * rg + R) of the tile
// (row group rg), NFW output fragments.  The chunk's patch starts `cur`
// halves into `lds`; `zero` is the offset of 8 zero halves.  With PF,
// `acur` holds the chunk's column-group-0 weights on entry; each column
// group loads the next one's weights (or those of the next chunk, `wnext`)
// before its MFMAs, so weight loads overlap the matrix work, and on return
// `acur` holds the next chunk's.  `hook` runs once, right after the first
// of those prefetches is issued.
// The wave's window starts at patch row row0 and column col0; PWID is the
// patch width in pixels; SW selects the swizzled patch layout.  `wchunk` may
// point into LDS (weights staged there); `nf` is then the fragment count of
// a staged weight row.  TAP: a tap chunk (CG 2; one column group, slot 3 =
// group 1 of the centre pixel).  (Upsampled-source chunks: mma_chunk_up.)
template <int NFW, int R, int CG, bool PF, int PWID = PW, bool SW = false, bool TAP = false,
          bool BF = false, typename Hook>
__device__ __forceinline__ void mma_chunk(floatx4 (&acc)[R][NFW], uint4 (&acur)[3][NFW],
                                          const _Float16* lds, int cur, int zero,
                                          const uint4* wchunk, const uint4* wnext, int nf,
                                          int row0, int col0, int g, int c, Hook&& hook) {
  static_assert(!TAP || CG == 2, "tap chunks are 16-lane sources");
  constexpr int NCG = TAP ? 1 : (3 * CG + 3) / 4;
#pragma unroll 1
  for (int j = 0; j < NCG; ++j) {
    if constexpr (!PF) {
      // no register double buffer (keeps occupancy): load this group's weights now
#pragma unroll
      for (int ky = 0; ky < 3; ++ky)
#pragma unroll
        for (int q = 0; q < NFW; ++q) acur[ky][q] = wchunk[((size_t)(j * 3 + ky) * nf + q) * 64];
    }
    const uint4* wn = !PF ? nullptr : j + 1 < NCG ? wchunk + (size_t)(j + 1) * 3 * nf * 64 : wnext;
    uint4 anext[3][NFW];
    if (wn) {
#pragma unroll
      for (int ky = 0; ky < 3; ++ky)
#pragma unroll
        for (int q = 0; q < NFW; ++q) anext[ky][q] = wn[(ky * nf + q) * 64];
    }
    if (j == 0) hook();
    const int slot = 4 * j + g;
    int base = zero, rstride = 0;
    if (TAP || slot < 3 * CG) {
      const int kx = TAP ? (slot < 3 ? slot : 1) : slot / CG;
      const int grp = TAP ? (slot < 3 ? 0 : 1) : slot - kx * CG;
      constexpr int PS = pstride<CG, SW>();
      const int col = col0 + c + kx;
      base = cur + (row0 * PWID + col) * PS + 8 * gslot<CG, SW>(col, grp);
      rstride = PWID * PS;
    }
#pragma unroll
    for (int p = 0; p < R + 2; ++p) {
      const uint4 b = *reinterpret_cast<const uint4*>(lds + base + p * rstride);
#pragma unroll
      for (int ky = 0; ky < 3; ++ky) {
        const int r = p - ky;
        if (r >= 0 && r < R) {
#pragma unroll
          for (int q = 0; q < NFW; ++q)
            acc[r][q] = mfma16<BF>(acur[ky][q], b, acc[r][q]);
        }
      }
    }
    if (wn) {
#pragma unroll
      for (int ky = 0; ky < 3; ++ky)
#pragma unroll
        for (int q = 0; q < NFW; ++q) acur[ky][q] = anext[ky][q];
    }
  }
}

// MFMAs of one chunk of the nearest-2x-upsampled source, sub-pixel over
// rows.  Through its three ky taps, an output row y = 2 Y + py of the
// upsampled image reads only two low-resolution rows: Y - 1 (weight W0)
// and Y (W1 + W2) when py = 0; Y (W0 + W1) and Y + 1 (W2) when py = 1 --
// exact in real arithmetic (the zero padding of row -1 and row 2 H maps to
// low-resolution rows -1 and H, which the patch holds as zeros).  The
// chunk's weights hold these four row combinations a = 0..3 per column group
// (A index (j * 4 + a) * nf + q), so an output row takes two MFMAs per
// column group instead of three, and low-resolution patch row qr of the
// wave's window serves output rows 2 qr (a = 0), 2 qr - 2 (a = 1),
// 2 qr - 1 (a = 2) and 2 qr - 3 (a = 3): R / 2 + 2 B reads per column group
// instead of R + 2.  Low-resolution patch column (c + kx + 1) / 2 holds
// the full-resolution column c + kx - 1 of the wave's window (row0 even).
// The A operands are loaded per column group and combination (from LDS or
// global memory).
template <int NFW, int R, int CG, bool SW, bool BF = false>
__device__ __forceinline__ void mma_chunk_up(floatx4 (&acc)[R][NFW], const _Float16* lds, int cur,
                                             int zero, const uint4* wchunk, int nf, int row0,
                                             int col0, int g, int c) {
  static_assert(R % 2 == 0, "output rows come in pairs");
  constexpr int NCG = (3 * CG + 3) / 4;
#pragma unroll 1
  for (int j = 0; j < NCG; ++j) {
    const int slot = 4 * j + g;
    int base = zero, rstride = 0;
    if (slot < 3 * CG) {
      const int kx = slot / CG;
      const int grp = slot - kx * CG;
      constexpr int PS = pstride<CG, SW>();
      const int col = (col0 + c + kx + 1) >> 1;
      base = cur + ((row0 >> 1) * LPW + col) * PS + 8 * gslot<CG, SW>(col, grp);
      rstride = LPW * PS;
    }
    // the column group's R / 2 + 2 B fragments, then one row combination's
    // A operands at a time (registers: B rows + NFW A, not 4 NFW A)
    uint4 b[R / 2 + 2];
#pragma unroll
    for (int qr = 0; qr < R / 2 + 2; ++qr)
      b[qr] = *reinterpret_cast<const uint4*>(lds + base + qr * rstride);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      uint4 aa[NFW];
#pragma unroll
      for (int q = 0; q < NFW; ++q) aa[q] = wchunk[((size_t)(j * 4 + a) * nf + q) * 64];
#pragma unroll
      for (int qr = 0; qr < R / 2 + 2; ++qr) {
        const int r = a == 0 ? 2 * qr : a == 1 ? 2 * qr - 2 : a == 2 ? 2 * qr - 1 : 2 * qr - 3;
        if (r >= 0 && r < R) {
#pragma unroll
          for (int q = 0; q < NFW; ++q)
            acc[r][q] = mfma16<BF>(aa[q], b[qr], acc[r][q]);
        }
      }
    }
  }
}

template <bool OUTF32, bool BF>
__device__ __forceinline__ void store4(void* y, size_t idx, float v0, float v1, float v2, float v3) {
  if constexpr (OUTF32) {
    *reinterpret_cast<float4*>(static_cast<float*>(y) + idx) = make_float4(v0, v1, v2, v3);
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + idx) =
        make_uint2(pack2<BF>(v0, v1), pack2<BF>(v2, v3));
  }
}

template <bool OUTF32, bool BF>
__device__ __forceinline__ void store8(void* y, size_t idx, const float (&v)[8]) {
  if constexpr (OUTF32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(y) + idx);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + idx) =
        make_uint4(pack2<BF>(v[0], v[1]), pack2<BF>(v[2], v[3]), pack2<BF>(v[4], v[5]),
                   pack2<BF>(v[6], v[7]));
  }
}

// Stores one pixel's values of this lane's NFW fragments (fragments q0 ..):
// v[q][i] is output channel chan[q] + i.  The two fragments of a pair held
// by the same lane are 8 consecutive channels and go out as one 16-byte
// store when all 8 are stored channels; others as 8-byte stores.  Channels
// at or past cout_stored (a multiple of 4) are never written.
template <int NFW, bool OUTF32, bool BF>
__device__ __forceinline__ void store_pixel(void* y, size_t pix, const int (&chan)[NFW],
                                            const bool (&lead)[NFW], const bool (&tail)[NFW],
                                            int cout_stored, const float (&v)[NFW][4]) {
#pragma unroll
  for (int q = 0; q < NFW; ++q) {
    if (chan[q] >= cout_stored) continue;
    if (tail[q] && chan[q] + 4 <= cout_stored) continue;   // written with its pair's lead
    if (q + 1 < NFW && lead[q] && chan[q] + 8 <= cout_stored) {
      const float w8[8] = {v[q][0], v[q][1], v[q][2], v[q][3],
                           v[q + 1][0], v[q + 1][1], v[q + 1][2], v[q + 1][3]};
      store8<OUTF32, BF>(y, pix + chan[q], w8);
    } else {
      store4<OUTF32, BF>(y, pix + chan[q], v[q][0], v[q][1], v[q][2], v[q][3]);
    }
  }
}

// Epilogue of one wave: bias, ReLU, then the store or the fused 2x2 pool.
// acc[r][q] holds, for this lane (16-lane group g), rows 4 g .. 4 g + 3 of
// fragment q0 + q for pixel (yb + r, x); c is the pixel column in the tile.
// Pixels at or past column xend (<= the image width) are not stored.
// EpiChan holds this lane's output channels and biases.
template <int NFW>
struct EpiChan {
  int chan[NFW];
  bool lead[NFW], tail[NFW];   // first / second fragment of a pair this lane holds both of
  float bv[NFW][4];
};

template <int NFW>
__device__ __forceinline__ EpiChan<NFW> epi_chan(const float* bias, int nf, int q0, int g) {
  EpiChan<NFW> e;
#pragma unroll
  for (int q = 0; q < NFW; ++q) {
    const int f = q0 + q;
    const bool paired = (f | 1) < nf;
    e.chan[q] = 32 * (f >> 1) + (paired ? 8 * g + 4 * (f & 1) : 4 * g);
    e.lead[q] = paired && (f & 1) == 0 && q + 1 < NFW;
    e.tail[q] = paired && (f & 1) == 1 && q >= 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) e.bv[q][i] = bias[e.chan[q] + i];
  }
  return e;
}

template <int NFW, int R, bool OUTF32, bool BF>
__device__ __forceinline__ void store_tile_chan(const floatx4 (&acc)[R][NFW], const EpiChan<NFW>& e,
                                                const ConvF16Args& a, void* y, int yb, int x, int c,
                                                int pool, int relu, int xend) {
  const int (&chan)[NFW] = e.chan;
  const bool (&lead)[NFW] = e.lead;
  const bool (&tail)[NFW] = e.tail;
  const float (&bv)[NFW][4] = e.bv;
  // relu is uniform: each branch gets its own copy of the loops (a select
  // per value otherwise)
  auto plain = [&](auto with_relu) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int yy = yb + r;
      if (yy < a.h && x < xend) {
        float v[NFW][4];
#pragma unroll
        for (int q = 0; q < NFW; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[q][i] = acc[r][q][i] + bv[q][i];
            if constexpr (decltype(with_relu)::value) v[q][i] = fmaxf(v[q][i], 0.f);
          }
        store_pixel<NFW, OUTF32, BF>(y, ((size_t)yy * a.w + x) * a.cout_stored, chan, lead, tail,
                                 a.cout_stored, v);
      }
    }
  };
  // 2x2 max of the biased values (adding the bias commutes with the max:
  // rounding is monotone).  After ReLU the values are +0 or positive, whose
  // bit patterns order like the values: integer maxima, no NaN quieting.
  auto pooled = [&](auto with_relu) {
    const int ow = a.w >> 1;
#pragma unroll
    for (int rp = 0; rp < R / 2; ++rp) {
      float m[NFW][4];
#pragma unroll
      for (int q = 0; q < NFW; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (decltype(with_relu)::value) {
            const int v0 = __float_as_int(fmaxf(acc[2 * rp][q][i] + bv[q][i], 0.f));
            const int v1 = __float_as_int(fmaxf(acc[2 * rp + 1][q][i] + bv[q][i], 0.f));
            const int v = max(v0, v1);
            m[q][i] = __int_as_float(max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false)));
          } else {
            const float v = fmaxf(acc[2 * rp][q][i], acc[2 * rp + 1][q][i]) + bv[q][i];
            m[q][i] = fmaxf(v, swap_pair(v));
          }
        }
      const int yy = yb + 2 * rp;
      if ((c & 1) == 0 && yy < a.h && x < xend)
        store_pixel<NFW, OUTF32, BF>(y, ((size_t)(yy >> 1) * ow + (x >> 1)) * a.cout_stored, chan,
                                 lead, tail, a.cout_stored, m);
    }
  };
  if (!pool) {
    if (relu) plain(std::true_type{}); else plain(std::false_type{});
  } else {
    if (relu) pooled(std::true_type{}); else pooled(std::false_type{});
  }
}

template <int NFW, int R, bool OUTF32, bool BF>
__device__ __forceinline__ void store_tile(const floatx4 (&acc)[R][NFW], const ConvF16Args& a,
                                           void* y, int q0, int g, int yb, int x, int c, int pool,
                                           int relu, int xend) {
  store_tile_chan<NFW, R, OUTF32, BF>(acc, epi_chan<NFW>(a.bias, a.nf, q0, g), a, y, yb, x, c, pool,
                                      relu, xend);
}

// Direct global -> LDS copy of a chunk's weight rows for the workgroup's FB
// fragments: NB = (column groups) x 3 x FB blocks of 1 KB; block k is
// fragment k % FB of weight row k / FB (a row holds nf fragments, `w` points
// at the workgroup's first one, lane offset included).  The four waves
// issue them round-robin; the barrier that follows drains them (with ASM,
// after an explicit vmcnt wait).
template <int NB, bool ASM = false>
__device__ __forceinline__ void stage_weights(_Float16* dst, const uint4* w, int nf, int fb,
                                              int wave) {
  uint4* slots = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int i = 0; i < (NB + 3) / 4; ++i) {
    const int k = wave + 4 * i;
    if (k >= NB) break;
    const int row = k / fb;
    dma16<ASM>(w + (size_t)(row * nf + (k - row * fb)) * 64, slots + k * 64);
  }
}

// Weight prefetch doubles the A registers (12 NFW more); use it only where
// accumulators and both A sets leave room for two waves per SIMD.
template <int NFW, int R>
constexpr bool kPrefetch = 4 * R * NFW + 24 * NFW <= 176;

// Staged weights: the workgroup's FB fragments of one chunk take 9 FB KB
// (3 column groups x 3 ky x FB, 1 KB each), 12 FB KB for an upsampled
// chunk (4 row combinations), which sits after that chunk's smaller
// half-resolution patch.  They go to LDS where the swizzled patches and
// those weights leave room for two workgroups per CU.
template <int TH>
constexpr int kUpPatch = ((TH / 2 + 2) * LPW * 32 + 511) / 512 * 512;   // halves (swizzled)
template <int NFW, int R, int WR>
constexpr int kWlHalves = cmax(Tile<WR * R, true>::PATCH + 8 * 9 * NFW * (4 / WR) * 64,
                               kUpPatch<WR * R> + 8 * 12 * NFW * (4 / WR) * 64);
template <int NFW, int R, int WR>
constexpr bool kWeightsInLds = 2 * (2 * kWlHalves<NFW, R, WR> + 16) <= 160 * 1024;

// A workgroup of 4 waves covers a (WR R) x 16 tile for FB = NFW (4 / WR)
// output fragments: wave w computes rows [R (w % WR), + R) for the NFW
// fragments starting at FB blockIdx.y + NFW (w / WR).
// With the weights in LDS (WL) each chunk's weight rows for the FB
// fragments are copied there with the chunk's patch (one 1 KB direct load
// per (column group, ky, fragment)), so the four waves share one copy and
// the A operands come from LDS; the patch uses the swizzled layout.  Else
// every wave reads its A operands from global memory (L1/L2), with the next
// column group's prefetched into registers where they fit.
template <int NFW, int R, int WR, bool OUTF32, bool BF>
__device__ __forceinline__ void conv3x3_body(const ConvF16Args& __restrict__ a, int upcat, int pool, int relu) {
  static_assert(WR == 1 || WR == 2 || WR == 4, "row groups");
  constexpr bool WL = kWeightsInLds<NFW, R, WR>;
  constexpr bool SW = WL;
  constexpr int FB = NFW * (4 / WR);             // fragments per workgroup
  using T = Tile<WR * R, SW>;
  constexpr int WOFF = T::PATCH;                 // staged weights of a plain chunk (halves)
  constexpr int WOFF_UP = kUpPatch<WR * R>;      // ... of an upsampled chunk
  constexpr int ZERO = WL ? kWlHalves<NFW, R, WR> : T::PATCH;
  __shared__ __attribute__((aligned(16))) _Float16 lds[ZERO + 8];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int nf = a.nf;
  const int rg = wave % WR;
  const int q0 = (blockIdx.y * (4 / WR) + wave / WR) * NFW;   // this wave's output fragments
  (void)upcat;
  constexpr bool PF = !WL && kPrefetch<NFW, R>;

  int tx, ty;
  if (!tile_of_block(blockIdx.x, a.tiles_x, a.tiles_y, tx, ty)) return;
  const int y0 = ty * T::TH, x0 = tx * TW;
  // this tile of the batch (locals: writing to `a` would copy all of it,
  // chunk table included, to scratch)
  const size_t boff = (size_t)blockIdx.z * a.bstride;
  const _Float16* const src0 = reinterpret_cast<const _Float16*>(static_cast<const char*>(a.src0) + boff);
  const _Float16* const src1 =
      a.src1 ? reinterpret_cast<const _Float16*>(static_cast<const char*>(a.src1) + boff) : nullptr;
  void* const ydst = static_cast<char*>(a.y) + boff;

  if (tid < 2) reinterpret_cast<uint2*>(lds + ZERO)[tid] = make_uint2(0u, 0u);

  floatx4 acc[R][NFW];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int q = 0; q < NFW; ++q) acc[r][q] = floatx4{0.f, 0.f, 0.f, 0.f};

  const uint4* wf = static_cast<const uint4*>(a.wfrag) + lane + q0 * 64;
  // the workgroup's weight rows (direct loads) and this wave's staged A operands
  const uint4* wblk = static_cast<const uint4*>(a.wfrag) + lane + blockIdx.y * FB * 64;
  const uint4* wl = reinterpret_cast<const uint4*>(lds + WOFF) + lane + (wave / WR) * NFW * 64;
  const uint4* wl_up = reinterpret_cast<const uint4*>(lds + WOFF_UP) + lane + (wave / WR) * NFW * 64;
  uint4 acur[3][NFW];
  // PF: acur holds the first plain chunk's column-group-0 weights on entry
  // to the plain loops (upsampled chunks load theirs per column group)
  auto preload = [&](int ci) {
#pragma unroll
    for (int ky = 0; ky < 3; ++ky)
#pragma unroll
      for (int q = 0; q < NFW; ++q)
        acur[ky][q] = wf[((size_t)a.chunk[ci].wfrag + ky * nf + q) * 64];
  };
  if (PF && a.nup == 0) preload(0);
  // Chunks run in five loops of one shape each: upsampled source (32- then
  // 16-channel chunks), then the plain source (32- then 16-channel chunks,
  // then a tap chunk).
  const int bounds[6] = {0, a.nup4, a.nup, a.nup + a.npl4, a.nchunks - a.ntap, a.nchunks};
#define OIDN_UP_LOOP(K, CG)                                                                     \
  _Pragma("unroll 1") for (int ci = bounds[K]; ci < bounds[K + 1]; ++ci) {                      \
    const ConvChunk ch = a.chunk[ci];                                                           \
    const _Float16* src = src0;                                                                 \
    __syncthreads();                                                                            \
    if ((a.cs0 & 7) == 0)                                                                       \
      stage_patch_direct<T::TH, 4, T::PATCH / 8, CG, true, SW>(reinterpret_cast<uint4*>(lds),    \
                                                               src, a.cs0, ch.coff, a.h, a.w,   \
                                                               y0, x0, wave, lane);             \
    else                                                                                        \
      stage_patch<T::TH, CG, false, true, SW>(lds, src, a.cs0, ch.coff, a.h, a.w, y0, x0, tid);  \
    if constexpr (WL) stage_weights<(3 * CG + 3) / 4 * 4 * FB>(                                 \
                          lds + WOFF_UP, wblk + (size_t)ch.wfrag * 64, nf, FB, wave);           \
    __syncthreads();                                                                            \
    if constexpr (WL)                                                                           \
      mma_chunk_up<NFW, R, CG, SW, BF>(acc, lds, 0, ZERO, wl_up, FB, R * rg, 0, g, c);          \
    else                                                                                        \
      mma_chunk_up<NFW, R, CG, SW, BF>(acc, lds, 0, ZERO, wf + (size_t)ch.wfrag * 64, nf, R * rg, 0, \
                                   g, c);                                                       \
  }
#define OIDN_CHUNK_LOOP(K, CG, TAP)                                                             \
  _Pragma("unroll 1") for (int ci = bounds[K]; ci < bounds[K + 1]; ++ci) {                      \
    const ConvChunk ch = a.chunk[ci];                                                           \
    const _Float16* src = ch.src ? src1 : src0;                                                 \
    const int cs = ch.src ? a.cs1 : a.cs0;                                                      \
    const uint4* wnext = ci + 1 < a.nchunks ? wf + (size_t)a.chunk[ci + 1].wfrag * 64 : nullptr; \
    __syncthreads();                                                                            \
    if ((cs & 7) == 0)                                                                          \
      stage_patch_direct<T::TH, 4, T::PATCH / 8, CG, false, SW>(reinterpret_cast<uint4*>(lds),   \
                                                                src, cs, ch.coff, a.h, a.w, y0, \
                                                                x0, wave, lane);                \
    else                                                                                        \
      stage_patch<T::TH, CG, false, false, SW>(lds, src, cs, ch.coff, a.h, a.w, y0, x0, tid);   \
    if constexpr (WL) stage_weights<(TAP ? 1 : (3 * CG + 3) / 4) * 3 * FB>(                      \
                          lds + WOFF, wblk + (size_t)ch.wfrag * 64, nf, FB, wave);              \
    __syncthreads();                                                                            \
    if constexpr (WL)                                                                           \
      mma_chunk<NFW, R, CG, false, PW, SW, TAP, BF>(acc, acur, lds, 0, ZERO, wl, nullptr, FB,    \
                                                R * rg, 0, g, c, [] {});                        \
    else                                                                                        \
      mma_chunk<NFW, R, CG, PF, PW, false, TAP, BF>(acc, acur, lds, 0, ZERO,                     \
                                                wf + (size_t)ch.wfrag * 64, wnext, nf, R * rg,  \
                                                0, g, c, [] {});                                \
  }
  OIDN_UP_LOOP(0, 4)
  OIDN_UP_LOOP(1, 2)
  if (PF && a.nup > 0 && a.nup < a.nchunks) preload(a.nup);
  OIDN_CHUNK_LOOP(2, 4, false)
  OIDN_CHUNK_LOOP(3, 2, false)
  OIDN_CHUNK_LOOP(4, 2, true)
#undef OIDN_CHUNK_LOOP
#undef OIDN_UP_LOOP
  (void)upcat;

  store_tile<NFW, R, OUTF32, BF>(acc, a, ydst, q0, g, y0 + R * rg, x0 + c, c, pool, relu, a.w);
}

// ---------------------------------------------------------------------------
// Weight-stationary producer / consumer form, for layers whose whole weight
// set (the workgroup's FB fragments of every chunk) fits in LDS next to two
// patch slots.  In the form above every tile re-copies its chunks' weight
// rows (108 KB per tile at dec_conv1a against 43 KB of patches), and the
// CU's LDS fill rate bounds the layer.  Here a persistent workgroup of eight
// waves copies the weights once and walks its tiles' chunks as one stream
// of steps: waves 0-3 (one per SIMD) multiply step s from patch slot s & 1
// and, after a tile's last chunk, run its epilogue and stores; waves 4-7
// copy the patch of step s + 1 into the other slot and wait for it; one
// barrier per step.  The matrix waves read nothing from global memory after
// the biases (kept in LDS), so no wait of theirs covers a store, and the
// copy waves store nothing, so their waits cover their copies only.
// LDS (halves): [slot 0 | slot 1 | weights of chunk 0, 1, ... | biases | zero].
// Tiles of a workgroup: bx = blockIdx.x + k gridDim.x (gridDim.x a multiple
// of kXcds, so all of them map to one XCD).
// ---------------------------------------------------------------------------
constexpr int WS_THREADS = 512;
#ifndef OIDN_WS_ENABLE
#define OIDN_WS_ENABLE 1
#endif
template <int NFW, int R, int WR>
constexpr bool kWsCandidate = NFW == 4 && R == 8 && WR == 4;

// Halves of weights a chunk kind occupies for FB fragments.
__host__ __device__ constexpr int ws_chunk_weights(int ncg, bool up, int fb) {
  return ncg * (up ? 4 : 3) * fb * 512;
}

template <int NFW, int R, int WR, bool OUTF32, bool BF>
__device__ __forceinline__ void conv3x3_ws_body(const ConvF16Args& __restrict__ a, int pool, int relu) {
  constexpr bool SW = true;
  constexpr int FB = NFW * (4 / WR);
  using T = Tile<WR * R, SW>;
  extern __shared__ __attribute__((aligned(16))) _Float16 lds[];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int nf = a.nf;
  const int nch = a.nchunks;
  const int pslot = a.ws_pslot;
  const int wbase = 2 * pslot;
  int wtot = 0;
  for (int ci = 0; ci < nch; ++ci) wtot += ws_chunk_weights(a.chunk[ci].ncg, ci < a.nup, FB);
  float* const bias_lds = reinterpret_cast<float*>(lds + wbase + wtot);
  const int zero = wbase + wtot + 2 * 16 * nf;
  if (tid < 2) reinterpret_cast<uint2*>(lds + zero)[tid] = make_uint2(0u, 0u);
  // the slots of every batched tile in one sequence: slot t is tile slot
  // t mod grid_x of batch entry t / grid_x (grid_x is a multiple of kXcds)
  const int nslots = (a.batch > 1 ? a.batch : 1) * a.grid_x;
  const int ntile = (nslots - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int nsteps = ntile * nch;
  const int bounds[6] = {0, a.nup4, a.nup, a.nup + a.npl4, a.nchunks - a.ntap, a.nchunks};
  // tile k of this workgroup: its origin and batch byte offset; a padding
  // slot past the last tile becomes a tile below the image (zero patches,
  // nothing stored)
  auto tile = [&](int k, int& y0, int& x0, size_t& boff) {
    const int t = (int)blockIdx.x + k * (int)gridDim.x;
    const int z = t / a.grid_x;
    boff = (size_t)z * a.bstride;
    int tx, ty;
    if (tile_of_block(t - z * a.grid_x, a.tiles_x, a.tiles_y, tx, ty)) {
      y0 = ty * T::TH;
      x0 = tx * TW;
    } else {
      y0 = a.h + 2;
      x0 = 0;
    }
  };

  if (wave >= 4) {
    // copy waves: the weights once, then one patch per step
    const int cw = wave - 4;
    const uint4* const wblk = static_cast<const uint4*>(a.wfrag) + lane + blockIdx.y * FB * 64;
    {
      int woff = wbase;
      for (int ci = 0; ci < nch; ++ci) {
        const ConvChunk ch = a.chunk[ci];
        const uint4* const w = wblk + (size_t)ch.wfrag * 64;
        _Float16* const dst = lds + woff;
        const int K = ci < bounds[1] ? 0 : ci < bounds[2] ? 1 : ci < bounds[3] ? 2 : ci < bounds[4] ? 3 : 4;
        if (K == 0) stage_weights<3 * 4 * FB, true>(dst, w, nf, FB, cw);
        else if (K == 1) stage_weights<2 * 4 * FB, true>(dst, w, nf, FB, cw);
        else if (K == 2) stage_weights<3 * 3 * FB, true>(dst, w, nf, FB, cw);
        else if (K == 3) stage_weights<2 * 3 * FB, true>(dst, w, nf, FB, cw);
        else stage_weights<1 * 3 * FB, true>(dst, w, nf, FB, cw);
        woff += ws_chunk_weights(ch.ncg, ci < a.nup, FB);
      }
    }
    auto copy = [&](int s) {
      int ln = lane, ct = tid - 256;
      asm volatile("" : "+v"(ln), "+v"(ct));
      const int k = s / nch, ci = s - k * nch;
      int y0, x0;
      size_t boff;
      tile(k, y0, x0, boff);
      const _Float16* const src0 =
          reinterpret_cast<const _Float16*>(static_cast<const char*>(a.src0) + boff);
      const _Float16* const src1 =
          a.src1 ? reinterpret_cast<const _Float16*>(static_cast<const char*>(a.src1) + boff) : nullptr;
      const ConvChunk ch = a.chunk[ci];
      _Float16* const base = lds + (s & 1) * pslot;
      uint4* const slots = reinterpret_cast<uint4*>(base);
      const int K = ci < bounds[1] ? 0 : ci < bounds[2] ? 1 : ci < bounds[3] ? 2 : ci < bounds[4] ? 3 : 4;
      if (K <= 1) {
        if ((a.cs0 & 7) != 0) {
          if (K == 0) stage_patch<T::TH, 4, false, true, SW>(base, src0, a.cs0, ch.coff, a.h, a.w, y0, x0, ct);
          else stage_patch<T::TH, 2, false, true, SW>(base, src0, a.cs0, ch.coff, a.h, a.w, y0, x0, ct);
        } else if (K == 0) {
          stage_patch_direct<T::TH, 4, T::PATCH / 8, 4, true, SW, true>(slots, src0, a.cs0, ch.coff, a.h,
                                                                        a.w, y0, x0, cw, ln);
        } else {
          stage_patch_direct<T::TH, 4, T::PATCH / 8, 2, true, SW, true>(slots, src0, a.cs0, ch.coff, a.h,
                                                                        a.w, y0, x0, cw, ln);
        }
        return;
      }
      const _Float16* src = ch.src ? src1 : src0;
      const int cs = ch.src ? a.cs1 : a.cs0;
      if ((cs & 7) != 0) {
        if (K == 2) stage_patch<T::TH, 4, false, false, SW>(base, src, cs, ch.coff, a.h, a.w, y0, x0, ct);
        else stage_patch<T::TH, 2, false, false, SW>(base, src, cs, ch.coff, a.h, a.w, y0, x0, ct);
      } else if (K == 2) {
        stage_patch_direct<T::TH, 4, T::PATCH / 8, 4, false, SW, true>(slots, src, cs, ch.coff, a.h, a.w,
                                                                       y0, x0, cw, ln);
      } else {
        stage_patch_direct<T::TH, 4, T::PATCH / 8, 2, false, SW, true>(slots, src, cs, ch.coff, a.h, a.w,
                                                                       y0, x0, cw, ln);
      }
    };
    if (nsteps > 0) copy(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
#pragma unroll 1
    for (int s = 0; s < nsteps; ++s) {
      __builtin_amdgcn_s_barrier();
      if (s + 1 < nsteps) copy(s + 1);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    }
    return;
  }

  // matrix waves
  const int g = lane >> 4, c = lane & 15;
  const int rg = wave % WR;
  const int q0 = (blockIdx.y * (4 / WR) + wave / WR) * NFW;
  for (int i = tid; i < 16 * nf; i += 256) bias_lds[i] = a.bias[i];
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  const uint4* const wl = reinterpret_cast<const uint4*>(lds) + lane + (wave / WR) * NFW * 64;
  floatx4 acc[R][NFW];
  uint4 acur[3][NFW];
  int s = 0;
#pragma unroll 1
  for (int k = 0; k < ntile; ++k) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int q = 0; q < NFW; ++q) acc[r][q] = floatx4{0.f, 0.f, 0.f, 0.f};
    int woff = wbase;
#define OIDN_WS_UP(K, CG)                                                                       \
    _Pragma("unroll 1") for (int ci = bounds[K]; ci < bounds[K + 1]; ++ci, ++s) {               \
      __builtin_amdgcn_s_barrier();                                                             \
      mma_chunk_up<NFW, R, CG, SW, BF>(acc, lds, (s & 1) * pslot, zero, wl + woff / 8, FB, R * rg, 0, g, c); \
      woff += ws_chunk_weights(a.chunk[ci].ncg, true, FB);                                      \
    }
#define OIDN_WS_PL(K, CG, TAP)                                                                  \
    _Pragma("unroll 1") for (int ci = bounds[K]; ci < bounds[K + 1]; ++ci, ++s) {               \
      __builtin_amdgcn_s_barrier();                                                             \
      mma_chunk<NFW, R, CG, false, PW, SW, TAP, BF>(acc, acur, lds, (s & 1) * pslot, zero, wl + woff / 8, \
                                                    nullptr, FB, R * rg, 0, g, c, [] {});       \
      woff += ws_chunk_weights(a.chunk[ci].ncg, false, FB);                                     \
    }
    OIDN_WS_UP(0, 4)
    OIDN_WS_UP(1, 2)
    OIDN_WS_PL(2, 4, false)
    OIDN_WS_PL(3, 2, false)
    OIDN_WS_PL(4, 2, true)
#undef OIDN_WS_UP
#undef OIDN_WS_PL
    int y0, x0;
    size_t boff;
    tile(k, y0, x0, boff);
    store_tile_chan<NFW, R, OUTF32, BF>(acc, epi_chan<NFW>(bias_lds, nf, q0, g), a,
                                        static_cast<char*>(a.y) + boff, y0 + R * rg, x0 + c, c, pool,
                                        relu, a.w);
  }
}

template <int NFW, int R, int WR, bool OUTF32>
__global__ __launch_bounds__(WS_THREADS, 1) void conv3x3_ws_f16(ConvF16Args a, int pool, int relu) {
  if constexpr (kWsCandidate<NFW, R, WR>) conv3x3_ws_body<NFW, R, WR, OUTF32, false>(a, pool, relu);
}
template <int NFW, int R, int WR, bool OUTF32>
__global__ __launch_bounds__(WS_THREADS, 1) void conv3x3_ws_bf16(ConvF16Args a, int pool, int relu) {
  if constexpr (kWsCandidate<NFW, R, WR>) conv3x3_ws_body<NFW, R, WR, OUTF32, true>(a, pool, relu);
}

// LDS bytes of the weight-stationary form for a's chunks (0 if it does not
// fit in a CU's 160 KB), and the patch slot size it sets in a.ws_pslot.
template <int NFW, int R, int WR>
size_t ws_lds_bytes(ConvF16Args& a) {
  constexpr int FB = NFW * (4 / WR);
  using T = Tile<WR * R, true>;
  const int tap_patch = ((WR * R + 2) * PW * 16 + 511) / 512 * 512;
  int pslot = 0, wtot = 0;
  for (int ci = 0; ci < a.nchunks; ++ci) {
    const ConvChunk& ch = a.chunk[ci];
    const bool up = ci < a.nup;
    const int patch = up ? kUpPatch<WR * R> : ch.cg == 4 ? T::PATCH : tap_patch;
    pslot = patch > pslot ? patch : pslot;
    wtot += ws_chunk_weights(ch.ncg, up, FB);
  }
  a.ws_pslot = pslot;
  const size_t bytes = (size_t)(2 * pslot + wtot) * 2 + 16 * 4 * (size_t)a.nf + 16;
  return bytes <= 160 * 1024 ? bytes : 0;
}

int device_cus();

// Workgroups along x of the weight-stationary launch: one per CU (shared by
// the nsplit y slices), a multiple of kXcds, at most the batch's tile slots.
int ws_grid_x(int grid_x, int batch, int nsplit) {
  const int nslots = (batch > 1 ? batch : 1) * grid_x;
  int gx = device_cus() / nsplit / kXcds * kXcds;
  return gx < kXcds ? kXcds : gx > nslots ? nslots : gx;
}

// Compute units of the current device (looked up once per device).
int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Raises kernel `fn`'s dynamic LDS limit to at least `bytes` on the current
// device: once per device and kernel (slot 0 / 1: the fp16 / bf16 form),
// again only for a larger size.
hipError_t allow_dynamic_lds(const void* fn, int slot, int bytes) {
  static std::atomic<int> granted[64][2];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (granted[dev][slot].load(std::memory_order_acquire) >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  int cur = granted[dev][slot].load(std::memory_order_relaxed);
  while (cur < bytes && !granted[dev][slot].compare_exchange_weak(cur, bytes)) {
  }
  return hipSuccess;
}

// The kernels: fp16 and bf16 storage.
template <int NFW, int R, int WR, bool OUTF32>
__global__ __launch_bounds__(THREADS, 2) void conv3x3_f16_mfma(ConvF16Args a, int upcat, int pool,
                                                               int relu) {
  conv3x3_body<NFW, R, WR, OUTF32, false>(a, upcat, pool, relu);
}
template <int NFW, int R, int WR, bool OUTF32>
__global__ __launch_bounds__(THREADS, 2) void conv3x3_bf16_mfma(ConvF16Args a, int upcat, int pool,
                                                                int relu) {
  conv3x3_body<NFW, R, WR, OUTF32, true>(a, upcat, pool, relu);
}

template <int NFW, int R, int WR>
hipError_t launch_shape(ConvF16Args a, int nsplit, bool upcat, bool pool, bool relu,
                        bool out_f32, bool bf16, hipStream_t stream) {
  a.tiles_x = cdiv(a.w, TW);
  a.tiles_y = cdiv(a.h, WR * R);
  const int ntiles = a.tiles_x * a.tiles_y;
  a.grid_x = cdiv(ntiles, kXcds) * kXcds;
  if constexpr (kWsCandidate<NFW, R, WR>) {
    // (fp16 / bf16 outputs only: no network layer with an fp32 output fits)
    const size_t lds = OIDN_WS_ENABLE && !out_f32 ? ws_lds_bytes<NFW, R, WR>(a) : 0;
    if (lds > 0) {
      const int gx = ws_grid_x(a.grid_x, a.batch, nsplit);
      const void* fn = bf16 ? (const void*)conv3x3_ws_bf16<NFW, R, WR, false>
                            : (const void*)conv3x3_ws_f16<NFW, R, WR, false>;
      hipError_t e = allow_dynamic_lds(fn, bf16 ? 1 : 0, (int)lds);
      if (e != hipSuccess) return e;
      const dim3 wgrid(gx, nsplit, 1), wblock(WS_THREADS);
      if (bf16)
        hipLaunchKernelGGL((conv3x3_ws_bf16<NFW, R, WR, false>), wgrid, wblock, lds, stream, a, (int)pool, (int)relu);
      else
        hipLaunchKernelGGL((conv3x3_ws_f16<NFW, R, WR, false>), wgrid, wblock, lds, stream, a, (int)pool, (int)relu);
      return hipGetLastError();
    }
  }
  const dim3 grid(cdiv(ntiles, kXcds) * kXcds, nsplit, a.batch > 1 ? a.batch : 1), block(THREADS);
  if (bf16 && out_f32)
    hipLaunchKernelGGL((conv3x3_bf16_mfma<NFW, R, WR, true>), grid, block, 0, stream, a,
                       (int)upcat, (int)pool, (int)relu);
  else if (bf16)
    hipLaunchKernelGGL((conv3x3_bf16_mfma<NFW, R, WR, false>), grid, block, 0, stream, a,
                       (int)upcat, (int)pool, (int)relu);
  else if (out_f32)
    hipLaunchKernelGGL((conv3x3_f16_mfma<NFW, R, WR, true>), grid, block, 0, stream, a,
                       (int)upcat, (int)pool, (int)relu);
  else
    hipLaunchKernelGGL((conv3x3_f16_mfma<NFW, R, WR, false>), grid, block, 0, stream, a,
                       (int)upcat, (int)pool, (int)relu);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Fused pair: y = convB(relu(convA(x))) for a 32-channel intermediate that
// never leaves LDS.  A workgroup of 4 waves covers a 16 x 30 output tile:
// convA runs on the 18 x 32 intermediate window around it (two B fragments
// per row, rows split 9 + 9 between wave pairs), its fp16 result -- zero
// outside the image, the zero padding convB sees -- overwrites the input
// patch in LDS, and convB runs on the 16 x 32 output window (the last two
// columns are computed but not stored).  Every value is rounded and
// accumulated as by two separate launches, so the results are identical.
// ---------------------------------------------------------------------------
constexpr int PAIR_TH = 16, PAIR_TW = 30;          // output tile
constexpr int PAIR_MH = PAIR_TH + 2;               // intermediate rows
constexpr int PAIR_IH = PAIR_TH + 4;               // input patch rows
constexpr int PAIR_PW = 34;                        // patch width (input and intermediate)

// With 32-channel convA chunks (SW) the input patch and the intermediate
// use the swizzled layout and the weights are staged in LDS: each convA
// chunk's rows (2 fragments) with its patch, then convB's (NFB <= 2
// fragments) while the intermediate is written -- the four waves share one
// copy instead of each reading every A operand from global memory.  That
// still leaves two workgroups per CU.  16-channel convA chunks (three
// workgroups per CU, no LDS to spare) keep the padded input patch and
// global weights; their intermediate is swizzled (MSW) where the input pass
// runs in the staging: 39 KB, four workgroups per CU.
template <int CGA, bool MSW = CGA == 4>
struct PairLds {
  static constexpr bool SW = CGA == 4;
  static constexpr int IN = PAIR_IH * PAIR_PW * pstride<CGA, SW>();     // halves
  static constexpr int MID = PAIR_MH * PAIR_PW * pstride<4, MSW>();
  static constexpr int REGION = ((IN > MID ? IN : MID) + 511) / 512 * 512;
  static constexpr int WSLOTS = SW ? 9 * 2 * 64 : 0;                 // weight rows (16 B slots)
  static constexpr int WOFF = REGION;
  static constexpr int ZERO = REGION + 8 * WSLOTS;
};

// Stages one convA chunk: the (PAIR_IH x PAIR_PW)-pixel window at
// (y0 - 2, x0 - 2), same slot rules as stage_patch_direct.
template <int CG, bool SW>
__device__ __forceinline__ void stage_pair_input(uint4* slots, const _Float16* src, int cs,
                                                 int coff, int h, int w, int y0, int x0,
                                                 int wave, int lane) {
  constexpr int NPIX = PAIR_IH * PAIR_PW;
  constexpr int SPP = pstride<CG, SW>() / 8;
  constexpr int NLOAD = (NPIX * SPP + 63) / 64;
  static_assert(NLOAD * 64 * 8 <= PairLds<CG>::REGION, "pair patch buffer");
#pragma unroll
  for (int i = 0; i < (NLOAD + 3) / 4; ++i) {
    const int k = wave + 4 * i;
    if (k >= NLOAD) break;
    const int sl = k * 64 + lane;
    const int pp = sl / SPP;
    const int u = sl - pp * SPP;
    if (u < CG && pp < NPIX) {
      const int py = pp / PAIR_PW;
      const int px = pp - py * PAIR_PW;
      const int iy = y0 - 2 + py;
      const int ix = x0 - 2 + px;
      const int c = coff + 8 * gslot<CG, SW>(px, u);
      const void* gp = g_zero16;
      if (iy >= 0 && iy < h && ix >= 0 && ix < w && c < cs)
        gp = src + ((size_t)iy * w + ix) * cs + c;
      __builtin_amdgcn_global_load_lds(gp, slots + k * 64, 16, 0, 0);
    }
  }
}

// The input pass fused into convA's staging (one 16-channel chunk, padded
// layout): patch pixel (py, px) of the window at (y0 - 2, x0 - 2) is network
// tile pixel (y, x).  Inside the tile it holds the packed input as the input
// pass computes it (clamp-to-edge image read, the same per-channel
// arithmetic; with TAPS channel 8 of the row neighbours in lanes 8..10, zero
// outside the tile), outside the tile zero (the conv's padding).  The
// pixels of the workgroup's own output tile are also stored to `in.packed`
// (in.lanes per pixel) for the decoder's later skip read.  Every image load
// is issued before the first value is used.
template <bool TAPS, bool BF>
__device__ __forceinline__ void stage_pair_images(uint4* slots, const PackArgs& in, int h, int w,
                                                  int y0, int x0, int tid) {
  constexpr int NPIX = PAIR_IH * PAIR_PW;
  constexpr int NIT = (NPIX + THREADS - 1) / THREADS;
  constexpr int SPP = pstride<2, false>() / 8;     // 16-byte slots per pixel
  // RGB only (alpha is not an input channel): 3 dwords per image pixel
  float3 col[NIT], alb[NIT], nrm[NIT];
  float zl[NIT], zr[NIT];
  auto rgb = [](const float4* img, size_t i) { return *reinterpret_cast<const float3*>(img + i); };
  // Clamp-to-edge coordinates are always inside the image, so every lane
  // loads, with no branches: what lies outside the tile (or past the
  // patch, in the last round) is zeroed or dropped below.
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int pp = tid + THREADS * i;
    const int py = pp / PAIR_PW, px = pp - py * PAIR_PW;
    const int y = y0 - 2 + py, x = x0 - 2 + px;
    const size_t row = (size_t)min(max(y + in.tile_y, 0), in.img_h - 1) * in.img_w;
    const size_t src = row + min(max(x + in.tile_x, 0), in.img_w - 1);
    col[i] = rgb(in.color, src);
    alb[i] = nrm[i] = make_float3(0.f, 0.f, 0.f);
    zl[i] = zr[i] = 0.f;
    if (in.sources > 1) alb[i] = rgb(in.albedo, src);
    if (in.sources > 2) nrm[i] = rgb(in.normal, src);
    if (TAPS) {
      zl[i] = in.normal[row + min(max(x - 1 + in.tile_x, 0), in.img_w - 1)].z;
      zr[i] = in.normal[row + min(max(x + 1 + in.tile_x, 0), in.img_w - 1)].z;
    }
  }
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int pp = tid + THREADS * i;
    if (pp >= NPIX) break;
    const int py = pp / PAIR_PW, px = pp - py * PAIR_PW;
    const int y = y0 - 2 + py, x = x0 - 2 + px;
    const bool inside = y >= 0 && y < h && x >= 0 && x < w;
    float ch[12];
#pragma unroll
    for (int k = 0; k < 12; ++k) ch[k] = 0.f;
    ch[0] = in_color<true>(col[i].x, in.hdr, in.input_scale);
    ch[1] = in_color<true>(col[i].y, in.hdr, in.input_scale);
    ch[2] = in_color<true>(col[i].z, in.hdr, in.input_scale);
    if (in.sources > 1) {
      ch[3] = in_albedo(alb[i].x);
      ch[4] = in_albedo(alb[i].y);
      ch[5] = in_albedo(alb[i].z);
    }
    if (in.sources > 2) {
      ch[6] = in_normal(nrm[i].x);
      ch[7] = in_normal(nrm[i].y);
      ch[8] = in_normal(nrm[i].z);
    }
    if (TAPS) {
      ch[9] = ch[8];
      ch[8] = x > 0 ? in_normal(zl[i]) : 0.f;
      ch[10] = x + 1 < w ? in_normal(zr[i]) : 0.f;
    }
    uint4 g0 = make_uint4(0u, 0u, 0u, 0u), g1 = g0;
    if (inside) {
      g0 = make_uint4(pack2<BF>(ch[0], ch[1]), pack2<BF>(ch[2], ch[3]), pack2<BF>(ch[4], ch[5]),
                      pack2<BF>(ch[6], ch[7]));
      if (in.lanes > 8) g1 = make_uint4(pack2<BF>(ch[8], ch[9]), pack2<BF>(ch[10], ch[11]), 0u, 0u);
      if (py >= 2 && py < 2 + PAIR_TH && px >= 2 && px < 2 + PAIR_TW) {
        // 32-bit offset formed here (a hoisted 64-bit address is spilled)
        int o = (y * w + x) * (in.lanes / 8);
        asm volatile("" : "+v"(o));
        uint4* out = static_cast<uint4*>(in.packed) + o;
        out[0] = g0;
        if (in.lanes > 8) out[1] = g1;
      }
    }
    slots[pp * SPP] = g0;
    slots[pp * SPP + 1] = g1;
  }
}

// A 16-channel convA source leaves LDS for three workgroups per CU; the
// registers are held to that.  32-channel chunks need more LDS: two.  With
// the input pass in the staging and a tap chunk (no chunk loop, one column
// group, swizzled intermediate: 126 VGPRs, 39 KB) four.
template <int CGA, int IN>
constexpr int kPairWaves = IN == (kPairInImages | kPairInTaps) ? 4 : CGA == 2 ? 3 : 2;

// The output pass in convB's epilogue (the network's last conv, one output
// fragment whose RGB weights and biases are replicated in all four 4-channel
// lane groups, lane 3 of each zero): lane group g of column x takes the rows
// r = g, g + 4, ... of the wave's R rows, so the transfer's arithmetic runs
// on every lane.  Each value is the one store_tile would have written as
// fp32 from lane group 0.  `alpha` holds the input colour's alpha of those
// rows, loaded at the start of the kernel (see image_alpha).
template <int R>
__device__ __forceinline__ bool image_index(const OutputPass& o, int h, int g, int k, int yb, int x,
                                            int xend, size_t& i) {
  const int y = yb + g + 4 * k;
  const int lx = x - o.in_off_x, ly = y - o.in_off_y;
  if (x >= xend || y >= h || lx < 0 || lx >= o.out_w || ly < 0 || ly >= o.out_h) return false;
  i = (size_t)(ly + o.out_y) * o.img_w + lx + o.out_x;
  return true;
}

template <int R>
__device__ __forceinline__ void image_alpha(float (&alpha)[R / 4], const OutputPass& o, int h, int g,
                                            int yb, int x, int xend) {
#pragma unroll
  for (int k = 0; k < R / 4; ++k) {
    size_t i;
    alpha[k] = image_index<R>(o, h, g, k, yb, x, xend, i) ? o.color[i].w : 0.f;
  }
}

template <int R>
__device__ __forceinline__ void store_image(const floatx4 (&acc)[R][1], const float (&alpha)[R / 4],
                                            const OutputPass& o, const float* bias, int h, int g,
                                            int yb, int x, int xend, int relu) {
  static_assert(R % 4 == 0, "rows are spread over the four lane groups");
  const float b0 = bias[4 * g], b1 = bias[4 * g + 1], b2 = bias[4 * g + 2];
#pragma unroll
  for (int k = 0; k < R / 4; ++k) {
    // row g + 4 k of this lane's column, chosen by selects (a loop of
    // conditional copies becomes a dynamic index into acc, i.e. scratch)
    const floatx4 v = g == 0 ? acc[4 * k][0] : g == 1 ? acc[4 * k + 1][0]
                    : g == 2 ? acc[4 * k + 2][0] : acc[4 * k + 3][0];
    size_t i;
    if (!image_index<R>(o, h, g, k, yb, x, xend, i)) continue;
    o.out[i] = output_pixel(act(v[0] + b0, relu), act(v[1] + b1, relu), act(v[2] + b2, relu),
                            alpha[k], o.hdr, o.input_scale);
  }
}

// IN: a PairIn (convA reads packed fp16, the tap-packed network input, or
// the images through the fused input pass, with or without taps).
// OUT: a PairOut (convB's result as fp16, fp32, or through the output pass).
template <int CGA, int NFB, int OUT, int IN, bool BF>
__device__ __forceinline__ void conv3x3_pair_body(const PairArgs& __restrict__ p, int pool, int relu) {
  constexpr bool TAP = (IN & kPairInTaps) != 0, IMG = (IN & kPairInImages) != 0;
  static_assert(!TAP || CGA == 2, "tap chunks are 16-lane sources");
  static_assert(!IMG || CGA == 2, "the input pass writes one 16-lane chunk");
  static_assert(OUT != kPairImage || NFB == 1, "the output pass reads one fragment");
  constexpr bool MSW = CGA == 4 || IMG;           // swizzled intermediate
  using L = PairLds<CGA, MSW>;
  constexpr bool WL = L::SW;                      // weights in LDS, swizzled layouts
  __shared__ __attribute__((aligned(16))) _Float16 lds[L::ZERO + 8];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;
  const int cf = wave & 1, rh = wave >> 1;        // column fragment, row half

  // A packed source was written by the previous launch in ascending tile
  // (and batch) order; walking the tiles in descending order reads the most
  // recently written lines first, while the memory-side cache still holds
  // them (dec_conv1a's 267 MB output at 1080p exceeds that cache).  Block b
  // still runs on XCD b mod 8 and walks one contiguous band of tiles.
  constexpr bool REV = !IMG;
  const int bx = REV ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
  int tx, ty;
  if (!tile_of_block(bx, p.tiles_x, p.tiles_y, tx, ty)) return;
  const int y0 = ty * PAIR_TH, x0 = tx * PAIR_TW;
  if (tid < 2) reinterpret_cast<uint2*>(lds + L::ZERO)[tid] = make_uint2(0u, 0u);
  constexpr int RB = PAIR_TH / 2;                 // convB rows per wave
  const int xend = x0 + PAIR_TW < p.w ? x0 + PAIR_TW : p.w;
  // this tile of the batch: activations at its offset, its image rectangle
  const int bt = REV ? (int)gridDim.z - 1 - (int)blockIdx.z : (int)blockIdx.z;
  const size_t boff = (size_t)bt * p.bstride;
  OutputPass img = p.img;
  if constexpr (OUT == kPairImage) {
    const TileRect& t = p.rect[bt];
    img.in_off_x = t.out_x - t.in_x;
    img.in_off_y = t.out_y - t.in_y;
    img.out_x = t.out_x;
    img.out_y = t.out_y;
    img.out_w = t.out_w;
    img.out_h = t.out_h;
  }
  float alpha[OUT == kPairImage ? RB / 4 : 1];
  if constexpr (OUT == kPairImage)
    image_alpha<RB>(alpha, img, p.h, g, y0 + RB * rh, x0 + 16 * cf + c, xend);

  // convA's biases for this lane: lane group g of the pair of fragments owns
  // channels 8 g .. 8 g + 7 (one 16-byte slot of the intermediate).  Read
  // up front with staged weights (see below); else after convA, where the
  // registers are free (three workgroups per CU leave no room during it).
  float bA[8];
  auto load_bias = [&] {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bA[i] = p.biasA[8 * g + i];
      bA[4 + i] = p.biasA[8 * g + 4 + i];
    }
  };
  if constexpr (WL) load_bias();
  // convA: intermediate rows [9 rh, 9 rh + 9), columns [16 cf, 16 cf + 16)
  // of the window at (y0 - 1, x0 - 1); both fragments of the 32 channels.
  constexpr int RA = PAIR_MH / 2;
  floatx4 acc[RA][2];
#pragma unroll
  for (int r = 0; r < RA; ++r) acc[r][0] = acc[r][1] = floatx4{0.f, 0.f, 0.f, 0.f};
  {
    const uint4* wf = static_cast<const uint4*>(p.wA) + lane;
    uint4 acur[3][2];
    auto load_a = [&] {
#pragma unroll
      for (int ky = 0; ky < 3; ++ky)
#pragma unroll
        for (int q = 0; q < 2; ++q) acur[ky][q] = wf[(ky * 2 + q) * 64];
    };
    // (with the input pass the image registers come first)
    if constexpr (!WL && !IMG) load_a();
    const _Float16* src = reinterpret_cast<const _Float16*>(static_cast<const char*>(p.x) + boff);
    const uint4* wl = reinterpret_cast<const uint4*>(lds + L::WOFF) + lane;
    if constexpr (IMG) {
      // one chunk: straight-line code (in the chunk loop the compiler keeps
      // the staging's addresses live across it and spills them)
      PackArgs in = p.in;
      in.tile_x = p.rect[bt].in_x;
      in.tile_y = p.rect[bt].in_y;
      in.packed = static_cast<char*>(in.packed) + boff;
      stage_pair_images<TAP, BF>(reinterpret_cast<uint4*>(lds), in, p.h, p.w, y0, x0, tid);
      load_a();
      __syncthreads();
      mma_chunk<2, RA, CGA, true, PAIR_PW, false, TAP, BF>(acc, acur, lds, 0, L::ZERO, wf, nullptr, 2,
                                                       RA * rh, 16 * cf, g, c, [] {});
    }
#pragma unroll 1
    for (int ci = 0; ci < (IMG ? 0 : p.nchunks); ++ci) {
      __syncthreads();
      stage_pair_input<CGA, WL>(reinterpret_cast<uint4*>(lds), src, p.cs, ci * kChunkChannels,
                                p.h, p.w, y0, x0, wave, lane);
      const uint4* wchunk = wf + (size_t)p.wfragA[ci] * 64;
      if constexpr (WL) stage_weights<(3 * CGA + 3) / 4 * 3 * 2>(lds + L::WOFF, wchunk, 2, 2, wave);
      __syncthreads();
      if constexpr (WL) {
        mma_chunk<2, RA, CGA, false, PAIR_PW, true, false, BF>(acc, acur, lds, 0, L::ZERO, wl, nullptr, 2,
                                                    RA * rh, 16 * cf, g, c, [] {});
      } else {
        const uint4* wnext = ci + 1 < p.nchunks ? wf + (size_t)p.wfragA[ci + 1] * 64 : nullptr;
        mma_chunk<2, RA, CGA, true, PAIR_PW, false, TAP, BF>(acc, acur, lds, 0, L::ZERO, wchunk, wnext,
                                                         2, RA * rh, 16 * cf, g, c, [] {});
      }
    }
  }
  // bias, ReLU, fp16; zero outside the image (see bA above).  convB's weight
  // copy goes out through inline assembly, so no wait for it lands before
  // the intermediate is written; the barrier before convB waits for it.
  // The empty asm consumes the biases first: the compiler's wait for them
  // (which, not knowing the copy, would be a full drain) lands here, long
  // after they arrived.
  if constexpr (WL)
    asm volatile("" ::"v"(bA[0]), "v"(bA[1]), "v"(bA[2]), "v"(bA[3]), "v"(bA[4]), "v"(bA[5]),
                 "v"(bA[6]), "v"(bA[7]));
  else
    load_bias();
  __syncthreads();   // every wave is done with the input patch (and convA's weights)
  if constexpr (WL)
    stage_weights<9 * NFB, true>(lds + L::WOFF, static_cast<const uint4*>(p.wB) + lane, NFB, NFB,
                                 wave);
  {
    const int x = x0 - 1 + 16 * cf + c;
#pragma unroll
    for (int r = 0; r < RA; ++r) {
      const int y = y0 - 1 + RA * rh + r;
      const bool inside = y >= 0 && y < p.h && x >= 0 && x < p.w;
      uint4 v;
      uint32_t* wv = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i0 = 2 * k, i1 = 2 * k + 1;
        const float f0 = (i0 < 4 ? acc[r][0][i0] : acc[r][1][i0 - 4]) + bA[i0];
        const float f1 = (i1 < 4 ? acc[r][0][i1] : acc[r][1][i1 - 4]) + bA[i1];
        // mask, not a conditional: the compiler branches around the conversion
        wv[k] = pack2<BF>(fmaxf(f0, 0.f), fmaxf(f1, 0.f)) & (0u - (uint32_t)inside);
      }
      const int col = 16 * cf + c;
      const int px = (RA * rh + r) * PAIR_PW + col;
      *reinterpret_cast<uint4*>(lds + px * pstride<4, MSW>() + 8 * gslot<4, MSW>(col, g)) = v;
    }
  }
  if constexpr (WL) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // convB's weight copy
  __syncthreads();
  // convB: output rows [8 rh, 8 rh + 8), columns [16 cf, 16 cf + 16).
  floatx4 accb[RB][NFB];
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int q = 0; q < NFB; ++q) accb[r][q] = floatx4{0.f, 0.f, 0.f, 0.f};
  {
    const uint4* wf = static_cast<const uint4*>(p.wB) + lane;
    uint4 acur[3][NFB];
    if constexpr (WL) {
      const uint4* wl = reinterpret_cast<const uint4*>(lds + L::WOFF) + lane;
      mma_chunk<NFB, RB, 4, false, PAIR_PW, true, false, BF>(accb, acur, lds, 0, L::ZERO, wl, nullptr, NFB,
                                                  RB * rh, 16 * cf, g, c, [] {});
    } else {
#pragma unroll
      for (int ky = 0; ky < 3; ++ky)
#pragma unroll
        for (int q = 0; q < NFB; ++q) acur[ky][q] = wf[(ky * NFB + q) * 64];
      mma_chunk<NFB, RB, 4, true, PAIR_PW, MSW, false, BF>(accb, acur, lds, 0, L::ZERO, wf, nullptr, NFB, RB * rh,
                                           16 * cf, g, c, [] {});
    }
  }
  if constexpr (OUT == kPairImage) {
    store_image<RB>(accb, alpha, img, p.biasB, p.h, g, y0 + RB * rh, x0 + 16 * cf + c, xend, relu);
  } else {
    ConvF16Args a{};
    a.h = p.h;
    a.w = p.w;
    a.bias = p.biasB;
    a.y = nullptr;
    a.cout_stored = p.cout_stored;
    a.nf = NFB;
    store_tile<NFB, RB, OUT == kPairF32, BF>(accb, a, static_cast<char*>(p.y) + boff, 0, g,
                                         y0 + RB * rh, x0 + 16 * cf + c, c, pool,
                                         relu, xend);
  }
}

// The kernels: fp16 and bf16 storage.
template <int CGA, int NFB, int OUT, int IN>
__global__ __launch_bounds__(THREADS, (kPairWaves<CGA, IN>)) void conv3x3_pair_f16(PairArgs p, int pool,
                                                                                  int relu) {
  conv3x3_pair_body<CGA, NFB, OUT, IN, false>(p, pool, relu);
}
template <int CGA, int NFB, int OUT, int IN>
__global__ __launch_bounds__(THREADS, (kPairWaves<CGA, IN>)) void conv3x3_pair_bf16(PairArgs p, int pool,
                                                                                   int relu) {
  conv3x3_pair_body<CGA, NFB, OUT, IN, true>(p, pool, relu);
}

template <int CGA, int NFB, int OUT, int IN, bool BF>
void launch_pair_kernel(const PairArgs& p, dim3 grid, bool pool, bool relu, hipStream_t stream) {
  if constexpr (BF)
    hipLaunchKernelGGL((conv3x3_pair_bf16<CGA, NFB, OUT, IN>), grid, dim3(THREADS), 0, stream, p,
                       (int)pool, (int)relu);
  else
    hipLaunchKernelGGL((conv3x3_pair_f16<CGA, NFB, OUT, IN>), grid, dim3(THREADS), 0, stream, p,
                       (int)pool, (int)relu);
}

template <int CGA, int NFB, int IN, bool BF>
hipError_t launch_pair_shape(PairArgs p, bool pool, bool relu, int out, hipStream_t stream) {
  p.tiles_x = cdiv(p.w, PAIR_TW);
  p.tiles_y = cdiv(p.h, PAIR_TH);
  const dim3 grid(cdiv(p.tiles_x * p.tiles_y, kXcds) * kXcds, 1, p.batch > 1 ? p.batch : 1);
  if (out == kPairF32) {
    launch_pair_kernel<CGA, NFB, kPairF32, IN, BF>(p, grid, pool, relu, stream);
  } else if (out == kPairF16) {
    launch_pair_kernel<CGA, NFB, kPairF16, IN, BF>(p, grid, pool, relu, stream);
  } else {
    // the network's last pair only: 64 -> 32 -> one fragment, no pool
    if constexpr (CGA == 4 && NFB == 1 && IN == kPairInPacked) {
      if (out != kPairImage || pool || !p.img.color || !p.img.out) return hipErrorInvalidValue;
      launch_pair_kernel<CGA, NFB, kPairImage, IN, BF>(p, grid, pool, relu, stream);
    } else {
      return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <bool BF>
hipError_t launch_pair_typed(const PairArgs& p, int cga, int nfb, int in, bool pool, bool relu,
                             int out, hipStream_t stream) {
  if (in & kPairInImages) {
    // the network's first pair: 16-lane input chunk, 32 -> 32 (pool)
    if (cga != 2 || nfb != 2 || !p.in.color || !p.in.packed) return hipErrorInvalidValue;
    if (in == kPairInImages)
      return launch_pair_shape<2, 2, kPairInImages, BF>(p, pool, relu, out, stream);
    if (in == (kPairInImages | kPairInTaps))
      return launch_pair_shape<2, 2, kPairInImages | kPairInTaps, BF>(p, pool, relu, out, stream);
    return hipErrorInvalidValue;
  }
  if (in == kPairInTaps) {
    if (cga == 2 && nfb == 2) return launch_pair_shape<2, 2, kPairInTaps, BF>(p, pool, relu, out, stream);
    if (cga == 2 && nfb == 1) return launch_pair_shape<2, 1, kPairInTaps, BF>(p, pool, relu, out, stream);
    return hipErrorInvalidValue;
  }
  if (in != kPairInPacked) return hipErrorInvalidValue;
  if (cga == 2 && nfb == 2) return launch_pair_shape<2, 2, kPairInPacked, BF>(p, pool, relu, out, stream);
  if (cga == 2 && nfb == 1) return launch_pair_shape<2, 1, kPairInPacked, BF>(p, pool, relu, out, stream);
  if (cga == 4 && nfb == 2) return launch_pair_shape<4, 2, kPairInPacked, BF>(p, pool, relu, out, stream);
  if (cga == 4 && nfb == 1) return launch_pair_shape<4, 1, kPairInPacked, BF>(p, pool, relu, out, stream);
  return hipErrorInvalidValue;
}

// The instances the planner can choose (see kPlanCandidates).
#define OIDN_PLAN_INSTANCES(X) \
  X(1, 4, 4) X(1, 2, 4) X(1, 8, 2) X(1, 4, 2) X(1, 8, 1) X(2, 16, 2) X(2, 8, 2) X(2, 4, 2) \
  X(3, 8, 4) X(3, 4, 4) X(3, 2, 4) X(3, 8, 2) X(3, 4, 2) X(4, 8, 4) X(4, 8, 2) X(4, 4, 2)  \
  X(5, 4, 4) X(7, 4, 4)

hipError_t launch_plan(const ConvF16Args& a, const ConvPlan& P, int nsplit, bool upcat, bool pool,
                       bool relu, bool out_f32, bool bf16, hipStream_t stream) {
#define OIDN_TRY(NFW, R, WR)                                                                \
  if (P.nfw == NFW && P.rows == R && P.wr == WR)                                            \
    return launch_shape<NFW, R, WR>(a, nsplit, upcat, pool, relu, out_f32, bf16, stream);
  OIDN_PLAN_INSTANCES(OIDN_TRY)
#undef OIDN_TRY
  return hipErrorInvalidValue;
}

}  // namespace

// Work decomposition.  For each fragment count nf, candidate plans from the
// fewest workgroups per tile and the largest per-wave tiles (weights loaded
// by fewer waves, patch rows reused longer) to the most workgroups; the
// planner takes the first that gives at least kMinBlocks workgroups (about
// two per CU), else the one with the most.  The lists come from timing every
// plan at the UNet's layer shapes (each layer's kernel durations in a
// kernel trace, in the network and alone): large layers keep all fragments
// in one workgroup, small deep layers split the output channels.  For
// nf = 4 with four or more K chunks per tile, waves of four fragments win.
constexpr long kMinBlocks = 480;
// Tiles of a batched launch the count above takes in: at most 4.  Counting
// all of them (12 at 4K) lets plans through whose workgroups run long serial
// chains (dec_conv4a at 4K: 7 fragments x 5 chunks per workgroup, 114 vs
// 66 us); 3 to 8 measured alike.
constexpr int kPlanBatchCap = 4;
constexpr int kMaxCandidates = 4;
const ConvPlan kPlanCandidates[9][kMaxCandidates] = {
    {},
    {{4, 1, 4}, {2, 1, 4}},                                  // nf = 1
    {{8, 1, 2}, {4, 1, 2}, {2, 1, 4}},                       // nf = 2
    {{8, 3, 4}, {4, 3, 4}, {2, 3, 4}, {2, 1, 4}},            // nf = 3
    {{16, 2, 2}, {8, 2, 2}, {8, 1, 1}, {2, 1, 4}},           // nf = 4, up to 3 chunks
    {{4, 5, 4}, {2, 1, 4}},                                  // nf = 5
    {{8, 3, 2}, {4, 3, 2}, {4, 1, 2}, {2, 1, 4}},            // nf = 6
    {{4, 7, 4}, {4, 1, 4}, {2, 1, 4}},                       // nf = 7
    {{8, 4, 2}, {4, 4, 2}, {4, 2, 2}, {2, 1, 4}},            // nf = 8
};
const ConvPlan kPlanManyChunks[kMaxCandidates] = {{8, 4, 4}, {8, 2, 2}, {8, 1, 1}, {2, 1, 4}};

const ConvPlan* plan_candidates(int nf, int nchunks, int nup) {
  if (nf == 4 && (nup > 0 || nchunks >= 4)) return kPlanManyChunks;
  return kPlanCandidates[nf < 1 ? 1 : nf > 8 ? 8 : nf];
}

long plan_blocks(int h, int w, int nf, const ConvPlan& P) {
  const int frags = P.nfw * (4 / P.wr);
  return (long)cdiv(cdiv(w, TW) * cdiv(h, P.wr * P.rows), kXcds) * kXcds * (nf / frags);
}

ConvPlan conv_f16_plan(int h, int w, int nf, int nchunks, int nup, int batch) {
  ConvPlan best{};
  long most = -1;
  const ConvPlan* cand = plan_candidates(nf, nchunks, nup);
  for (int i = 0; i < kMaxCandidates; ++i) {
    const ConvPlan& P = cand[i];
    if (P.rows == 0) break;
    const long b = plan_blocks(h, w, nf, P) * (batch > kPlanBatchCap ? kPlanBatchCap
                                                : batch > 1 ? batch : 1);
    if (b >= kMinBlocks) return P;
    if (b > most) {
      most = b;
      best = P;
    }
  }
  return best;
}

// Fragments one workgroup computes.
int plan_block_frags(const ConvPlan& P) { return P.nfw * (4 / P.wr); }

// Workgroups of the launch (for reporting).
int conv_f16_blocks(int h, int w, int nf, int nchunks, int nup, int batch) {
  return (int)plan_blocks(h, w, nf, conv_f16_plan(h, w, nf, nchunks, nup, batch)) *
         (batch > 1 ? batch : 1);
}

bool conv_f16_layout(int cin0_stored, int cin1_stored, int cout, ConvLayout* out,
                     int tap_src) {
  ConvLayout L{};
  L.nf = cdiv(stored_channels(cout), 16);
  if (L.nf < 1 || L.nf > 8) return false;
  // a tap chunk is the last source's only chunk: 12 or 16 stored channels
  const int last_src = cin1_stored > 0 ? 1 : 0;
  if (tap_src >= 0) {
    const int st = last_src ? cin1_stored : cin0_stored;
    if (tap_src != last_src || st < 12 || st > 16) return false;
  }
  // Chunks of up to 32 channels, sources in order, channels in order; a chunk
  // is processed as 4 groups of 8 channels if it holds more than 16, else as
  // 2 (missing channels are zero).  With two sources the first is the
  // upsampled one.  Only a source's last chunk can be a 2-group chunk, so the
  // order is: upsampled 4-group, upsampled 2-group, plain 4-group, plain
  // 2-group, tap -- the kernel's five loops.
  const bool two = cin1_stored > 0;
  const int cs[2] = {cin0_stored, cin1_stored};
  int frag = 0, n = 0;
  for (int s = 0; s < 2; ++s)
    for (int off = 0; off < cs[s]; off += kChunkChannels) {
      if (n >= kMaxChunks) return false;
      const int rem = cs[s] - off < kChunkChannels ? cs[s] - off : kChunkChannels;
      ConvChunk& ch = L.chunk[n++];
      ch.src = s;
      ch.coff = off;
      ch.cg = rem > 16 ? 4 : 2;
      ch.ncg = s == tap_src ? 1 : cdiv(3 * ch.cg, 4);
      ch.wfrag = frag;
      const bool up = two && s == 0;
      frag += ch.ncg * (up ? 4 : 3) * L.nf;   // an upsampled chunk has 4 row combinations
      if (up && ch.cg == 4) ++L.nup4;
      if (up) ++L.nup;
      if (!up && ch.cg == 4) ++L.npl4;
      if (s == tap_src) ++L.ntap;
    }
  L.nchunks = n;
  L.total_frags = frag;
  L.bias_bytes = align256(sizeof(float) * 16 * L.nf);
  L.bytes = L.bias_bytes + (size_t)frag * kFragBytes;
  *out = L;
  return true;
}

void conv_f16_describe(const ConvF16Args& a, int nf, bool out_f32, bool bf16, char* buf, int cap,
                       int* blocks) {
  const int h = a.h, w = a.w;
  const ConvPlan P = conv_f16_plan(h, w, nf, a.nchunks, a.nup, a.batch);
  if (OIDN_WS_ENABLE && !out_f32 && P.nfw == 4 && P.rows == 8 && P.wr == 4) {
    ConvF16Args b = a;
    b.nf = nf;
    if (ws_lds_bytes<4, 8, 4>(b) > 0) {
      const int nsplit = nf / plan_block_frags(P);
      snprintf(buf, cap, "conv3x3_ws_%s<4, 8, 4, %s>", bf16 ? "bf16" : "f16", out_f32 ? "true" : "false");
      *blocks = ws_grid_x(cdiv(cdiv(w, TW) * cdiv(h, 4 * 8), kXcds) * kXcds, a.batch, nsplit) * nsplit;
      return;
    }
  }
  snprintf(buf, cap, "conv3x3_%s_mfma<%d, %d, %d, %s>", bf16 ? "bf16" : "f16", P.nfw, P.rows, P.wr,
           out_f32 ? "true" : "false");
  *blocks = conv_f16_blocks(h, w, nf, a.nchunks, a.nup, a.batch);
}

hipError_t launch_conv_f16(const ConvF16Args& a, int nf, bool upcat, bool pool, bool relu,
                           bool out_f32, bool bf16, hipStream_t stream) {
  if (a.batch > 65535) return hipErrorInvalidValue;
  ConvF16Args b = a;
  b.nf = nf;
  const ConvPlan P = conv_f16_plan(a.h, a.w, nf, a.nchunks, a.nup, a.batch);
  const int nsplit = nf / plan_block_frags(P);
  return launch_plan(b, P, nsplit, upcat, pool, relu, out_f32, bf16, stream);
}

hipError_t launch_conv_pair_f16(const PairArgs& p, int cga, int nfb, int in, bool pool,
                                bool relu, int out, bool bf16, hipStream_t stream) {
  if (p.batch > kMaxBatch) return hipErrorInvalidValue;
  return bf16 ? launch_pair_typed<true>(p, cga, nfb, in, pool, relu, out, stream)
              : launch_pair_typed<false>(p, cga, nfb, in, pool, relu, out, stream);
}

int conv_pair_blocks(int h, int w) {
  return cdiv(cdiv(w, PAIR_TW) * cdiv(h, PAIR_TH), kXcds) * kXcds;
}

}  // namespace oidn
