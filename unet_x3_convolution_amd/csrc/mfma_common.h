// Device helpers shared by the fp16 / bf16 MFMA convolution kernels: operand
// types, the MFMA call, the LDS patch layouts, the direct global -> LDS
// load and the XCD-aware tile order.
#pragma once

#include "internal.h"

namespace oidn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Activations and weights are stored as fp16 or (BF) bf16, both rounded to
// nearest even from fp32; the matching MFMA multiplies them with fp32
// accumulate.  Operands travel as raw 16-byte groups of 8 values.
template <bool BF>
__device__ __forceinline__ floatx4 mfma16(uint4 a, uint4 b, floatx4 c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                   __builtin_bit_cast(half8, b), c, 0, 0, 0);
}


constexpr int TW = 16;                        // tile width (one B fragment)
constexpr int PW = TW + 2;                    // patch width
constexpr int PSTR = 40;                      // halves per patch pixel: 32 + 8 pad (80 B)
// Two patch layouts.  Padded (SW false): a chunk of CG channel groups takes
// 4 groups -> 5 slots (80 B), 2 groups -> 3 slots (48 B) per pixel; the odd
// stride keeps 16 consecutive pixels of a fragment read on distinct LDS
// banks.  Swizzled (SW true): no pad (64 B / 32 B per pixel); channel group
// grp of the pixel in patch column col sits in slot gslot(col, grp), the
// group index XOR column bits, which spreads the same 16-pixel reads over 16
// distinct 16-byte bank groups in 4/5 (CG 4) or 2/3 (CG 2) of the space.
template <int CG, bool SW = false>
constexpr int pstride() { return SW ? 8 * CG : CG == 4 ? PSTR : 24; }
template <int CG, bool SW>
__device__ __forceinline__ int gslot(int col, int grp) {
  if constexpr (!SW) return grp;
  else return CG == 4 ? grp ^ ((col >> 2) & 3) : grp ^ ((col >> 3) & 1);
}
constexpr int THREADS = 256;
constexpr int kXcds = 8;

constexpr int LPW = TW / 2 + 2;               // half-resolution patch width

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int TH_, bool SW = false>
struct Tile {
  static constexpr int TH = TH_;                // tile height (rows)
  static constexpr int PH = TH + 2;
  static constexpr int LPH = TH / 2 + 2;        // half-resolution patch height
  // The patch occupies whole 64-slot (1 KB) blocks so that direct
  // global -> LDS loads, which fill 64 consecutive 16-byte slots each, stay
  // inside it.
  static constexpr int PATCH = (PH * PW * pstride<4, SW>() + 511) / 512 * 512;   // halves
};

// One direct global -> LDS load: 16 bytes per lane, lane i filling the
// 16-byte slot i from `lds` (wave-uniform).  ASM issues it through inline
// assembly: the compiler then tracks no LDS write for it and adds no wait
// for it before later memory operations, so the caller must wait (vmcnt)
// before reading what it copies.  M0 is set right before the load (the
// compiler sets M0 itself before each of its own uses).
template <bool ASM>
__device__ __forceinline__ void dma16(const void* gp, uint4* lds) {
  if constexpr (ASM) {
    const unsigned m0 = __builtin_amdgcn_readfirstlane(
        (unsigned)(unsigned long)(__attribute__((address_space(3))) void*)lds);
    // an SALU write of M0 needs one wait state before a load that uses it
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0),
                 "v"(gp)
                 : "memory");
  } else {
    __builtin_amdgcn_global_load_lds(gp, lds, 16, 0, 0);
  }
}

// Zero block that padding lanes of the direct patch loads read from.
__device__ __attribute__((aligned(16))) unsigned int g_zero16[4] = {0u, 0u, 0u, 0u};


// Tile order.  Tiles are walked in super-tiles of kSuperW x kSuperH tiles
// (row-major inside a super-tile, super-tiles row-major), and XCD x takes
// the x-th contiguous eighth of that order; block b runs on XCD b % 8.  The
// 64 or so workgroups an XCD runs at once then cover a near-square patch of
// the image, so halo rows and columns shared by neighbouring tiles are
// fetched into that XCD's L2 once.  Returns false for the padding blocks
// past the last tile.
constexpr int kSuperW = 8, kSuperH = 8;
// Tile of linear index t in that order (t < tiles_x * tiles_y).
__device__ __forceinline__ void tile_at(int t, int tiles_x, int tiles_y, int& tx, int& ty) {
  const int row0 = t / (kSuperH * tiles_x) * kSuperH;    // first tile row of the super-row
  const int sh = min(kSuperH, tiles_y - row0);            // its rows
  const int u = t - row0 * tiles_x;                       // index inside the super-row
  const int col0 = u / (sh * kSuperW) * kSuperW;          // first tile column of the super-tile
  const int sw = min(kSuperW, tiles_x - col0);            // its columns
  const int v = u - col0 * sh;                            // index inside the super-tile
  ty = row0 + v / sw;
  tx = col0 + v - (v / sw) * sw;
}

__device__ __forceinline__ bool tile_of_block(int b, int tiles_x, int tiles_y, int& tx, int& ty) {
  const int ntiles = tiles_x * tiles_y;
  const int per = (ntiles + kXcds - 1) / kXcds;
  const int t = (b % kXcds) * per + b / kXcds;
  if (t >= ntiles) return false;
  tile_at(t, tiles_x, tiles_y, tx, ty);
  return true;
}

__device__ __forceinline__ float act(float v, int relu) { return relu ? fmaxf(v, 0.f) : v; }

__device__ __forceinline__ float swap_pair(float v) {
  // DPP quad_perm [1, 0, 3, 2]: exchange with the neighbouring lane.
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

}  // namespace
}  // namespace oidn
