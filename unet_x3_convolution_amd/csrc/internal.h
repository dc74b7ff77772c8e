// Internal declarations shared by the host C-ABI code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "oidn_mi355x.h"

namespace oidn {

constexpr int kMaxChunks = 20;        // 32-channel K chunks per conv (two sources)
constexpr int kChunkChannels = 32;    // channels of one LDS-staged K chunk
constexpr int kFragBytes = 1024;      // one 16x32 fp16 MFMA operand fragment (64 lanes x 16 B)

inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline int stored_channels(int c) { return 4 * cdiv(c, 4); }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// ---------------------------------------------------------------------------
// fp16 MFMA implicit-GEMM conv.
//
// K runs over (input chunk of <= 32 stored channels of one source) x (column
// group) x (ky).  Inside a chunk of cg 8-channel groups the 3 * cg
// (kx, group) "slots" are dealt four at a time (slot = kx * cg + group) to
// the four 16-lane groups of an MFMA operand; such a set of four slots is a
// column group (ncg = ceil(3 * cg / 4) per chunk), and each column group is
// repeated for ky = 0, 1, 2.  Because every lane of one column group reads
// the same patch row, one B fragment loaded from LDS serves three output
// rows (one per ky).
// ---------------------------------------------------------------------------
struct ConvChunk {
  int src;    // 0: first source (upsampled source for the decoder), 1: skip
  int coff;   // first stored channel of the chunk within its source
  int cg;     // 8-channel groups the chunk is processed as (2 or 4)
  int ncg;    // column groups of the chunk: ceil(3 * cg / 4), 1 for a tap chunk
  int wfrag;  // index of the chunk's first weight fragment
};

// Weight fragment of (chunk, column group j, row set t, output fragment q):
//   chunk.wfrag + (j * T + t) * nf + q
// with T = 3 row sets, the ky rows, for a plain source and T = 4 for the
// nearest-2x-upsampled source: the row combinations W0, W1 + W2, W0 + W1,
// W2 (an output row of parity 0 reads low-resolution rows Y - 1, Y with the
// first two, one of parity 1 reads Y, Y + 1 with the last two).
// 64 lanes x 8 halves; lane l holds output row r = l % 16 and slot
// 4 * j + l / 16 of the chunk.  Slot s is (kx, group) = (s / cg, s % cg),
// channels coff + 8 * group + 0..7 of the pixel in column x + kx - 1.
//
// Tap chunk (a 9-channel source stored in 16 lanes whose lanes 8, 9, 10 hold
// channel 8 of the pixels in columns x - 1, x, x + 1, zero past the image
// edge -- the packed network input): one column group, slots 0..2 are
// (kx, group 0) = channels 0..7, slot 3 is group 1 of the centre pixel, whose
// lanes 0..2 carry the weights of channel 8 for kx = 0, 1, 2.  The chunk
// takes 3 MFMA K-steps per output instead of 6.
struct ConvLayout {           // shared by the weight packer and the launcher
  int nf;                     // 16-row output-channel fragments (N = 16 * nf)
  int nchunks;
  int nup4, nup;               // upsampled-source chunks (4-group ones, all)
  int npl4;                    // plain-source 4-group chunks
  int ntap;                    // tap chunks (the last ones; 0 or 1)
  int total_frags;
  ConvChunk chunk[kMaxChunks];
  size_t bias_bytes;          // fp32 bias, 16 * nf floats, 256-aligned
  size_t bytes;               // bias + fragments
};

// Computes the fp16 layout; returns false if the shape exceeds the limits.
// tap_src (0 or 1, the last source, stored as 12 or 16 channels of which 9
// are data): that source is one tap chunk; -1: none.
bool conv_f16_layout(int cin0_stored, int cin1_stored, int cout, ConvLayout* out,
                     int tap_src = -1);

// Output fragments go in pairs (2p, 2p + 1) that cover the 32 channels
// [32 p, 32 p + 32).  Row r (0..15) of fragment q holds output channel
//   32 (q / 2) + 8 (r / 4) + 4 (q % 2) + r % 4   if q is in a full pair,
//   32 (q / 2) + r                                for the last fragment of an odd nf,
// so that the 16-lane group g of a pair's two accumulators owns 8
// consecutive channels: one 16-byte store per lane, 64 contiguous bytes
// per pixel per store instruction.
inline bool frag_paired(int nf, int q) { return (q | 1) < nf; }
inline int frag_row_to_cout(int nf, int q, int r) {
  return 32 * (q / 2) + (frag_paired(nf, q) ? 8 * (r / 4) + 4 * (q % 2) + r % 4 : r);
}

struct ConvF16Args {
  const void* src0;   // fp16, h x w (or h/2 x w/2 when upsampled) x cs0
  const void* src1;   // fp16, h x w x cs1 (skip), may be null
  int cs0, cs1;       // stored channels per source
  int h, w;           // conv input == output size before pooling
  const float* bias;  // 16 * nf floats
  const void* wfrag;  // fragments
  void* y;
  int cout_stored;
  int nf;             // output fragments of the whole conv
  int tiles_x, tiles_y;
  int grid_x;         // tile slots along grid x (tiles rounded up to a multiple of 8)
  int ws_pslot;       // patch slot (halves) of the weight-stationary form
  int nchunks;
  int nup4, nup, npl4;   // chunk ranges of the kernel's loops (see ConvLayout)
  int ntap;
  int batch;          // tiles in the launch (grid z), >= 1
  size_t bstride;     // bytes between tiles for src0, src1 and y (0 if batch == 1)
  ConvChunk chunk[kMaxChunks];
};

// bf16: the 16-bit storage is bf16 (conv3x3_bf16_mfma), else fp16.
hipError_t launch_conv_f16(const ConvF16Args& a, int nf, bool upcat, bool pool, bool relu,
                           bool out_f32, bool bf16, hipStream_t stream);

// Launch plan of a conv: a workgroup of 4 waves covers a (wr * rows) x 16
// tile; each wave computes `rows` rows of `nfw` output fragments, the waves
// forming wr row groups x (4 / wr) fragment groups; the nf fragments are
// split across nf / (nfw * 4 / wr) workgroups.
struct ConvPlan {
  int rows, nfw, wr;
};
// batch: tiles in the launch; the plan counts the whole launch's workgroups.
ConvPlan conv_f16_plan(int h, int w, int nf, int nchunks, int nup, int batch = 1);
int conv_f16_blocks(int h, int w, int nf, int nchunks, int nup, int batch = 1);

// Name of the kernel instance launch_conv_f16 would run for `a` (h, w,
// cs0, cs1 and the chunk fields set) and its grid.
void conv_f16_describe(const ConvF16Args& a, int nf, bool out_f32, bool bf16, char* buf, int cap,
                       int* blocks);

// Tiles of one size run through the network together: one launch per layer
// with the tile index in grid z, each tile's activations at its own byte
// offset (batch stride) in the workspace.
constexpr int kMaxBatch = 16;

// A tile's input window origin and output rectangle in the image.
struct TileRect {
  int in_x, in_y;
  int out_x, out_y, out_w, out_h;
};

// Output pass of one tile ([webgpu-0.6] outputShader): the network's pixel
// (y, x) in tile coordinates lands on image pixel (y - in_off_y + out_y,
// x - in_off_x + out_x) when 0 <= y - in_off_y < out_h and
// 0 <= x - in_off_x < out_w; RGB sanitized and (hdr) taken back through the
// transfer and the input scale, alpha copied from the input colour.
struct OutputPass {
  const float4* color;     // h x img_w RGBA float32 (alpha source)
  float4* out;             // h x img_w RGBA float32
  int img_w;
  int in_off_x, in_off_y;
  int out_x, out_y, out_w, out_h;
  int hdr;
  float input_scale;
};

// Fused pair y = convB(relu(convA(x))) through a 32-channel intermediate kept
// in LDS (both fp16 layouts as above; convA: one source whose stored channel
// count is a multiple of 8, all chunks of one kind; convB: 32 -> cout <= 32).
// convB's result goes to `y` as fp16 or fp32 (cout_stored lanes), or, for the
// network's last two layers, straight through the output pass into `img`.
enum PairOut { kPairF16 = 0, kPairF32 = 1, kPairImage = 2 };
// convA's source: packed fp16 (optionally the tap-packed network input), or
// the caller's images through the input pass run in convA's staging (bits).
enum PairIn { kPairInPacked = 0, kPairInTaps = 1, kPairInImages = 2 };
struct PackArgs {
  const float4* color;
  const float4* albedo;
  const float4* normal;
  int img_w, img_h;
  int tile_x, tile_y, tile_w, tile_h;
  int hdr;
  float input_scale;
  int sources;       // 1, 2 or 3
  int lanes;         // stored channels per output pixel (>= 4 * ceil(3 * sources / 4))
  int taps;          // fp16, 3 sources, 16 lanes: lanes 8..10 = channel 8 at x - 1, x, x + 1
  void* packed;
};

struct PairArgs {
  const void* x;           // fp16, h x w x cs
  int cs, h, w;
  int nchunks;             // convA chunks (<= 32 channels each, in order)
  int wfragA[8];           // first weight fragment of each convA chunk
  const float* biasA;      // 32 floats
  const void* wA;          // convA fragments (nf = 2)
  const float* biasB;      // 16 * nfB floats
  const void* wB;          // convB fragments (one 32-channel chunk)
  void* y;
  int cout_stored;
  int tiles_x, tiles_y;
  OutputPass img;          // out == kPairImage (cga 4, nfb 1, convB without ReLU)
  PackArgs in;             // in & kPairInImages (cga 2, nfb 2): x is not read, the
                           // packed tile is written to in.packed
  int batch;               // tiles in the launch (grid z), >= 1
  size_t bstride;          // bytes between tiles for x, y and in.packed
  TileRect rect[kMaxBatch];  // per tile: in.tile_x/y and img's rectangle (images only)
};
// in: PairIn bits (kPairInTaps: convA's one chunk is a tap chunk, cga 2);
// out: a PairOut.
hipError_t launch_conv_pair_f16(const PairArgs& p, int cga, int nfb, int in, bool pool,
                                bool relu, int out, bool bf16, hipStream_t stream);
int conv_pair_blocks(int h, int w);

// ---------------------------------------------------------------------------
// fp32 conv on the matrix cores.  Packed weights: bias (cout_stored floats,
// 256-aligned) then, per 16-channel output fragment, tap and 32-channel
// input chunk (stored channels over both sources), the 64 lanes' 8 values of
// the MFMA A operand (conv_f32_weight_index).
// ---------------------------------------------------------------------------
struct ConvF32Args {
  const float* src0;
  const float* src1;
  int cs0, cs1;
  int h, w;
  const float* bias;
  const float* wt;
  float* y;
  int cout_stored;
};

size_t conv_f32_bytes(int cin_stored_total, int cout);
int conv_f32_chunks(int cin_stored_total);
// Workgroups and kernel instance of the launch for an h x w conv input.
int conv_f32_blocks(int h, int w, int cout);
const char* conv_f32_kernel_name(int h, int w, int cout);
// Float index (after the bias) of the weight of output channel o, tap
// (3 ky + kx) and stored input channel c.
size_t conv_f32_weight_index(int o, int tap, int c, int cin_stored_total);
hipError_t launch_conv_f32(const ConvF32Args& a, bool upcat, bool pool, bool relu,
                           hipStream_t stream);

// ---------------------------------------------------------------------------
// Elementwise / gather passes.
// ---------------------------------------------------------------------------
// dtype: OIDN_F32, OIDN_F16 or OIDN_BF16 storage of the packed / pooled /
// concatenated tensors.
hipError_t launch_pack(const PackArgs& a, int dtype, hipStream_t stream);

struct UnpackArgs {
  const float4* net;       // tile of RGBA float32 network output, tile_w wide
  int tile_w;
  OutputPass o;
};
hipError_t launch_unpack(const UnpackArgs& a, hipStream_t stream);

hipError_t launch_pool(const void* x, int h, int w, int cs, void* y, int dtype, hipStream_t stream);
// b16: 16-bit storage (fp16 or bf16: a bit copy either way), else fp32.
hipError_t launch_upcat(const void* low, int cs_low, const void* skip, int cs_skip, int h, int w,
                        void* z, bool b16, hipStream_t stream);

// Measurement helper: independent MFMA streams with no memory traffic
// (calibrate.hip).  Work of a launch in FLOPs (2 per multiply-add).
hipError_t launch_mfma_stream(int bf16, long iters, int blocks, float* sink, hipStream_t stream);
long mfma_stream_flops(long iters, int blocks);
// Measurement helper: reads `bytes` (a multiple of 16) once.
hipError_t launch_read_stream(const void* p, size_t bytes, float* sink, hipStream_t stream);

// The end-to-end denoise (oidn_unet_forward's body) with as many tiles per
// launch as `ws_bytes` holds, at least one; bytes of one tile's workspace
// plan for that image.  Both set the thread-local error on failure.
int denoise_fit(const void* d_weights, int in_channels, const float* color, const float* albedo,
                const float* normal, int w, int h, int hdr, int transfer, float input_scale,
                int max_tile, int overlap, void* workspace, size_t ws_bytes, float* out_rgba,
                int dtype, hipStream_t stream);
int tile_workspace_bytes(int in_channels, int w, int h, int max_tile, int overlap, int dtype,
                         size_t* bytes);
int set_error(int code, const char* what);   // returns code
int clear_error();                            // returns OIDN_OK

}  // namespace oidn
