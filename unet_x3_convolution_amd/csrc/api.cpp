// Host side of the C ABI: argument validation and error reporting, the tile
// planner, weight packing, the liveness-planned UNet workspace and the
// per-tile launch sequence.  Every device step is one of the HIP kernels in
// this directory; nothing here computes on the host except packing weights.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/oidn_mi355x.h"
#include "internal.h"

using namespace oidn;

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int ok() {
  g_error.clear();
  return OIDN_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(OIDN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The input and output passes index pixels with 32-bit ints (and round the
// grid up to whole workgroups): rectangles above this many pixels are refused.
constexpr long long kMaxPassPixels = 2147483647LL - 1024;

int check_dtype(int dtype) {
  if (dtype == OIDN_F32 || dtype == OIDN_F16 || dtype == OIDN_BF16) return OIDN_OK;
  return fail(OIDN_E_INVALID, "unknown dtype %d", dtype);
}

size_t esize(int dtype) { return dtype == OIDN_F32 ? 4 : 2; }

// fp16 and bf16 storage run the same MFMA kernels (16-bit path).
bool b16(int dtype) { return dtype == OIDN_F16 || dtype == OIDN_BF16; }

// double -> bf16 bits, rounded to nearest even once (8 significant bits;
// subnormals below 2^-126 at a fixed 2^-133 step; overflow to infinity).
uint16_t bf16_bits(double v) {
  if (std::isnan(v)) return 0x7fc0;
  if (v == 0.0) return std::signbit(v) ? 0x8000 : 0x0000;
  int e = 0;
  std::frexp(v, &e);                       // |v| = m 2^e, 0.5 <= m < 1
  const int shift = e >= -125 ? 8 - e : 133;
  const double r = std::nearbyint(std::ldexp(v, shift));   // ties to even
  const float f = (float)std::ldexp(r, -shift);            // exact, or +-inf past the range
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

// One stored weight value: fp16 (rounded once from double) or bf16.
void put16(void* frag, size_t i, double v, int dtype) {
  if (dtype == OIDN_BF16) {
    static_cast<uint16_t*>(frag)[i] = bf16_bits(v);
  } else {
    static_cast<_Float16*>(frag)[i] = (_Float16)v;
  }
}

// ------------------------------------------------------------ tile planner
struct Span { int in0, in_size, out0, out_size; };

int align_up(int v, int a) { return (v + a - 1) / a * a; }

int plan_axis(int extent, int tile, int overlap, std::vector<Span>& out) {
  out.clear();
  const int ea = align_up(extent, OIDN_TILE_ALIGN);
  if (ea <= tile) {
    out.push_back({0, ea, 0, extent});
    return OIDN_OK;
  }
  const int step = tile - 2 * overlap;
  if (step <= 0) return fail(OIDN_E_INVALID, "tile size %d must exceed twice the overlap %d", tile, overlap);
  const int n = cdiv(extent, step);
  const int span = align_up(cdiv(extent, n), OIDN_TILE_ALIGN);
  const int size = span + 2 * overlap < ea ? span + 2 * overlap : ea;
  for (int i = 0; i < n; ++i) {
    const int o0 = i * span;
    if (o0 >= extent) break;
    const int o1 = o0 + span < extent ? o0 + span : extent;
    int lo = o0 - overlap > 0 ? o0 - overlap : 0;
    if (lo > ea - size) lo = ea - size;
    out.push_back({lo, size, o0, o1 - o0});
  }
  return OIDN_OK;
}

int plan(int w, int h, int max_tile, int overlap, std::vector<oidn_tile>& tiles) {
  if (w <= 0 || h <= 0) return fail(OIDN_E_INVALID, "image dimensions must be positive (got %dx%d)", w, h);
  if (w > 65536 || h > 65536) return fail(OIDN_E_INVALID, "image dimensions above 65536 are not supported");
  if (overlap < 0) overlap = OIDN_DEFAULT_OVERLAP;
  if (overlap % OIDN_TILE_ALIGN) return fail(OIDN_E_INVALID, "overlap %d is not a multiple of 16", overlap);
  if (max_tile < 0 || max_tile % OIDN_TILE_ALIGN)
    return fail(OIDN_E_INVALID, "max tile size %d must be 0 or a positive multiple of 16", max_tile);
  const int tile = max_tile > 0 ? max_tile : align_up(w > h ? w : h, OIDN_TILE_ALIGN);
  std::vector<Span> xs, ys;
  int rc = plan_axis(w, tile, overlap, xs);
  if (rc) return rc;
  rc = plan_axis(h, tile, overlap, ys);
  if (rc) return rc;
  tiles.clear();
  for (const Span& y : ys)
    for (const Span& x : xs)
      tiles.push_back({x.in0, y.in0, x.in_size, y.in_size, x.out0, y.out0, x.out_size, y.out_size});
  return OIDN_OK;
}

// ----------------------------------------------------------- conv helpers
int conv_weights_bytes(int cin0, int cin1, int cout, int dtype, size_t* bytes, int tap_src = -1) {
  int rc = check_dtype(dtype);
  if (rc) return rc;
  if (cin0 <= 0 || cin1 < 0 || cout <= 0)
    return fail(OIDN_E_INVALID, "channel counts must be positive (cin0=%d cin1=%d cout=%d)", cin0, cin1, cout);
  if (cin0 > OIDN_MAX_SOURCE_CHANNELS || cin1 > OIDN_MAX_SOURCE_CHANNELS || cout > OIDN_MAX_OUT_CHANNELS)
    return fail(OIDN_E_UNSUPPORTED, "channel counts above the limits (%d per source, %d out)",
                OIDN_MAX_SOURCE_CHANNELS, OIDN_MAX_OUT_CHANNELS);
  if (cin1 > 0 && cin0 % 4)
    return fail(OIDN_E_INVALID, "the upsampled source needs a multiple of 4 channels (got %d)", cin0);
  if (b16(dtype)) {
    ConvLayout L;
    if (!conv_f16_layout(stored_channels(cin0), cin1 ? stored_channels(cin1) : 0, cout, &L, tap_src))
      return fail(OIDN_E_UNSUPPORTED, "conv shape exceeds the fp16 kernel limits");
    *bytes = L.bytes;
  } else {
    *bytes = conv_f32_bytes(stored_channels(cin0) + (cin1 ? stored_channels(cin1) : 0), cout);
  }
  return OIDN_OK;
}

// Host-side packing into `out` (sized by conv_weights_bytes).  tap_src: the
// source packed as a tap chunk (16-bit storage only; see ConvChunk), -1 for
// none.  fp16 and bf16 share the layout.
void pack_conv_host(const float* w, const float* b, int cin0, int cin1, int cout, int dtype,
                    std::vector<unsigned char>& out, int tap_src = -1) {
  const int cin = cin0 + cin1;
  const int cs0 = stored_channels(cin0), cs1 = cin1 ? stored_channels(cin1) : 0;
  auto wat = [&](int o, int tap, int i) -> float {  // OHWI, logical channels
    return w[((size_t)o * 9 + tap) * cin + i];
  };
  // logical input channel of stored channel `c` of source `s`, or -1
  auto logical = [&](int s, int c) -> int {
    if (s == 0) return c < cin0 ? c : -1;
    return c < cin1 ? cin0 + c : -1;
  };
  std::fill(out.begin(), out.end(), 0);
  if (b16(dtype)) {
    ConvLayout L;
    conv_f16_layout(cs0, cs1, cout, &L, tap_src);
    float* bias = reinterpret_cast<float*>(out.data());
    for (int o = 0; o < cout; ++o) bias[o] = b[o];
    unsigned char* frag = out.data() + L.bias_bytes;
    // Upsampled-source chunks hold four row combinations a per column group
    // instead of the three ky rows: W0, W1 + W2, W0 + W1, W2 (the two rows
    // of the low-resolution source an even / odd output row reads), each sum
    // formed in double and rounded once to the storage type.
    static const int kCombo[4][2] = {{0, -1}, {1, 2}, {0, 1}, {2, -1}};
    for (int ci = 0; ci < L.nchunks; ++ci) {
      const ConvChunk& ch = L.chunk[ci];
      const bool up = ci < L.nup;
      const int rows = up ? 4 : 3;
      for (int j = 0; j < ch.ncg; ++j)
        for (int ky = 0; ky < rows; ++ky)
          for (int q = 0; q < L.nf; ++q) {
            unsigned char* f = frag + ((size_t)(ch.wfrag + (j * rows + ky) * L.nf + q)) * kFragBytes;
            for (int lane = 0; lane < 64; ++lane) {
              const int r = lane & 15, slot = 4 * j + (lane >> 4);
              const int o = frag_row_to_cout(L.nf, q, r);
              if (up) {
                if (o >= cout || slot >= 3 * ch.cg) continue;
                const int kx = slot / ch.cg, grp = slot % ch.cg;
                for (int jj = 0; jj < 8; ++jj) {
                  const int li = logical(ch.src, ch.coff + 8 * grp + jj);
                  if (li < 0) continue;
                  double v = wat(o, 3 * kCombo[ky][0] + kx, li);
                  if (kCombo[ky][1] >= 0) v += wat(o, 3 * kCombo[ky][1] + kx, li);
                  put16(f, lane * 8 + jj, v, dtype);
                }
                continue;
              }
              if (ch.src == tap_src) {
                // slots 0..2: channels 0..7 at kx = slot; slot 3: channel 8 at kx = lane 0..2
                if (o >= cout) continue;
                const int c8 = logical(ch.src, 8);
                for (int jj = 0; jj < 8; ++jj) {
                  const int li = slot < 3 ? logical(ch.src, jj) : jj < 3 ? c8 : -1;
                  const int kx = slot < 3 ? slot : jj;
                  if (li >= 0) put16(f, lane * 8 + jj, wat(o, 3 * ky + kx, li), dtype);
                }
                continue;
              }
              if (o >= cout || slot >= 3 * ch.cg) continue;
              const int kx = slot / ch.cg, grp = slot % ch.cg;
              const int tap = 3 * ky + kx;
              for (int jj = 0; jj < 8; ++jj) {
                const int li = logical(ch.src, ch.coff + 8 * grp + jj);
                if (li >= 0) put16(f, lane * 8 + jj, wat(o, tap, li), dtype);
              }
            }
          }
    }
  } else {
    const int cs = stored_channels(cout), cst = cs0 + cs1;
    float* bias = reinterpret_cast<float*>(out.data());
    for (int o = 0; o < cout; ++o) bias[o] = b[o];
    float* wt = reinterpret_cast<float*>(out.data() + align256(sizeof(float) * cs));
    for (int o = 0; o < cout; ++o)
      for (int tap = 0; tap < 9; ++tap)
        for (int c = 0; c < cst; ++c) {
          const int li = c < cs0 ? logical(0, c) : logical(1, c - cs0);
          if (li < 0) continue;
          wt[conv_f32_weight_index(o, tap, c, cst)] = wat(o, tap, li);
        }
  }
}

// Shape fields of an fp16 conv launch (no pointers); cs0/cs1 as in run_conv.
ConvF16Args f16_args(int cin0, int cin1, int cout, int h, int w, int cs0, int cs1, ConvLayout* L,
                     int tap_src = -1) {
  conv_f16_layout(stored_channels(cin0), cin1 ? stored_channels(cin1) : 0, cout, L, tap_src);
  ConvF16Args a{};
  a.cs0 = cs0 ? cs0 : stored_channels(cin0);
  a.cs1 = cin1 ? (cs1 ? cs1 : stored_channels(cin1)) : 0;
  a.h = h;
  a.w = w;
  a.cout_stored = stored_channels(cout);
  a.nchunks = L->nchunks;
  a.nup4 = L->nup4;
  a.nup = L->nup;
  a.npl4 = L->npl4;
  a.ntap = L->ntap;
  for (int i = 0; i < L->nchunks; ++i) a.chunk[i] = L->chunk[i];
  return a;
}

// Validates and launches one conv.  Pointers already checked by the caller.
// cs0/cs1: stored channels per pixel of the sources (0 = 4 * ceil(cin / 4)).
// batch, bstride (fp16): that many tiles, each at + b * bstride bytes.
int run_conv(const void* src0, int cin0, const void* src1, int cin1, bool upcat, int h, int w,
             const void* wpk, void* y, int cout, int in_dtype, int out_dtype, unsigned flags,
             hipStream_t stream, int cs0 = 0, int cs1 = 0, int tap_src = -1, int batch = 1,
             size_t bstride = 0) {
  const bool pool = flags & OIDN_POOL2X2, relu = flags & OIDN_RELU;
  hipError_t e;
  if (b16(in_dtype)) {
    ConvLayout L;
    ConvF16Args a = f16_args(cin0, cin1, cout, h, w, cs0, cs1, &L, tap_src);
    a.src0 = src0;
    a.src1 = src1;
    a.bias = static_cast<const float*>(wpk);
    a.wfrag = static_cast<const unsigned char*>(wpk) + L.bias_bytes;
    a.y = y;
    a.batch = batch;
    a.bstride = bstride;
    e = launch_conv_f16(a, L.nf, upcat, pool, relu, out_dtype == OIDN_F32, in_dtype == OIDN_BF16,
                        stream);
  } else {
    if (batch != 1) return fail(OIDN_E_UNSUPPORTED, "batched fp32 convs");
    ConvF32Args a{};
    a.src0 = static_cast<const float*>(src0);
    a.src1 = static_cast<const float*>(src1);
    a.cs0 = stored_channels(cin0);
    a.cs1 = cin1 ? stored_channels(cin1) : 0;
    a.h = h;
    a.w = w;
    a.bias = static_cast<const float*>(wpk);
    a.wt = reinterpret_cast<const float*>(static_cast<const unsigned char*>(wpk) +
                                          align256(sizeof(float) * stored_channels(cout)));
    a.y = static_cast<float*>(y);
    a.cout_stored = stored_channels(cout);
    e = launch_conv_f32(a, upcat, pool, relu, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "conv3x3 launch");
  return OIDN_OK;
}

int check_conv(int h, int w, int cin0, int cin1, int cout, int in_dtype, int out_dtype,
               unsigned flags, bool upcat) {
  int rc = check_dtype(in_dtype);
  if (rc) return rc;
  rc = check_dtype(out_dtype);
  if (rc) return rc;
  if (in_dtype == OIDN_F32 && out_dtype != OIDN_F32)
    return fail(OIDN_E_UNSUPPORTED, "fp32 input needs fp32 output");
  if (b16(out_dtype) && out_dtype != in_dtype)
    return fail(OIDN_E_UNSUPPORTED, "a 16-bit output needs the same 16-bit input type");
  if (h <= 0 || w <= 0 || h > 65536 || w > 65536)
    return fail(OIDN_E_INVALID, "conv size %dx%d out of range", w, h);
  if (flags & ~(OIDN_RELU | OIDN_POOL2X2)) return fail(OIDN_E_INVALID, "unknown conv flags 0x%x", flags);
  if ((flags & OIDN_POOL2X2) && (h % 2 || w % 2))
    return fail(OIDN_E_INVALID, "fused 2x2 pool needs even sizes (got %dx%d)", w, h);
  if (upcat && (h % 2 || w % 2))
    return fail(OIDN_E_INVALID, "upsample-concat needs even sizes (got %dx%d)", w, h);
  size_t bytes;
  rc = conv_weights_bytes(cin0, cin1, cout, in_dtype, &bytes);
  if (rc) return rc;
  if ((double)h * w * (stored_channels(cin0) + stored_channels(cin1 > 0 ? cin1 : 0) + stored_channels(cout)) > 2.0e9)
    return fail(OIDN_E_UNSUPPORTED, "tensor too large for 32-bit pixel indexing");
  return OIDN_OK;
}

// ------------------------------------------------------------ fused conv pair
// y = convB(relu(convA(x))), convA: cin -> 32, convB: 32 -> cout (fp16
// storage).  cs: stored channels per pixel of x (0 = 4 * ceil(cin / 4)).
// Supported when x moves in 16-byte units and convA's chunks are all of one
// kind (one chunk, or whole 32-channel chunks).
bool pair_supported(int cin, int cs, int cout) {
  const int st = stored_channels(cin);
  if (!cs) cs = st;
  return cs % 8 == 0 && (st <= kChunkChannels || st % kChunkChannels == 0) &&
         st <= 8 * kChunkChannels && cout >= 1 && cout <= 32;
}

// img: the network's last pair writes through the output pass instead of y.
// in_pass: the network's first pair reads the images through the input pass
// (instead of x) and writes the packed tile to in_pass->packed.
// batch, bstride, rects: that many tiles, activations at + b * bstride bytes,
// rects[b] the input pass origin / output pass rectangle of tile b.
// bf16: the 16-bit storage (x, the intermediate, a 16-bit y) is bf16.
int run_pair(const void* x, int cin, int cs, int h, int w, const void* wA, const void* wB, void* y,
             int cout, int out_dtype, unsigned flags, hipStream_t stream, bool tap = false,
             const OutputPass* img = nullptr, const PackArgs* in_pass = nullptr, int batch = 1,
             size_t bstride = 0, const TileRect* rects = nullptr, bool bf16 = false) {
  ConvLayout LA, LB;
  conv_f16_layout(stored_channels(cin), 0, 32, &LA, tap ? 0 : -1);
  conv_f16_layout(32, 0, cout, &LB);
  PairArgs p{};
  p.x = x;
  p.cs = cs ? cs : stored_channels(cin);
  p.h = h;
  p.w = w;
  p.nchunks = LA.nchunks;
  for (int i = 0; i < LA.nchunks; ++i) p.wfragA[i] = LA.chunk[i].wfrag;
  p.biasA = static_cast<const float*>(wA);
  p.wA = static_cast<const unsigned char*>(wA) + LA.bias_bytes;
  p.biasB = static_cast<const float*>(wB);
  p.wB = static_cast<const unsigned char*>(wB) + LB.bias_bytes;
  p.y = img ? nullptr : y;
  p.cout_stored = stored_channels(cout);
  if (img) p.img = *img;
  if (in_pass) p.in = *in_pass;
  if (batch < 1 || batch > kMaxBatch || ((img || in_pass) && !rects))
    return fail(OIDN_E_INVALID, "bad tile batch");
  p.batch = batch;
  p.bstride = bstride;
  for (int b = 0; rects && b < batch; ++b) p.rect[b] = rects[b];
  const int out = img ? kPairImage : out_dtype == OIDN_F32 ? kPairF32 : kPairF16;
  const int in = (tap ? kPairInTaps : 0) | (in_pass ? kPairInImages : 0);
  hipError_t e = launch_conv_pair_f16(p, LA.chunk[0].cg, LB.nf, in, flags & OIDN_POOL2X2,
                                      flags & OIDN_RELU, out, bf16, stream);
  if (e != hipSuccess) return hip_fail(e, "conv3x3 pair launch");
  return OIDN_OK;
}

// ------------------------------------------------------------ UNet table
struct Layer {
  const char* name;
  int src;     // value id: 0 = network input, k = output of layer k-1
  int skip;    // value id or -1
  int cout;
  bool pool;
  bool relu;
};

constexpr int kLayers = 16;
const Layer kUNet[kLayers] = {
    {"enc_conv0", 0, -1, 32, false, true},   {"enc_conv1", 1, -1, 32, true, true},
    {"enc_conv2", 2, -1, 48, true, true},    {"enc_conv3", 3, -1, 64, true, true},
    {"enc_conv4", 4, -1, 80, true, true},    {"enc_conv5a", 5, -1, 96, false, true},
    {"enc_conv5b", 6, -1, 96, false, true},  {"dec_conv4a", 7, 4, 112, false, true},
    {"dec_conv4b", 8, -1, 112, false, true}, {"dec_conv3a", 9, 3, 96, false, true},
    {"dec_conv3b", 10, -1, 96, false, true}, {"dec_conv2a", 11, 2, 64, false, true},
    {"dec_conv2b", 12, -1, 64, false, true}, {"dec_conv1a", 13, 0, 64, false, true},
    {"dec_conv1b", 14, -1, 32, false, true}, {"dec_conv0", 15, -1, 3, false, false},
};

struct LayerShape {
  int cin0, cin1, cout, level;  // level of the conv's output before pooling
};

bool unet_shapes(int in_channels, LayerShape* out) {
  if (in_channels != 3 && in_channels != 6 && in_channels != 9) return false;
  int ch[kLayers + 1], lvl[kLayers + 1];
  ch[0] = in_channels;
  lvl[0] = 0;
  for (int i = 0; i < kLayers; ++i) {
    const Layer& L = kUNet[i];
    const int level = L.skip >= 0 ? lvl[L.skip] : lvl[L.src];
    out[i] = {ch[L.src], L.skip >= 0 ? ch[L.skip] : 0, L.cout, level};
    ch[i + 1] = L.cout;
    lvl[i + 1] = level + (L.pool ? 1 : 0);
  }
  return true;
}

size_t unet_layer_offset(const LayerShape* s, int dtype, int layer) {
  size_t off = 0;
  for (int i = 0; i < layer; ++i) {
    size_t b = 0;
    conv_weights_bytes(s[i].cin0, s[i].cin1, s[i].cout, dtype, &b);
    off += align256(b);
  }
  return off;
}

// Tap variants.  With 9 input channels on the fp16 path the end-to-end call
// packs the input with channel 8's row taps (PackArgs::taps), and the layers
// that read the input (enc_conv0 from its source, dec_conv1a from its skip)
// run that source as a tap chunk: half the MFMA K-steps for it.  Their
// weights in that layout follow the sixteen plain ones in the packed blob;
// the plain ones serve oidn_unet_forward_packed, whose input is packed by
// the caller without taps.
bool unet_taps(int in_channels, int dtype) { return b16(dtype) && in_channels == 9; }

// Source of layer i read as a tap chunk when the input carries taps, or -1.
int unet_tap_src(int i) { return kUNet[i].src == 0 ? 0 : kUNet[i].skip == 0 ? 1 : -1; }

// Offset of layer i's tap-variant weights (unet_tap_src(i) >= 0); with
// layer = kLayers: the size of the whole blob.
size_t unet_tap_offset(const LayerShape* s, int dtype, int layer) {
  size_t off = unet_layer_offset(s, dtype, kLayers);
  for (int i = 0; i < layer && i < kLayers; ++i) {
    if (unet_tap_src(i) < 0) continue;
    size_t b = 0;
    conv_weights_bytes(s[i].cin0, s[i].cin1, s[i].cout, dtype, &b, unet_tap_src(i));
    off += align256(b);
  }
  return off;
}

size_t unet_weights_total(const LayerShape* s, int in_channels, int dtype) {
  return unet_taps(in_channels, dtype) ? unet_tap_offset(s, dtype, kLayers)
                                       : unet_layer_offset(s, dtype, kLayers);
}

// Liveness-planned workspace ([web-0.4] NativeUNetExecutor._createExecution
// reuses activation slots after a value's last use).  Values: 0 = input,
// k = output of layer k-1 (pooled if the layer pools); the network output
// (value 16) and, for the end-to-end call, the packed input are planned too
// when `own_io` is set.  Greedy first fit in decreasing size.
struct Plan {
  size_t offset[kLayers + 1];
  size_t bytes;
};

// Stored channels of the network input inside the end-to-end fp16 path: a
// multiple of 8, so the conv's patch loads move whole 16-byte channel groups.
int internal_input_lanes(int in_channels, int dtype) {
  const int cs = stored_channels(in_channels);
  return b16(dtype) ? (cs + 7) / 8 * 8 : cs;
}

// Layer i runs fused with layer i + 1 (y = conv_{i+1}(conv_i(x)) through LDS)
// when conv_i is a plain ReLU conv to 32 channels whose output only conv_{i+1}
// reads, conv_{i+1} is a plain 32 -> <= 32 conv, and the pair kernel takes
// conv_i's source.  In this network: enc_conv0 -> enc_conv1 and
// dec_conv1b -> dec_conv0 on the fp16 path.
bool fuse_with_next(int in_channels, int i, int dtype, bool own_io) {
  if (!b16(dtype) || i + 1 >= kLayers) return false;
  LayerShape s[kLayers];
  unet_shapes(in_channels, s);
  const Layer &A = kUNet[i], &B = kUNet[i + 1];
  if (A.skip >= 0 || A.pool || !A.relu || s[i].cout != 32) return false;
  if (B.src != i + 1 || B.skip >= 0 || s[i + 1].cin0 != 32 || s[i + 1].cout > 32) return false;
  for (int j = 0; j < kLayers; ++j)
    if (j != i + 1 && (kUNet[j].src == i + 1 || kUNet[j].skip == i + 1)) return false;
  const int cs = A.src == 0 && own_io ? internal_input_lanes(in_channels, dtype) : 0;
  return pair_supported(s[i].cin0, cs, s[i + 1].cout);
}

// The end-to-end path runs the output pass in the epilogue of the network's
// last conv when that conv is the second layer of a fused pair (fp16); the
// network output is then never stored.
bool output_fused(int in_channels, int dtype) {
  return fuse_with_next(in_channels, kLayers - 2, dtype, true);
}

// Likewise the input pass runs in the staging of the network's first conv
// when that conv is the first layer of a fused pair (fp16, a 16-lane chunk).
// The packed input is still written (the decoder's last skip reads it).
bool input_fused(int in_channels, int dtype) {
  return fuse_with_next(in_channels, 0, dtype, true) && b16(dtype) &&
         stored_channels(in_channels) <= 16;
}

// Tiles the end-to-end path runs through the network together: up to
// kMaxBatch tiles of one size when both image passes run inside the convs
// (the fp16 path), else one.
int tile_batch(int in_channels, int dtype, size_t ntiles) {
  if (!input_fused(in_channels, dtype) || !output_fused(in_channels, dtype)) return 1;
  return ntiles < (size_t)kMaxBatch ? (int)ntiles : kMaxBatch;
}

void plan_workspace(int in_channels, int tw, int th, int dtype, bool own_io, Plan* p) {
  LayerShape s[kLayers];
  unet_shapes(in_channels, s);
  size_t size[kLayers + 1];
  int def[kLayers + 1], last[kLayers + 1];
  const size_t px0 = (size_t)tw * th;
  size[0] = px0 * (own_io ? internal_input_lanes(in_channels, dtype)
                          : stored_channels(in_channels)) * esize(dtype);
  def[0] = -1;
  last[0] = -1;
  for (int i = 0; i < kLayers; ++i) {
    const int lvl = s[i].level + (kUNet[i].pool ? 1 : 0);
    const size_t px = px0 >> (2 * lvl);
    const bool final_layer = i == kLayers - 1;
    size[i + 1] = px * stored_channels(s[i].cout) * (final_layer ? 4 : esize(dtype));
    def[i + 1] = i;
    last[i + 1] = i;
  }
  for (int i = 0; i < kLayers; ++i) {
    last[kUNet[i].src] = i > last[kUNet[i].src] ? i : last[kUNet[i].src];
    if (kUNet[i].skip >= 0) last[kUNet[i].skip] = i > last[kUNet[i].skip] ? i : last[kUNet[i].skip];
  }
  last[kLayers] = kLayers;  // consumed by the output pass
  if (own_io && output_fused(in_channels, dtype)) size[kLayers] = 0;
  // A fused pair (layers i, i + 1) reads layer i's source while it writes
  // layer i + 1's output, so that source lives through layer i + 1; the
  // intermediate between them is never stored.
  for (int i = 0; i + 1 < kLayers; ++i)
    if (fuse_with_next(in_channels, i, dtype, own_io)) {
      int& l = last[kUNet[i].src];
      l = l > i + 1 ? l : i + 1;
      size[i + 1] = 0;
    }
  bool placed[kLayers + 1] = {};
  size_t end = 0;
  for (int n = 0; n <= kLayers; ++n) {
    int best = -1;
    for (int v = 0; v <= kLayers; ++v) {
      const bool external = !own_io && (v == 0 || v == kLayers);
      if (placed[v] || external) continue;
      if (best < 0 || size[v] > size[best]) best = v;
    }
    if (best < 0) break;
    // candidate offsets: 0 and the end of every placed value alive at the same time
    size_t chosen = (size_t)-1;
    std::vector<size_t> cands{0};
    for (int v = 0; v <= kLayers; ++v)
      if (placed[v]) cands.push_back(p->offset[v] + align256(size[v]));
    for (size_t c : cands) {
      bool clash = false;
      for (int v = 0; v <= kLayers && !clash; ++v) {
        if (!placed[v]) continue;
        const bool live = !(last[v] < def[best] || last[best] < def[v]);
        const bool overlap = c < p->offset[v] + align256(size[v]) && p->offset[v] < c + align256(size[best]);
        clash = live && overlap;
      }
      if (!clash && c < chosen) chosen = c;
    }
    p->offset[best] = chosen;
    placed[best] = true;
    if (chosen + align256(size[best]) > end) end = chosen + align256(size[best]);
  }
  p->bytes = end;
}

// Runs the sixteen convs of one tile, or of `batch` tiles of one size
// together (each with its own copy of the plan at + b * P.bytes; needs both
// image passes fused, rects[b] their rectangles).  events: optional,
// events[k] recorded before layer k and events[16] after the last layer.
// img (own_io, with output_fused): the output pass, run by the last pair;
// in_pass (own_io, with input_fused): the input pass, run by the first.
int run_network(const unsigned char* weights, int in_channels, const void* packed_in, int tw,
                int th, unsigned char* ws, const Plan& P, bool own_io, float* net_out, int dtype,
                hipStream_t stream, void* const* events, const OutputPass* img = nullptr,
                const PackArgs* in_pass = nullptr, int batch = 1, const TileRect* rects = nullptr) {
  const size_t bstride = batch > 1 ? P.bytes : 0;   // each tile has its own copy of the plan
  LayerShape s[kLayers];
  unet_shapes(in_channels, s);
  const void* val[kLayers + 1];
  val[0] = own_io ? ws + P.offset[0] : packed_in;
  for (int i = 1; i <= kLayers; ++i) val[i] = ws + P.offset[i];
  if (!own_io) val[kLayers] = net_out;
  size_t woff = 0;
  for (int i = 0; i < kLayers; ++i) {
    const Layer& L = kUNet[i];
    const int lvl = s[i].level;
    const int h = th >> lvl, w = tw >> lvl;
    if (events && events[i]) {
      hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[i]), stream);
      if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    const unsigned flags = (L.relu ? OIDN_RELU : 0u) | (L.pool ? OIDN_POOL2X2 : 0u);
    const int out_dtype = i == kLayers - 1 ? OIDN_F32 : dtype;
    const int in_cs = own_io ? internal_input_lanes(in_channels, dtype) : 0;
    const int tap_src = own_io && unet_taps(in_channels, dtype) ? unet_tap_src(i) : -1;
    const unsigned char* wl = tap_src >= 0 ? weights + unet_tap_offset(s, dtype, i) : weights + woff;
    if (fuse_with_next(in_channels, i, dtype, own_io)) {
      const Layer& B = kUNet[i + 1];
      const unsigned flags_b = (B.relu ? OIDN_RELU : 0u) | (B.pool ? OIDN_POOL2X2 : 0u);
      size_t ba = 0, bb = 0;
      conv_weights_bytes(s[i].cin0, 0, 32, dtype, &ba);
      conv_weights_bytes(32, 0, s[i + 1].cout, dtype, &bb);
      int rc = run_pair(val[L.src], s[i].cin0, L.src == 0 ? in_cs : 0, h, w, wl,
                        weights + woff + align256(ba), const_cast<void*>(val[i + 2]),
                        s[i + 1].cout, i + 1 == kLayers - 1 ? OIDN_F32 : dtype, flags_b, stream,
                        tap_src == 0, i + 1 == kLayers - 1 ? img : nullptr,
                        i == 0 ? in_pass : nullptr, batch, bstride, rects, dtype == OIDN_BF16);
      if (rc) return rc;
      if (events && events[i + 1]) {   // the second layer's interval is empty
        hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[i + 1]), stream);
        if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
      }
      woff += align256(ba) + align256(bb);
      ++i;
      continue;
    }
    int rc = run_conv(val[L.src], s[i].cin0, L.skip >= 0 ? val[L.skip] : nullptr, s[i].cin1,
                      L.skip >= 0, h, w, wl, const_cast<void*>(val[i + 1]), s[i].cout, dtype,
                      out_dtype, flags, stream, L.src == 0 ? in_cs : 0, L.skip == 0 ? in_cs : 0,
                      tap_src, batch, bstride);
    if (rc) return rc;
    size_t b = 0;
    conv_weights_bytes(s[i].cin0, s[i].cin1, s[i].cout, dtype, &b);
    woff += align256(b);
  }
  if (events && events[kLayers]) {
    hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[kLayers]), stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  }
  return OIDN_OK;
}

int check_network_tile(int in_channels, int tw, int th, int dtype) {
  int rc = check_dtype(dtype);
  if (rc) return rc;
  if (in_channels != 3 && in_channels != 6 && in_channels != 9)
    return fail(OIDN_E_INVALID, "input channels must be 3, 6 or 9 (got %d)", in_channels);
  if (tw <= 0 || th <= 0 || tw % OIDN_TILE_ALIGN || th % OIDN_TILE_ALIGN)
    return fail(OIDN_E_INVALID, "network tile %dx%d must be positive multiples of 16", tw, th);
  if ((double)tw * th * 128 > 2.0e9) return fail(OIDN_E_UNSUPPORTED, "network tile %dx%d too large", tw, th);
  return OIDN_OK;
}

int denoise(const void* d_weights, int in_channels, const float* color, const float* albedo,
            const float* normal, int w, int h, int hdr, int transfer, float input_scale,
            int max_tile, int overlap, void* workspace, size_t ws_bytes, float* out_rgba,
            int dtype, hipStream_t stream, void* const* events, int n_events,
            bool fit_batch = false) {
  if (!d_weights || !color || !workspace || !out_rgba)
    return fail(OIDN_E_INVALID, "null weights, color, workspace or output pointer");
  const int sources = 1 + (albedo != nullptr) + (normal != nullptr);
  if (normal && !albedo) return fail(OIDN_E_INVALID, "a normal image needs an albedo image");
  if (in_channels != 3 * sources)
    return fail(OIDN_E_INVALID, "model expects %d input channels but %d images were given",
                in_channels, sources);
  if (transfer == OIDN_TRANSFER_PU && hdr)
    return fail(OIDN_E_UNSUPPORTED, "the 'pu' transfer is not supported (formula unavailable)");
  if (transfer != OIDN_TRANSFER_PU && transfer != OIDN_TRANSFER_LOG)
    return fail(OIDN_E_INVALID, "unknown transfer %d", transfer);
  if (hdr && !(input_scale > 0.f && input_scale < 3.402823466e+38f))
    return fail(OIDN_E_INVALID, "input scale must be positive and finite");
  if (events && n_events < kLayers + 3) return fail(OIDN_E_INVALID, "need at least 19 events");
  if (!aligned16(color) || (albedo && !aligned16(albedo)) || (normal && !aligned16(normal)) ||
      !aligned16(out_rgba) || !aligned16(workspace) || !aligned16(d_weights))
    return fail(OIDN_E_INVALID, "device pointers must be 16-byte aligned");
  std::vector<oidn_tile> tiles;
  int rc = plan(w, h, max_tile, overlap, tiles);
  if (rc) return rc;
  int tw = 0, th = 0;
  for (const oidn_tile& t : tiles) {
    tw = t.in_w > tw ? t.in_w : tw;
    th = t.in_h > th ? t.in_h : th;
  }
  rc = check_network_tile(in_channels, tw, th, dtype);
  if (rc) return rc;
  Plan P;
  plan_workspace(in_channels, tw, th, dtype, true, &P);
  int nb = tile_batch(in_channels, dtype, tiles.size());
  // fit_batch: as many tiles per launch as the workspace holds (at least one)
  if (fit_batch && P.bytes > 0 && ws_bytes / P.bytes < (size_t)nb)
    nb = ws_bytes / P.bytes > 0 ? (int)(ws_bytes / P.bytes) : 1;
  if (ws_bytes < P.bytes * nb)
    return fail(OIDN_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes,
                P.bytes * nb);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if (input_fused(in_channels, dtype) && output_fused(in_channels, dtype)) {
    // batches of up to nb consecutive tiles of one size, both image passes
    // in the convs (the fp16 path)
    PackArgs pa{};
    pa.color = reinterpret_cast<const float4*>(color);
    pa.albedo = reinterpret_cast<const float4*>(albedo);
    pa.normal = reinterpret_cast<const float4*>(normal);
    pa.img_w = w;
    pa.img_h = h;
    pa.hdr = hdr;
    pa.input_scale = input_scale;
    pa.sources = sources;
    pa.lanes = internal_input_lanes(in_channels, dtype);
    pa.taps = unet_taps(in_channels, dtype) && pa.lanes == 16;
    pa.packed = ws + P.offset[0];
    OutputPass op{};
    op.color = reinterpret_cast<const float4*>(color);
    op.out = reinterpret_cast<float4*>(out_rgba);
    op.img_w = w;
    op.hdr = hdr;
    op.input_scale = input_scale;
    for (size_t k = 0; k < tiles.size();) {
      const oidn_tile& t0 = tiles[k];
      TileRect rects[kMaxBatch];
      int n = 0;
      while (k + n < tiles.size() && n < nb && tiles[k + n].in_w == t0.in_w &&
             tiles[k + n].in_h == t0.in_h) {
        const oidn_tile& t = tiles[k + n];
        rects[n++] = TileRect{t.in_x, t.in_y, t.out_x, t.out_y, t.out_w, t.out_h};
      }
      void* const* ev = (events && k == 0) ? events : nullptr;
      hipError_t e;
      if (ev && ev[0] && (e = hipEventRecord(static_cast<hipEvent_t>(ev[0]), stream)) != hipSuccess)
        return hip_fail(e, "hipEventRecord");
      pa.tile_w = t0.in_w;
      pa.tile_h = t0.in_h;
      rc = run_network(static_cast<const unsigned char*>(d_weights), in_channels, nullptr, t0.in_w,
                       t0.in_h, ws, P, true, nullptr, dtype, stream, ev ? ev + 1 : nullptr, &op,
                       &pa, n, rects);
      if (rc) return rc;
      if (ev && ev[kLayers + 2] &&
          (e = hipEventRecord(static_cast<hipEvent_t>(ev[kLayers + 2]), stream)) != hipSuccess)
        return hip_fail(e, "hipEventRecord");
      k += n;
    }
    return ok();
  }
  for (size_t k = 0; k < tiles.size(); ++k) {
    const oidn_tile& t = tiles[k];
    void* const* ev = (events && k == 0) ? events : nullptr;
    hipError_t e;
    if (ev && ev[0] && (e = hipEventRecord(static_cast<hipEvent_t>(ev[0]), stream)) != hipSuccess)
      return hip_fail(e, "hipEventRecord");
    PackArgs pa{};
    pa.color = reinterpret_cast<const float4*>(color);
    pa.albedo = reinterpret_cast<const float4*>(albedo);
    pa.normal = reinterpret_cast<const float4*>(normal);
    pa.img_w = w;
    pa.img_h = h;
    pa.tile_x = t.in_x;
    pa.tile_y = t.in_y;
    pa.tile_w = t.in_w;
    pa.tile_h = t.in_h;
    pa.hdr = hdr;
    pa.input_scale = input_scale;
    pa.sources = sources;
    pa.lanes = internal_input_lanes(in_channels, dtype);
    pa.taps = unet_taps(in_channels, dtype) && pa.lanes == 16;
    pa.packed = ws + P.offset[0];
    // input pass, network with a stored float32 output, output pass (fp32)
    if ((e = launch_pack(pa, dtype, stream)) != hipSuccess) return hip_fail(e, "pack launch");
    rc = run_network(static_cast<const unsigned char*>(d_weights), in_channels, nullptr, t.in_w,
                     t.in_h, ws, P, true, nullptr, dtype, stream, ev ? ev + 1 : nullptr);
    if (rc) return rc;
    UnpackArgs ua{};
    ua.net = reinterpret_cast<const float4*>(ws + P.offset[kLayers]);
    ua.tile_w = t.in_w;
    ua.o.color = reinterpret_cast<const float4*>(color);
    ua.o.out = reinterpret_cast<float4*>(out_rgba);
    ua.o.img_w = w;
    ua.o.in_off_x = t.out_x - t.in_x;
    ua.o.in_off_y = t.out_y - t.in_y;
    ua.o.out_x = t.out_x;
    ua.o.out_y = t.out_y;
    ua.o.out_w = t.out_w;
    ua.o.out_h = t.out_h;
    ua.o.hdr = hdr;
    ua.o.input_scale = input_scale;
    if ((e = launch_unpack(ua, stream)) != hipSuccess) return hip_fail(e, "unpack launch");
    if (ev && ev[kLayers + 2] && (e = hipEventRecord(static_cast<hipEvent_t>(ev[kLayers + 2]), stream)) != hipSuccess)
      return hip_fail(e, "hipEventRecord");
  }
  return ok();
}

int upload(const std::vector<unsigned char>& host, void* dst, hipStream_t stream) {
  hipError_t e = hipMemcpyAsync(dst, host.data(), host.size(), hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "weight upload");
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "weight upload sync");
  return OIDN_OK;
}

}  // namespace

namespace oidn {

int denoise_fit(const void* d_weights, int in_channels, const float* color, const float* albedo,
                const float* normal, int w, int h, int hdr, int transfer, float input_scale,
                int max_tile, int overlap, void* workspace, size_t ws_bytes, float* out_rgba,
                int dtype, hipStream_t stream) {
  return denoise(d_weights, in_channels, color, albedo, normal, w, h, hdr, transfer, input_scale,
                 max_tile, overlap, workspace, ws_bytes, out_rgba, dtype, stream, nullptr, 0, true);
}

int tile_workspace_bytes(int in_channels, int w, int h, int max_tile, int overlap, int dtype,
                         size_t* bytes) {
  std::vector<oidn_tile> tiles;
  int rc = plan(w, h, max_tile, overlap, tiles);
  if (rc) return rc;
  int tw = 0, th = 0;
  for (const oidn_tile& t : tiles) {
    tw = t.in_w > tw ? t.in_w : tw;
    th = t.in_h > th ? t.in_h : th;
  }
  rc = check_network_tile(in_channels, tw, th, dtype);
  if (rc) return rc;
  Plan P;
  plan_workspace(in_channels, tw, th, dtype, true, &P);
  *bytes = P.bytes;
  return OIDN_OK;
}

int set_error(int code, const char* what) { return fail(code, "%s", what); }

int clear_error() { return ok(); }

}  // namespace oidn

extern "C" {

const char* oidn_last_error(void) { return g_error.c_str(); }

int oidn_version(void) { return 100; }

int oidn_plan_tiles(int w, int h, int max_tile, int overlap, oidn_tile* tiles, int cap, int* count) {
  if (!count) return fail(OIDN_E_INVALID, "null count pointer");
  std::vector<oidn_tile> t;
  int rc = plan(w, h, max_tile, overlap, t);
  if (rc) return rc;
  *count = (int)t.size();
  if ((int)t.size() > cap) {
    if (cap == 0 && tiles == nullptr) return ok();
    return fail(OIDN_E_WORKSPACE, "%zu tiles do not fit in a capacity of %d", t.size(), cap);
  }
  if (!tiles) return fail(OIDN_E_INVALID, "null tiles pointer");
  for (size_t i = 0; i < t.size(); ++i) tiles[i] = t[i];
  return ok();
}

int oidn_conv3x3_weights_bytes(int cin0, int cin1, int cout, int dtype, size_t* bytes) {
  if (!bytes) return fail(OIDN_E_INVALID, "null bytes pointer");
  int rc = conv_weights_bytes(cin0, cin1, cout, dtype, bytes);
  return rc ? rc : ok();
}

int oidn_conv3x3_pack_weights(const float* w_ohwi_host, const float* bias_host, int cin0, int cin1,
                              int cout, int dtype, void* d_packed, hipStream_t stream) {
  if (!w_ohwi_host || !bias_host || !d_packed) return fail(OIDN_E_INVALID, "null pointer");
  size_t bytes;
  int rc = conv_weights_bytes(cin0, cin1, cout, dtype, &bytes);
  if (rc) return rc;
  if (!aligned16(d_packed)) return fail(OIDN_E_INVALID, "packed weights must be 16-byte aligned");
  std::vector<unsigned char> host(bytes);
  pack_conv_host(w_ohwi_host, bias_host, cin0, cin1, cout, dtype, host);
  rc = upload(host, d_packed, stream);
  return rc ? rc : ok();
}

int oidn_conv3x3_pack_weights_host(const float* w_ohwi_host, const float* bias_host, int cin0,
                                   int cin1, int cout, int dtype, void* host_packed) {
  if (!w_ohwi_host || !bias_host || !host_packed) return fail(OIDN_E_INVALID, "null pointer");
  size_t bytes;
  int rc = conv_weights_bytes(cin0, cin1, cout, dtype, &bytes);
  if (rc) return rc;
  std::vector<unsigned char> host(bytes);
  pack_conv_host(w_ohwi_host, bias_host, cin0, cin1, cout, dtype, host);
  std::memcpy(host_packed, host.data(), bytes);
  return ok();
}

int oidn_conv3x3(const void* x, int h, int w, int cin, const void* w_packed, void* y, int cout,
                 int in_dtype, int out_dtype, unsigned flags, hipStream_t stream) {
  if (!x || !w_packed || !y) return fail(OIDN_E_INVALID, "null pointer");
  if (!aligned16(x) || !aligned16(w_packed) || !aligned16(y))
    return fail(OIDN_E_INVALID, "device pointers must be 16-byte aligned");
  int rc = check_conv(h, w, cin, 0, cout, in_dtype, out_dtype, flags, false);
  if (rc) return rc;
  rc = run_conv(x, cin, nullptr, 0, false, h, w, w_packed, y, cout, in_dtype, out_dtype, flags, stream);
  return rc ? rc : ok();
}

int oidn_conv3x3_upcat(const void* low, int c_low, const void* skip, int c_skip, int h, int w,
                       const void* w_packed, void* y, int cout, int in_dtype, int out_dtype,
                       unsigned flags, hipStream_t stream) {
  if (!low || !skip || !w_packed || !y) return fail(OIDN_E_INVALID, "null pointer");
  if (!aligned16(low) || !aligned16(skip) || !aligned16(w_packed) || !aligned16(y))
    return fail(OIDN_E_INVALID, "device pointers must be 16-byte aligned");
  if (c_skip <= 0) return fail(OIDN_E_INVALID, "skip channels must be positive");
  int rc = check_conv(h, w, c_low, c_skip, cout, in_dtype, out_dtype, flags, true);
  if (rc) return rc;
  rc = run_conv(low, c_low, skip, c_skip, true, h, w, w_packed, y, cout, in_dtype, out_dtype, flags,
                stream);
  return rc ? rc : ok();
}

int oidn_conv3x3_pair(const void* x, int h, int w, int cin, const void* wa_packed,
                      const void* wb_packed, void* y, int cout, int out_dtype, unsigned flags,
                      hipStream_t stream) {
  if (!x || !wa_packed || !wb_packed || !y) return fail(OIDN_E_INVALID, "null pointer");
  if (!aligned16(x) || !aligned16(wa_packed) || !aligned16(wb_packed) || !aligned16(y))
    return fail(OIDN_E_INVALID, "device pointers must be 16-byte aligned");
  int rc = check_conv(h, w, cin, 0, 32, OIDN_F16, OIDN_F16, OIDN_RELU, false);
  if (rc) return rc;
  rc = check_conv(h, w, 32, 0, cout, OIDN_F16, out_dtype, flags, false);
  if (rc) return rc;
  if (!pair_supported(cin, 0, cout))
    return fail(OIDN_E_UNSUPPORTED,
                "conv pair needs cin <= 32 or a multiple of 32 (and a multiple of 8 stored), "
                "cout <= 32 (got %d -> 32 -> %d)", cin, cout);
  rc = run_pair(x, cin, 0, h, w, wa_packed, wb_packed, y, cout, out_dtype, flags, stream);
  return rc ? rc : ok();
}

int oidn_conv3x3_kernel(int h, int w, int cin0, int cin1, int cout, int in_dtype, int out_dtype,
                        unsigned flags, char* buf, int cap, int* blocks) {
  if (!buf || cap <= 0) return fail(OIDN_E_INVALID, "null or empty name buffer");
  if (cin1 < 0) return fail(OIDN_E_INVALID, "skip channels must not be negative");
  int rc = check_conv(h, w, cin0, cin1, cout, in_dtype, out_dtype, flags, cin1 > 0);
  if (rc) return rc;
  int nb = 0;
  if (b16(in_dtype)) {
    ConvLayout L;
    const ConvF16Args a = f16_args(cin0, cin1, cout, h, w, 0, 0, &L);
    conv_f16_describe(a, L.nf, out_dtype == OIDN_F32, in_dtype == OIDN_BF16, buf, cap, &nb);
  } else {
    snprintf(buf, cap, "%s", conv_f32_kernel_name(h, w, cout));
    nb = conv_f32_blocks(h, w, cout);
  }
  if (blocks) *blocks = nb;
  return ok();
}

int oidn_pool2x2(const void* x, int h, int w, int c, void* y, int dtype, hipStream_t stream) {
  if (!x || !y) return fail(OIDN_E_INVALID, "null pointer");
  int rc = check_dtype(dtype);
  if (rc) return rc;
  if (h <= 0 || w <= 0 || c <= 0 || h % 2 || w % 2)
    return fail(OIDN_E_INVALID, "pool2x2 needs positive even sizes and channels (got %dx%dx%d)", w, h, c);
  if (!aligned16(x) || !aligned16(y)) return fail(OIDN_E_INVALID, "device pointers must be 16-byte aligned");
  if ((double)h * w * stored_channels(c) > 4.0e9) return fail(OIDN_E_UNSUPPORTED, "tensor too large");
  hipError_t e = launch_pool(x, h, w, stored_channels(c), y, dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "pool launch");
  return ok();
}

int oidn_upsample_concat(const void* low, int c_low, const void* skip, int c_skip, int h, int w,
                         void* z, int dtype, hipStream_t stream) {
  if (!low || !skip || !z) return fail(OIDN_E_INVALID, "null pointer");
  int rc = check_dtype(dtype);
  if (rc) return rc;
  if (h <= 0 || w <= 0 || h % 2 || w % 2) return fail(OIDN_E_INVALID, "upsample-concat needs positive even sizes");
  if (c_low <= 0 || c_skip <= 0 || c_low % 4)
    return fail(OIDN_E_INVALID, "channels must be positive and the upsampled source a multiple of 4");
  if (!aligned16(low) || !aligned16(skip) || !aligned16(z))
    return fail(OIDN_E_INVALID, "device pointers must be 16-byte aligned");
  if ((double)h * w * (c_low + stored_channels(c_skip)) > 4.0e9) return fail(OIDN_E_UNSUPPORTED, "tensor too large");
  hipError_t e = launch_upcat(low, c_low, skip, stored_channels(c_skip), h, w, z, b16(dtype), stream);
  if (e != hipSuccess) return hip_fail(e, "upsample-concat launch");
  return ok();
}

int oidn_pack_input(const float* color, const float* albedo, const float* normal, int img_w,
                    int img_h, int tile_x, int tile_y, int tile_w, int tile_h, int hdr,
                    int transfer, float input_scale, void* packed, int dtype, hipStream_t stream) {
  if (!color || !packed) return fail(OIDN_E_INVALID, "null color or packed pointer");
  if (normal && !albedo) return fail(OIDN_E_INVALID, "a normal image needs an albedo image");
  int rc = check_dtype(dtype);
  if (rc) return rc;
  if (img_w <= 0 || img_h <= 0 || tile_w <= 0 || tile_h <= 0)
    return fail(OIDN_E_INVALID, "image and tile dimensions must be positive");
  if (img_w > 65536 || img_h > 65536 || tile_w > 65536 || tile_h > 65536)
    return fail(OIDN_E_INVALID, "dimensions above 65536 are not supported");
  if (transfer == OIDN_TRANSFER_PU && hdr)
    return fail(OIDN_E_UNSUPPORTED, "the 'pu' transfer is not supported (formula unavailable)");
  if (transfer != OIDN_TRANSFER_PU && transfer != OIDN_TRANSFER_LOG)
    return fail(OIDN_E_INVALID, "unknown transfer %d", transfer);
  if (hdr && !(input_scale > 0.f && input_scale < 3.402823466e+38f))
    return fail(OIDN_E_INVALID, "input scale must be positive and finite");
  if (!aligned16(color) || (albedo && !aligned16(albedo)) || (normal && !aligned16(normal)) || !aligned16(packed))
    return fail(OIDN_E_INVALID, "device pointers must be 16-byte aligned");
  if ((long long)tile_w * tile_h > kMaxPassPixels)
    return fail(OIDN_E_UNSUPPORTED, "tile of %dx%d pixels exceeds the 32-bit pixel index", tile_w, tile_h);
  PackArgs a{};
  a.color = reinterpret_cast<const float4*>(color);
  a.albedo = reinterpret_cast<const float4*>(albedo);
  a.normal = reinterpret_cast<const float4*>(normal);
  a.img_w = img_w;
  a.img_h = img_h;
  a.tile_x = tile_x;
  a.tile_y = tile_y;
  a.tile_w = tile_w;
  a.tile_h = tile_h;
  a.hdr = hdr;
  a.input_scale = input_scale;
  a.sources = 1 + (albedo != nullptr) + (normal != nullptr);
  a.lanes = stored_channels(3 * a.sources);
  a.packed = packed;
  hipError_t e = launch_pack(a, dtype, stream);
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return ok();
}

int oidn_unpack_output(const float* net_rgba, int tile_w, int tile_h, int in_off_x, int in_off_y,
                       const float* color, int img_w, int img_h, int out_x, int out_y, int out_w,
                       int out_h, int hdr, int transfer, float input_scale, float* out_rgba,
                       hipStream_t stream) {
  if (!net_rgba || !color || !out_rgba) return fail(OIDN_E_INVALID, "null pointer");
  if (tile_w <= 0 || tile_h <= 0 || img_w <= 0 || img_h <= 0 || out_w <= 0 || out_h <= 0)
    return fail(OIDN_E_INVALID, "dimensions must be positive");
  if (in_off_x < 0 || in_off_y < 0 || in_off_x + out_w > tile_w || in_off_y + out_h > tile_h)
    return fail(OIDN_E_INVALID, "output rectangle reads outside the tile");
  if (out_x < 0 || out_y < 0 || out_x + out_w > img_w || out_y + out_h > img_h)
    return fail(OIDN_E_INVALID, "output rectangle lies outside the image");
  if (transfer == OIDN_TRANSFER_PU && hdr)
    return fail(OIDN_E_UNSUPPORTED, "the 'pu' transfer is not supported (formula unavailable)");
  if (transfer != OIDN_TRANSFER_PU && transfer != OIDN_TRANSFER_LOG)
    return fail(OIDN_E_INVALID, "unknown transfer %d", transfer);
  if (hdr && !(input_scale > 0.f && input_scale < 3.402823466e+38f))
    return fail(OIDN_E_INVALID, "input scale must be positive and finite");
  if (!aligned16(net_rgba) || !aligned16(color) || !aligned16(out_rgba))
    return fail(OIDN_E_INVALID, "device pointers must be 16-byte aligned");
  if ((long long)out_w * out_h > kMaxPassPixels)
    return fail(OIDN_E_UNSUPPORTED, "output rectangle of %dx%d pixels exceeds the 32-bit pixel index",
                out_w, out_h);
  UnpackArgs a{};
  a.net = reinterpret_cast<const float4*>(net_rgba);
  a.tile_w = tile_w;
  a.o.in_off_x = in_off_x;
  a.o.in_off_y = in_off_y;
  a.o.color = reinterpret_cast<const float4*>(color);
  a.o.img_w = img_w;
  a.o.out_x = out_x;
  a.o.out_y = out_y;
  a.o.out_w = out_w;
  a.o.out_h = out_h;
  a.o.hdr = hdr;
  a.o.input_scale = input_scale;
  a.o.out = reinterpret_cast<float4*>(out_rgba);
  hipError_t e = launch_unpack(a, stream);
  if (e != hipSuccess) return hip_fail(e, "unpack launch");
  return ok();
}

int oidn_unet_layer_count(void) { return kLayers; }

int oidn_unet_layer_info(int in_channels, int layer, int* cin0, int* cin1, int* cout, int* level,
                         unsigned* flags, const char** name) {
  LayerShape s[kLayers];
  if (!unet_shapes(in_channels, s)) return fail(OIDN_E_INVALID, "input channels must be 3, 6 or 9");
  if (layer < 0 || layer >= kLayers) return fail(OIDN_E_INVALID, "layer %d out of range", layer);
  if (cin0) *cin0 = s[layer].cin0;
  if (cin1) *cin1 = s[layer].cin1;
  if (cout) *cout = s[layer].cout;
  if (level) *level = s[layer].level;
  if (flags) *flags = (kUNet[layer].relu ? OIDN_RELU : 0u) | (kUNet[layer].pool ? OIDN_POOL2X2 : 0u);
  if (name) *name = kUNet[layer].name;
  return ok();
}

int oidn_unet_layer_kernel(int in_channels, int layer, int tw, int th, int batch, int dtype,
                           char* buf, int cap, int* blocks) {
  if (!buf || cap <= 0) return fail(OIDN_E_INVALID, "null or empty name buffer");
  if (batch < 1 || batch > kMaxBatch) return fail(OIDN_E_INVALID, "batch %d out of range", batch);
  int rc = check_network_tile(in_channels, tw, th, dtype);
  if (rc) return rc;
  if (layer < 0 || layer >= kLayers) return fail(OIDN_E_INVALID, "layer %d out of range", layer);
  LayerShape s[kLayers];
  unet_shapes(in_channels, s);
  const int h = th >> s[layer].level, w = tw >> s[layer].level;
  const bool final_layer = layer == kLayers - 1;
  int nb = 0;
  if (b16(dtype) && (fuse_with_next(in_channels, layer, dtype, true) ||
                            (layer > 0 && fuse_with_next(in_channels, layer - 1, dtype, true)))) {
    // both layers of a fused pair report the pair kernel (sized by the first)
    const int first = fuse_with_next(in_channels, layer, dtype, true) ? layer : layer - 1;
    const int fh = th >> s[first].level, fw = tw >> s[first].level;
    const int st = stored_channels(s[first].cin0);
    const int cs = kUNet[first].src == 0 ? internal_input_lanes(in_channels, dtype) : st;
    const bool tap = unet_taps(in_channels, dtype) && unet_tap_src(first) == 0;
    // output: 0 fp16, 1 fp32, 2 through the output pass (last layer, fused);
    // input: 1 taps | 2 images through the input pass (first layer, fused)
    const int out = first + 1 == kLayers - 1 ? (output_fused(in_channels, dtype) ? 2 : 1) : 0;
    const int in = (tap ? 1 : 0) | (first == 0 && input_fused(in_channels, dtype) ? 2 : 0);
    snprintf(buf, cap, "conv3x3_pair_%s<%d, %d, %d, %d>", dtype == OIDN_BF16 ? "bf16" : "f16",
             st > 16 ? 4 : 2, cdiv(stored_channels(s[first + 1].cout), 16), out, in);
    (void)cs;
    nb = conv_pair_blocks(fh, fw) * batch;
  } else if (b16(dtype)) {
    // as oidn_unet_forward runs it: the input packed with a multiple of 8 lanes
    const int in_cs = internal_input_lanes(in_channels, dtype);
    const Layer& L = kUNet[layer];
    ConvLayout lay;
    ConvF16Args a = f16_args(s[layer].cin0, s[layer].cin1, s[layer].cout, h, w,
                             L.src == 0 ? in_cs : 0, L.skip == 0 ? in_cs : 0, &lay,
                             unet_taps(in_channels, dtype) ? unet_tap_src(layer) : -1);
    a.batch = batch;
    conv_f16_describe(a, lay.nf, final_layer, dtype == OIDN_BF16, buf, cap, &nb);
  } else {
    snprintf(buf, cap, "%s", conv_f32_kernel_name(h, w, s[layer].cout));
    nb = conv_f32_blocks(h, w, s[layer].cout) * batch;
  }
  if (blocks) *blocks = nb;
  return ok();
}

int oidn_unet_weights_bytes(int in_channels, int dtype, size_t* bytes) {
  if (!bytes) return fail(OIDN_E_INVALID, "null bytes pointer");
  int rc = check_dtype(dtype);
  if (rc) return rc;
  LayerShape s[kLayers];
  if (!unet_shapes(in_channels, s)) return fail(OIDN_E_INVALID, "input channels must be 3, 6 or 9");
  *bytes = unet_weights_total(s, in_channels, dtype);
  return ok();
}

int oidn_unet_pack_weights(const float* const* w_ohwi_host, const float* const* bias_host,
                           int in_channels, int dtype, void* d_weights, hipStream_t stream) {
  if (!w_ohwi_host || !bias_host || !d_weights) return fail(OIDN_E_INVALID, "null pointer");
  int rc = check_dtype(dtype);
  if (rc) return rc;
  LayerShape s[kLayers];
  if (!unet_shapes(in_channels, s)) return fail(OIDN_E_INVALID, "input channels must be 3, 6 or 9");
  if (!aligned16(d_weights)) return fail(OIDN_E_INVALID, "weights must be 16-byte aligned");
  for (int i = 0; i < kLayers; ++i)
    if (!w_ohwi_host[i] || !bias_host[i]) return fail(OIDN_E_INVALID, "null weights of layer %d", i);
  std::vector<unsigned char> all(unet_weights_total(s, in_channels, dtype), 0);
  size_t off = 0;
  for (int i = 0; i < kLayers; ++i) {
    size_t b = 0;
    conv_weights_bytes(s[i].cin0, s[i].cin1, s[i].cout, dtype, &b);
    std::vector<unsigned char> one(b);
    if (i == kLayers - 1 && b16(dtype)) {
      // fp16: the last layer's RGB in all four 4-channel lane groups of its
      // output fragment (lane 3 of each zero), for the output pass in its
      // epilogue; the same bytes as the plain 3-channel packing
      const int cin = s[i].cin0 + s[i].cin1;
      std::vector<float> wr((size_t)16 * 9 * cin, 0.f), br(16, 0.f);
      for (int g = 0; g < 4; ++g)
        for (int o = 0; o < s[i].cout; ++o) {
          std::memcpy(&wr[(size_t)(4 * g + o) * 9 * cin], w_ohwi_host[i] + (size_t)o * 9 * cin,
                      sizeof(float) * 9 * cin);
          br[4 * g + o] = bias_host[i][o];
        }
      size_t b16 = 0;
      conv_weights_bytes(s[i].cin0, s[i].cin1, 16, dtype, &b16);
      if (b16 != b) return fail(OIDN_E_UNSUPPORTED, "last layer packing size mismatch");
      pack_conv_host(wr.data(), br.data(), s[i].cin0, s[i].cin1, 16, dtype, one);
    } else {
      pack_conv_host(w_ohwi_host[i], bias_host[i], s[i].cin0, s[i].cin1, s[i].cout, dtype, one);
    }
    std::memcpy(all.data() + off, one.data(), b);
    off += align256(b);
  }
  if (unet_taps(in_channels, dtype))
    for (int i = 0; i < kLayers; ++i) {
      const int ts = unet_tap_src(i);
      if (ts < 0) continue;
      size_t b = 0;
      conv_weights_bytes(s[i].cin0, s[i].cin1, s[i].cout, dtype, &b, ts);
      std::vector<unsigned char> one(b);
      pack_conv_host(w_ohwi_host[i], bias_host[i], s[i].cin0, s[i].cin1, s[i].cout, dtype, one, ts);
      std::memcpy(all.data() + unet_tap_offset(s, dtype, i), one.data(), b);
    }
  rc = upload(all, d_weights, stream);
  return rc ? rc : ok();
}

int oidn_unet_packed_workspace_bytes(int in_channels, int tw, int th, int dtype, size_t* bytes) {
  if (!bytes) return fail(OIDN_E_INVALID, "null bytes pointer");
  int rc = check_network_tile(in_channels, tw, th, dtype);
  if (rc) return rc;
  Plan P;
  plan_workspace(in_channels, tw, th, dtype, false, &P);
  *bytes = P.bytes;
  return ok();
}

int oidn_unet_forward_packed(const void* d_weights, int in_channels, const void* packed_in, int tw,
                             int th, void* workspace, size_t ws_bytes, float* net_out_rgba,
                             int dtype, hipStream_t stream) {
  if (!d_weights || !packed_in || !workspace || !net_out_rgba) return fail(OIDN_E_INVALID, "null pointer");
  int rc = check_network_tile(in_channels, tw, th, dtype);
  if (rc) return rc;
  if (!aligned16(d_weights) || !aligned16(packed_in) || !aligned16(workspace) || !aligned16(net_out_rgba))
    return fail(OIDN_E_INVALID, "device pointers must be 16-byte aligned");
  Plan P;
  plan_workspace(in_channels, tw, th, dtype, false, &P);
  if (ws_bytes < P.bytes)
    return fail(OIDN_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, P.bytes);
  rc = run_network(static_cast<const unsigned char*>(d_weights), in_channels, packed_in, tw, th,
                   static_cast<unsigned char*>(workspace), P, false, net_out_rgba, dtype, stream, nullptr);
  return rc ? rc : ok();
}

int oidn_unet_workspace_bytes(int in_channels, int w, int h, int max_tile, int overlap, int dtype,
                              size_t* bytes) {
  if (!bytes) return fail(OIDN_E_INVALID, "null bytes pointer");
  std::vector<oidn_tile> tiles;
  int rc = plan(w, h, max_tile, overlap, tiles);
  if (rc) return rc;
  int tw = 0, th = 0;
  for (const oidn_tile& t : tiles) {
    tw = t.in_w > tw ? t.in_w : tw;
    th = t.in_h > th ? t.in_h : th;
  }
  rc = check_network_tile(in_channels, tw, th, dtype);
  if (rc) return rc;
  Plan P;
  plan_workspace(in_channels, tw, th, dtype, true, &P);
  *bytes = P.bytes * tile_batch(in_channels, dtype, tiles.size());
  return ok();
}

int oidn_unet_tile_batch(int in_channels, int w, int h, int max_tile, int overlap, int dtype,
                         int* batch) {
  if (!batch) return fail(OIDN_E_INVALID, "null batch pointer");
  std::vector<oidn_tile> tiles;
  int rc = plan(w, h, max_tile, overlap, tiles);
  if (rc) return rc;
  LayerShape s[kLayers];
  if (!unet_shapes(in_channels, s)) return fail(OIDN_E_INVALID, "input channels must be 3, 6 or 9");
  rc = check_dtype(dtype);
  if (rc) return rc;
  *batch = tile_batch(in_channels, dtype, tiles.size());
  return ok();
}

int oidn_unet_input_layout(int in_channels, int w, int h, int max_tile, int overlap, int dtype,
                           size_t* offset, size_t* tile_stride, int* lanes, int* taps) {
  if (!offset || !tile_stride || !lanes || !taps) return fail(OIDN_E_INVALID, "null pointer");
  std::vector<oidn_tile> tiles;
  int rc = plan(w, h, max_tile, overlap, tiles);
  if (rc) return rc;
  int tw = 0, th = 0;
  for (const oidn_tile& t : tiles) {
    tw = t.in_w > tw ? t.in_w : tw;
    th = t.in_h > th ? t.in_h : th;
  }
  rc = check_network_tile(in_channels, tw, th, dtype);
  if (rc) return rc;
  Plan P;
  plan_workspace(in_channels, tw, th, dtype, true, &P);
  *offset = P.offset[0];
  *tile_stride = tile_batch(in_channels, dtype, tiles.size()) > 1 ? P.bytes : 0;
  *lanes = internal_input_lanes(in_channels, dtype);
  *taps = unet_taps(in_channels, dtype) && *lanes == 16;
  return ok();
}

int oidn_unet_forward(const void* d_weights, int in_channels, const float* color, const float* albedo,
                      const float* normal, int w, int h, int hdr, int transfer, float input_scale,
                      int max_tile, int overlap, void* workspace, size_t ws_bytes, float* out_rgba,
                      int dtype, hipStream_t stream) {
  return denoise(d_weights, in_channels, color, albedo, normal, w, h, hdr, transfer, input_scale,
                 max_tile, overlap, workspace, ws_bytes, out_rgba, dtype, stream, nullptr, 0);
}

int oidn_unet_forward_timed(const void* d_weights, int in_channels, const float* color,
                            const float* albedo, const float* normal, int w, int h, int hdr,
                            int transfer, float input_scale, int max_tile, int overlap,
                            void* workspace, size_t ws_bytes, float* out_rgba, int dtype,
                            hipStream_t stream, void* const* events, int n_events) {
  if (!events) return fail(OIDN_E_INVALID, "null events");
  return denoise(d_weights, in_channels, color, albedo, normal, w, h, hdr, transfer, input_scale,
                 max_tile, overlap, workspace, ws_bytes, out_rgba, dtype, stream, events, n_events);
}

int oidn_calibrate_mfma(int dtype, long iters, int blocks, float* sink, long long* flops,
                        hipStream_t stream) {
  if (!sink || !flops) return fail(OIDN_E_INVALID, "null sink or flops pointer");
  if (dtype != OIDN_F16 && dtype != OIDN_BF16)
    return fail(OIDN_E_INVALID, "the MFMA stream is fp16 or bf16 (got dtype %d)", dtype);
  if (iters <= 0 || iters > (1L << 30) || blocks <= 0 || blocks > (1 << 20))
    return fail(OIDN_E_INVALID, "iterations or workgroups out of range");
  hipError_t e = launch_mfma_stream(dtype == OIDN_BF16, iters, blocks, sink, stream);
  if (e != hipSuccess) return hip_fail(e, "MFMA stream launch");
  *flops = mfma_stream_flops(iters, blocks);
  return ok();
}

int oidn_calibrate_read(const void* buf, size_t bytes, float* sink, hipStream_t stream) {
  if (!buf || !sink) return fail(OIDN_E_INVALID, "null buffer or sink pointer");
  if (bytes == 0 || bytes % 16 || !aligned16(buf))
    return fail(OIDN_E_INVALID, "the read stream needs a 16-byte aligned buffer of 16-byte words");
  hipError_t e = launch_read_stream(buf, bytes, sink, stream);
  if (e != hipSuccess) return hip_fail(e, "read stream launch");
  return ok();
}

int oidn_event_create(void** event) {
  if (!event) return fail(OIDN_E_INVALID, "null event pointer");
  hipEvent_t e;
  hipError_t r = hipEventCreate(&e);
  if (r != hipSuccess) return hip_fail(r, "hipEventCreate");
  *event = e;
  return ok();
}

int oidn_event_destroy(void* event) {
  if (!event) return fail(OIDN_E_INVALID, "null event");
  hipError_t r = hipEventDestroy(static_cast<hipEvent_t>(event));
  if (r != hipSuccess) return hip_fail(r, "hipEventDestroy");
  return ok();
}

int oidn_event_elapsed_ms(void* start, void* end, float* ms) {
  if (!start || !end || !ms) return fail(OIDN_E_INVALID, "null pointer");
  hipError_t r = hipEventSynchronize(static_cast<hipEvent_t>(end));
  if (r != hipSuccess) return hip_fail(r, "hipEventSynchronize");
  r = hipEventElapsedTime(ms, static_cast<hipEvent_t>(start), static_cast<hipEvent_t>(end));
  if (r != hipSuccess) return hip_fail(r, "hipEventElapsedTime");
  return ok();
}

}  // extern "C"
