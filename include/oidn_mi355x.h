/*
 * oidn_mi355x.h -- C ABI of the MI355X (gfx950) OIDN-style UNet denoiser.
 *
 * Pages cited (by title and symbol):
 *   [web-0.4]    "oidn-web 0.3.4 -> 0.4.0", nativeUNet.ts
 *   [web-0.5]    "oidn-web 0.4.0 -> 0.5.0", nativeUNet.ts
 *   [webgpu-0.6] "oidn-webgpu 0.0.0-stage -> 0.6.0", native/denoise.ts
 *
 * Conventions shared by every call
 *   - Images and activations are NHWC with batch 1.  Activations keep their
 *     channels in 4-lane blocks ([web-0.4] blocksForChannels,
 *     activationByteSize): a tensor of C logical channels stores
 *     C_store = 4 * ceil(C / 4) values per pixel and the unused lanes are 0.
 *   - Tensor pointers are DEVICE pointers owned by the caller.  Host pointers
 *     are named *_host.  The library never allocates or frees device memory
 *     and never synchronises, except the two weight-pack calls, which copy
 *     from host memory and wait for that copy.
 *   - Device work is enqueued on the given stream (0 = the null stream) and
 *     the call returns at once.
 *   - Every call returns an int status: OIDN_OK (0) or a negative code.  On
 *     any error nothing is enqueued and outputs are untouched;
 *     oidn_last_error() returns the message (thread-local).
 *   - dtype selects the storage type of activations and weights: OIDN_F16
 *     (fp16 storage, fp32 accumulate, MFMA path), OIDN_BF16 (bf16 storage,
 *     the same kernels with the bf16 MFMA; every stored value rounded to
 *     nearest even from fp32, as fp16 is) or OIDN_F32 (fp32 storage and
 *     arithmetic).  A conv's 16-bit output has its input's type; any 16-bit
 *     path may write fp32 instead.  Weights are packed for one dtype.
 *     Biases are always fp32 ([web-0.4] packConvTensors keeps the bias in f32).
 *   - Overlapping calls on different streams that share buffers race; the
 *     caller orders them.
 */
#ifndef OIDN_MI355X_H
#define OIDN_MI355X_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define OIDN_OK              0
#define OIDN_E_INVALID      -1  /* null pointer, bad size, bad enum          */
#define OIDN_E_UNSUPPORTED  -2  /* valid request the library does not handle */
#define OIDN_E_WORKSPACE    -3  /* workspace or output capacity too small    */
#define OIDN_E_HIP          -4  /* a HIP runtime call or launch failed       */

/* ---- storage types ----------------------------------------------------- */
#define OIDN_F32   0
#define OIDN_F16   1
#define OIDN_BF16  2

/* ---- conv flags -------------------------------------------------------- */
#define OIDN_RELU     1u  /* y = max(y, 0) ([web-0.4] activationExpression)            */
#define OIDN_POOL2X2  2u  /* 2x2/2 max-pool fused after bias+ReLU; output h/2 x w/2
                             ([web-0.4] createFusedConvPoolShader)                    */

/* ---- HDR transfer ------------------------------------------------------ */
#define OIDN_TRANSFER_PU   0  /* named by [webgpu-0.6]; formula not on the pages:
                                 OIDN_E_UNSUPPORTED                                   */
#define OIDN_TRANSFER_LOG  1  /* F(x) = ln(1 + x), F^-1(y) = exp(y) - 1 (reading)    */

/* ---- limits ------------------------------------------------------------ */
#define OIDN_MAX_SOURCE_CHANNELS 256   /* logical channels per conv source */
#define OIDN_MAX_OUT_CHANNELS    128
#define OIDN_TILE_ALIGN           16   /* tile starts and sizes (four 2x2 pools) */
#define OIDN_DEFAULT_OVERLAP      96   /* alignUp(one-sided receptive reach 94, 16) */

/* One tile of a tile grid: the input rectangle the network runs on and the
 * output rectangle it writes ([webgpu-0.6] recordDenoiseExecution reads
 * tile.input.{x,y,width,height} and tile.output.{x,y,width,height}).
 * Input rectangles may extend past the image: those reads clamp to the edge. */
typedef struct oidn_tile {
  int in_x, in_y, in_w, in_h;
  int out_x, out_y, out_w, out_h;
} oidn_tile;

/* Message of the last failed call on this thread ("" if none). */
const char* oidn_last_error(void);

/* ABI version: major * 10000 + minor * 100 + patch. */
int oidn_version(void);

/* ========================================================================
 * 3x3 convolution, stride 1, zero padding 1, bias, optional ReLU and fused
 * 2x2 max-pool ([web-0.4] createConvShader: the sum starts at the bias and
 * skips taps outside the image; createFusedConvPoolShader).
 *
 *   y[p][o] = act(b[o] + sum_{ky,kx in 0..2} sum_i W[o][ky][kx][i] * x[p + (ky-1, kx-1)][i])
 *
 * Weights are OHWI float32 over LOGICAL input channels.  A conv over two
 * sources (the decoder's upsample + concat) indexes the logical concat
 * [upsampled source (cin0 channels), skip (cin1 channels)].
 * ======================================================================== */

/* Bytes of the packed weights+bias buffer for (cin0, cin1, cout, dtype).
 * cin1 = 0 for a one-source conv.  Host only. */
int oidn_conv3x3_weights_bytes(int cin0, int cin1, int cout, int dtype, size_t* bytes);

/* Packs OHWI float32 weights (cout x 3 x 3 x (cin0 + cin1), host) and a
 * float32 bias (cout, host) into the device layout of the chosen dtype
 * (fp16 and bf16: MFMA A-operand fragments in K-major chunk order, pad lanes 0, the
 * upsampled source of a two-source conv as four sums of ky rows -- W0,
 * W1 + W2, W0 + W1, W2, each rounded once to the storage type -- because an output row
 * reads only two low-resolution rows of it; fp32: [out block][tap][stored
 * input channel][4 out lanes]).  d_packed must hold
 * oidn_conv3x3_weights_bytes() bytes.  Blocks until the upload finished.
 * Two sources need cin0 % 4 == 0 (each source keeps its own 4-lane blocks,
 * [web-0.4] createTiledDecoderShader). */
int oidn_conv3x3_pack_weights(const float* w_ohwi_host, const float* bias_host,
                              int cin0, int cin1, int cout, int dtype,
                              void* d_packed, hipStream_t stream);

/* Same packing into host memory (host_packed: oidn_conv3x3_weights_bytes()
 * bytes), no device work.  For inspecting or caching the packed layout. */
int oidn_conv3x3_pack_weights_host(const float* w_ohwi_host, const float* bias_host,
                                   int cin0, int cin1, int cout, int dtype, void* host_packed);

/* One-source conv.  x: h x w x C_store(cin) of in_dtype; y: (h x w, or
 * h/2 x w/2 with OIDN_POOL2X2) x C_store(cout) of out_dtype.  in_dtype f32
 * needs out_dtype f32; in_dtype f16 allows f16 or f32 out.  POOL2X2 needs even
 * h and w.  w_packed from oidn_conv3x3_pack_weights(cin, 0, cout, in_dtype).
 * x and y must not overlap. */
int oidn_conv3x3(const void* x, int h, int w, int cin, const void* w_packed,
                 void* y, int cout, int in_dtype, int out_dtype, unsigned flags,
                 hipStream_t stream);

/* Decoder conv: nearest 2x upsample of `low` (h/2 x w/2 x c_low) concatenated
 * with `skip` (h x w x C_store(c_skip)), never materialised ([web-0.4]
 * createTiledDecoderShader reads the upsampled source at (x/2, y/2); blocks
 * of the first source come first).  h, w even; c_low % 4 == 0.  w_packed from
 * oidn_conv3x3_pack_weights(c_low, c_skip, cout, in_dtype). */
int oidn_conv3x3_upcat(const void* low, int c_low, const void* skip, int c_skip,
                       int h, int w, const void* w_packed, void* y, int cout,
                       int in_dtype, int out_dtype, unsigned flags, hipStream_t stream);

/* Two convs in one pass, y = convB(relu(convA(x))), the 32-channel
 * intermediate never leaving the chip: convA is cin -> 32 (bias, ReLU,
 * fp16 rounding as oidn_conv3x3 with OIDN_RELU), convB is 32 -> cout with
 * `flags` and `out_dtype` as in oidn_conv3x3.  Both convs as defined by
 * [web-0.4] createConvShader ("oidn-web 0.3.4 -> 0.4.0", nativeUNet.ts);
 * the fusion is this library's.  fp16 storage only.  wa_packed / wb_packed:
 * oidn_conv3x3_pack_weights output for (cin, 0, 32) and (32, 0, cout).
 * x: h x w x 4 ceil(cin / 4) fp16; y as oidn_conv3x3's output.  The result
 * equals oidn_conv3x3(convB) applied to oidn_conv3x3(convA) bit for bit.
 * Needs 4 ceil(cin / 4) a multiple of 8 and either <= 32 or a multiple of
 * 32, and cout <= 32 (else OIDN_E_UNSUPPORTED). */
int oidn_conv3x3_pair(const void* x, int h, int w, int cin, const void* wa_packed,
                      const void* wb_packed, void* y, int cout, int out_dtype, unsigned flags,
                      hipStream_t stream);

/* Name of the kernel instance that oidn_conv3x3 (cin1 == 0) or
 * oidn_conv3x3_upcat (cin0 = c_low, cin1 = c_skip) runs for this shape,
 * written NUL-terminated into buf (cap bytes), e.g.
 * "conv3x3_f16_mfma<4, 8, 4, false>"; *blocks (may be null) receives the
 * launch's workgroup count.  Same validation as those calls; host only. */
int oidn_conv3x3_kernel(int h, int w, int cin0, int cin1, int cout, int in_dtype,
                        int out_dtype, unsigned flags, char* buf, int cap, int* blocks);

/* ========================================================================
 * Elementwise and gather passes
 * ======================================================================== */

/* 2x2 max-pool, stride 2 ([web-0.4] createMaxPoolShader; [web-0.5] coalesced
 * "channels" layout).  x: h x w x C_store(c); y: h/2 x w/2 x C_store(c).
 * h and w must be even. */
int oidn_pool2x2(const void* x, int h, int w, int c, void* y, int dtype, hipStream_t stream);

/* Materialised nearest 2x upsample + concat: z[y][x] = [low[y/2][x/2] (C_store(c_low)
 * lanes), skip[y][x] (C_store(c_skip) lanes)].  low: h/2 x w/2; skip, z: h x w.
 * h, w even; c_low % 4 == 0. */
int oidn_upsample_concat(const void* low, int c_low, const void* skip, int c_skip,
                         int h, int w, void* z, int dtype, hipStream_t stream);

/* Input pass of one tile ([webgpu-0.6] inputShader; lane layout of [web-0.4]
 * createInputPackShader).  color/albedo/normal: img_h x img_w RGBA float32
 * (16 B per pixel); albedo and normal may be NULL (3 or 6 channels; normal
 * needs albedo).  For each tile pixel (tx, ty) the source pixel is
 * clamp((tile_x + tx, tile_y + ty), (0, 0), (img_w-1, img_h-1)).  Colour:
 * hdr ? F(sanitize(rgb * input_scale, 0, FLT_MAX)) : sanitize(rgb, 0, 1);
 * albedo: sanitize(rgb, 0, 1); normal: sanitize(rgb, -1, 1) * 0.5 + 0.5,
 * where sanitize maps NaN to 0 and clamps.  The 3/6/9 channels are packed
 * densely into 4-lane blocks (lane l of block b is channel 4b + l), unused
 * lanes 0.  packed: tile_h x tile_w x C_store(channels) of dtype.
 * tile_w * tile_h above 2^31 - 1025 pixels: OIDN_E_UNSUPPORTED. */
int oidn_pack_input(const float* color, const float* albedo, const float* normal,
                    int img_w, int img_h, int tile_x, int tile_y, int tile_w, int tile_h,
                    int hdr, int transfer, float input_scale, void* packed, int dtype,
                    hipStream_t stream);

/* Output pass of one tile ([webgpu-0.6] outputShader).  net_rgba: the
 * network's RGBA float32 output for a tile_w x tile_h tile.  For each pixel
 * (x, y) of the out_w x out_h output rectangle:
 *   d = sanitize(net[y + in_off_y][x + in_off_x].rgb, 0, hdr ? FLT_MAX : 1)
 *   out[out_y + y][out_x + x] = (hdr ? F^-1(d) / input_scale : d,
 *                                color[out_y + y][out_x + x].a)
 * out_rgba: img_h x img_w RGBA float32; only the rectangle is written.
 * out_w * out_h above 2^31 - 1025 pixels: OIDN_E_UNSUPPORTED. */
int oidn_unpack_output(const float* net_rgba, int tile_w, int tile_h, int in_off_x,
                       int in_off_y, const float* color, int img_w, int img_h, int out_x,
                       int out_y, int out_w, int out_h, int hdr, int transfer,
                       float input_scale, float* out_rgba, hipStream_t stream);

/* ========================================================================
 * Tile grid (host only, pure).  [webgpu-0.6] recordDenoiseExecution plans
 * tiles with maxTileSize (0 = the whole image, aligned up) and an overlap
 * from the receptive field aligned to the tile alignment; the planner body
 * is not on the pages.  Reading: per axis of extent E with tile limit T and
 * overlap O, one tile when alignUp(E, 16) <= T, else n = ceil(E / (T - 2O))
 * output spans of S = alignUp(ceil(E / n), 16) pixels whose input spans are
 * min(S + 2O, alignUp(E, 16)) wide, shifted to stay in [0, alignUp(E, 16)).
 * Tiles are listed row-major (y outer).  max_tile must be 0 or a multiple of
 * 16; overlap < 0 selects OIDN_DEFAULT_OVERLAP, otherwise a multiple of 16.
 * *count receives the number of tiles; OIDN_E_WORKSPACE if it exceeds cap
 * (tiles may be NULL with cap 0 to query the count).
 * ======================================================================== */
int oidn_plan_tiles(int w, int h, int max_tile, int overlap, oidn_tile* tiles, int cap,
                    int* count);

/* ========================================================================
 * UNet.  Sixteen 3x3 convs in this order (logical channels; the pages'
 * modelSpec is not shown -- wiring read from the OIDN-style channel list):
 *   enc_conv0 in->32, enc_conv1 32->32 +pool, enc_conv2 32->48 +pool,
 *   enc_conv3 48->64 +pool, enc_conv4 64->80 +pool, enc_conv5a 80->96,
 *   enc_conv5b 96->96, dec_conv4a [up(5b) 96 | pool3 64]->112, dec_conv4b
 *   112->112, dec_conv3a [up 112 | pool2 48]->96, dec_conv3b 96->96,
 *   dec_conv2a [up 96 | pool1 32]->64, dec_conv2b 64->64, dec_conv1a
 *   [up 64 | input in]->64, dec_conv1b 64->32, dec_conv0 32->3 (no ReLU,
 *   float32 RGBA output, lane 3 = 0).
 * in_channels is 3, 6 or 9 ([web-0.4] NativeUNetExecutor constructor).
 * ======================================================================== */

int oidn_unet_layer_count(void);

/* Shape of layer `layer` (0..15): logical channels of the (upsampled) source
 * and of the skip (0 if none), output channels, resolution level (0 = full,
 * 1 = /2, ...), flags (OIDN_RELU | OIDN_POOL2X2), and a static name. */
int oidn_unet_layer_info(int in_channels, int layer, int* cin0, int* cin1, int* cout,
                         int* level, unsigned* flags, const char** name);

/* Name of the kernel instance that runs `layer` on `batch` tw x th tiles per
 * launch (oidn_unet_tile_batch; the launch plan counts the whole launch's
 * workgroups) (for matching per-kernel timings and profiles), written NUL-terminated into
 * buf (cap bytes), e.g. "conv3x3_f16_mfma<2, 16, 2, false>" (fragments and
 * rows per wave, row groups, fp32 output) or, for both layers of a fused
 * pair, "conv3x3_pair_f16<2, 2, 0, 3>" (convA channel groups, convB
 * fragments, output: 0 16-bit, 1 fp32, 2 straight through the output pass;
 * input: bit 0 tap-packed, bit 1 the caller's images through the input pass),
 * or "conv3x3_ws_f16<4, 8, 4, false>" for a layer whose whole weight set fits
 * in LDS (dec_conv1a with the tap-packed skip): one persistent workgroup per
 * compute unit that walks the launch's tiles, so *blocks is that grid;
 * with bf16 storage "conv3x3_bf16_mfma", "conv3x3_pair_bf16" and
 * "conv3x3_ws_bf16".  *blocks receives the launch's workgroup count.  Host
 * only. */
int oidn_unet_layer_kernel(int in_channels, int layer, int tw, int th, int batch, int dtype,
                           char* buf, int cap, int* blocks);

/* Bytes of the packed weights of all sixteen layers.  With 9 input channels
 * on the 16-bit paths the blob also holds a second copy of enc_conv0's and
 * dec_conv1a's weights in the layout oidn_unet_forward uses for its
 * tap-packed input (channel 8's row neighbours beside it: half the matrix
 * steps for that source); oidn_unet_forward_packed uses the plain copies.
 * On the 16-bit paths dec_conv0's one output fragment holds its three output
 * channels' weights and biases in each of its four 4-channel groups (lanes
 * 4g .. 4g + 2, lane 4g + 3 zero), so the output pass fused into that
 * layer's kernel can spread its rows over all lanes; the size is unchanged. */
int oidn_unet_weights_bytes(int in_channels, int dtype, size_t* bytes);

/* Packs all layers: w_ohwi_host[i] is cout x 3 x 3 x cin (cin = cin0 + cin1
 * of layer i), bias_host[i] is cout floats.  Blocks until uploaded. */
int oidn_unet_pack_weights(const float* const* w_ohwi_host, const float* const* bias_host,
                           int in_channels, int dtype, void* d_weights, hipStream_t stream);

/* Workspace for oidn_unet_forward_packed on a tw x th tile (liveness-planned
 * activation buffers; input and output are the caller's). */
int oidn_unet_packed_workspace_bytes(int in_channels, int tw, int th, int dtype, size_t* bytes);

/* The network on one packed tile ([web-0.4] NativeUNetExecutor.execute: one
 * pass per node, the last writing float32).  packed_in: th x tw x
 * C_store(in_channels) of dtype (from oidn_pack_input); net_out_rgba: th x tw
 * x 4 float32.  tw, th: positive multiples of 16. */
int oidn_unet_forward_packed(const void* d_weights, int in_channels, const void* packed_in,
                             int tw, int th, void* workspace, size_t ws_bytes,
                             float* net_out_rgba, int dtype, hipStream_t stream);

/* Workspace for oidn_unet_forward on a w x h image with this tile plan
 * (on the 16-bit paths one copy of the per-tile plan for each tile of a batch,
 * see oidn_unet_tile_batch). */
int oidn_unet_workspace_bytes(int in_channels, int w, int h, int max_tile, int overlap,
                              int dtype, size_t* bytes);

/* Tiles of this plan that oidn_unet_forward runs through the network
 * together: on the 16-bit paths, where both image passes run inside the first
 * and last convs, up to 16 consecutive tiles of one size share one launch
 * per layer (tile index in grid z, or one tile sequence for the persistent
 * weight-stationary layer); else 1.  The per-kernel events of
 * oidn_unet_forward_timed cover the first such batch.  Host only. */
int oidn_unet_tile_batch(int in_channels, int w, int h, int max_tile, int overlap, int dtype,
                         int* batch);

/* Where oidn_unet_forward keeps the packed network input of a tile inside
 * its workspace (host only; for inspection and tests): tile k of the last
 * tile batch of the call (oidn_unet_tile_batch) at workspace + *offset +
 * k * *tile_stride (stride 0 when tiles run one by one), tile_h x tile_w
 * pixels of *lanes values of dtype.  With *taps (16-bit storage, nine
 * channels) lanes 0..7 hold channels 0..7, lanes 8, 9, 10 channel 8 of the
 * pixels in tile columns x - 1, x, x + 1 (zero past the tile's edge), the
 * rest zero; else the oidn_pack_input layout padded with zero lanes.  The
 * values stay there after the call until the workspace is reused. */
int oidn_unet_input_layout(int in_channels, int w, int h, int max_tile, int overlap, int dtype,
                           size_t* offset, size_t* tile_stride, int* lanes, int* taps);

/* End-to-end denoise ([webgpu-0.6] recordDenoiseExecution): plan the tile
 * grid, then for each tile in order: input pass, network, output pass into
 * the tile's output rectangle of out_rgba (h x w RGBA float32; on the 16-bit
 * path the network's first fused pair runs the input pass on the images and
 * the last writes that rectangle itself).  in_channels
 * must match the non-NULL images (color; + albedo; + normal). */
int oidn_unet_forward(const void* d_weights, int in_channels, const float* color,
                      const float* albedo, const float* normal, int w, int h, int hdr,
                      int transfer, float input_scale, int max_tile, int overlap,
                      void* workspace, size_t ws_bytes, float* out_rgba, int dtype,
                      hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * denoise as oidn_unet_forward, with no workspace argument.  Its workspace is
 * a static device array of OIDN_NOALLOC_SCRATCH_MB MiB inside the library,
 * one per GPU, held until the process ends; the call allocates and frees
 * nothing.  As many tiles run per launch as that array holds (the results
 * are the same bits as oidn_unet_forward's).  A plan whose single tile needs
 * more (oidn_unet_workspace_bytes / oidn_unet_tile_batch) is refused with
 * OIDN_E_WORKSPACE before any device work: 1920x1080 in one tile needs about
 * 400 MB, so such images need max_tile (512 fits).  Nothing in the array
 * needs to start at zero (every value is written before it is read).  All
 * calls on one GPU share the array: calls that overlap in time on one GPU
 * (other streams, other host threads) race and must be ordered by the
 * caller. */
#define OIDN_NOALLOC_SCRATCH_MB 64
int oidn_unet_forward_noalloc(const void* d_weights, int in_channels, const float* color,
                              const float* albedo, const float* normal, int w, int h, int hdr,
                              int transfer, float input_scale, int max_tile, int overlap,
                              float* out_rgba, int dtype, hipStream_t stream);

/* Size in bytes of the array oidn_unet_forward_noalloc uses.  Host only. */
int oidn_unet_noalloc_scratch_bytes(size_t* bytes);

/* Same as oidn_unet_forward, and records events[k] on the stream before the
 * k-th kernel of the FIRST tile or tile batch (k = 0: input pass, 1..16: layers, 17: output
 * pass) and events[18] after it, for per-kernel timing.  Where the first
 * layer's kernel runs the input pass itself (layer kernel input bit 1),
 * events[0] and events[1] are recorded back to back; where the last layer's
 * runs the output pass (output field 2), events[17] and events[18].
 * n_events >= 19; events are hipEvent_t handles (see oidn_event_create). */
int oidn_unet_forward_timed(const void* d_weights, int in_channels, const float* color,
                            const float* albedo, const float* normal, int w, int h, int hdr,
                            int transfer, float input_scale, int max_tile, int overlap,
                            void* workspace, size_t ws_bytes, float* out_rgba, int dtype,
                            hipStream_t stream, void* const* events, int n_events);

/* Measurement helper, not part of the denoise path: `blocks` workgroups of
 * 4 waves, each wave issuing iters x 8 independent 16x16x32 MFMAs (fp16, or
 * bf16 with dtype OIDN_BF16) with no memory traffic, to measure the matrix
 * rate the device sustains.  *flops receives the launch's work (2 per
 * multiply-add).  sink: a device buffer of at least 256 floats (written
 * only in a case the operands never produce).  Enqueued on `stream`. */
int oidn_calibrate_mfma(int dtype, long iters, int blocks, float* sink, long long* flops,
                        hipStream_t stream);

/* Measurement helper, not part of the denoise path: reads the `bytes` of
 * device buffer `buf` once (16-byte streaming loads, 2048 workgroups), to
 * measure the HBM read rate.  bytes: a multiple of 16; sink: a device buffer
 * of at least 256 floats (written only in a case the data never produces). */
int oidn_calibrate_read(const void* buf, size_t bytes, float* sink, hipStream_t stream);

/* Timing helpers: a hipEvent_t with timing enabled, its destruction, and the
 * milliseconds between two completed events (synchronises on `end`). */
int oidn_event_create(void** event);
int oidn_event_destroy(void* event);
int oidn_event_elapsed_ms(void* start, void* end, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* OIDN_MI355X_H */
