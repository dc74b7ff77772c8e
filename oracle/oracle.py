"""CPU oracle for the OIDN-style UNet denoise forward pass.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module.  It shares no code with the HIP library: it is a plain,
slow, direct-convolution restatement of what the pages compute, written in
numpy with float64 arithmetic.  The one library primitive it leans on is
``numpy.matmul`` for the per-tap channel contraction of the 3x3 convolution.

Pages cited (by title and symbol):

* [web-0.4] "oidn-web 0.3.4 -> 0.4.0", nativeUNet.ts
* [web-0.5] "oidn-web 0.4.0 -> 0.5.0", nativeUNet.ts (hunks over [web-0.4])
* [webgpu-0.6] "oidn-webgpu 0.0.0-stage -> 0.6.0", native/denoise.ts

Storage model.  A compute precision ``'f16'``, ``'bf16'`` or ``'f32'`` says how
every stored tensor is rounded: weights are rounded to it ([web-0.4]
packConvTensors converts weights to the activation precision), the bias stays
float32 ([web-0.4] packConvTensors: bias stays f32 because convolution
accumulates in f32), every activation is rounded after bias and ReLU (float64
-> float32 -> float16 or bfloat16 with round-to-nearest-even; bfloat16 is
not on the pages: it is read as the same model with the 16-bit format
swapped), and the last convolution
stores float32 ([web-0.4] NativeUNetExecutor._nodePipelineSpec and
_createExecution: the final node writes an f32 buffer).  Sums are taken in
float64, so only accumulation order separates this from an fp32-accumulating
GPU path.

Readings where the pages are silent:

* the UNet wiring (the ``modelSpec`` module is not on the pages): skips are the
  pool outputs pool1..pool3 and the packed network input; the decoder concat
  order is [upsampled source, skip];
* the HDR "log" transfer (``hdrTransfer.js`` is not on the pages):
  F(x) = ln(1 + x), F^-1(y) = exp(y) - 1.  Parity unpinned: its values are a
  chosen reading; only the round trip pins it;
* ``sanitize`` (``sanitize.js`` is not on the pages): NaN -> 0, otherwise clamp;
* the tile grid (``tileScheduler.js`` is not on the pages): the even split
  described at ``plan_tiles``.
"""
from __future__ import annotations

import math

import numpy as np

FLT_MAX = float(np.finfo(np.float32).max)
TILE_ALIGN = 16          # tile starts/sizes are multiples of 2^4 (four 2x2 pools)
DEFAULT_OVERLAP = 96     # alignUp(one-sided receptive reach 94, 16)


# ----------------------------------------------------------------------------
# Channel blocks ([web-0.4] blocksForChannels / activationByteSize): channels
# are stored in 4-lane blocks, unused lanes hold zero.
# ----------------------------------------------------------------------------
def blocks(c: int) -> int:
    return -(-c // 4)


def stored(c: int) -> int:
    return 4 * blocks(c)


def np_storage(precision: str):
    """numpy dtype holding stored values; bfloat16 values are held exactly in
    float32 (numpy has no bfloat16)."""
    if precision == "f16":
        return np.float16
    if precision in ("f32", "bf16"):
        return np.float32
    raise ValueError(f"unknown precision {precision!r}")


def float32_to_bfloat16(v32) -> np.ndarray:
    """float32 -> bfloat16 (8 significant bits, float32's exponent range),
    round to nearest, ties to even, written out on the bit pattern: keep the
    upper 16 bits after adding 0x7FFF plus the lowest kept bit; NaN stays NaN
    (the addition could carry a NaN payload into the exponent).  Overflow
    rounds to infinity.  Returned as float32."""
    v32 = np.ascontiguousarray(v32, dtype=np.float32)
    u = v32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    return np.where(np.isnan(v32), np.float32(np.nan), out)


def round_to(values, precision: str) -> np.ndarray:
    """Round float64 values to a stored precision: to float32 (RNE), then, for
    'f16', float32 -> float16 (RNE; overflow -> inf; subnormals kept), for
    'bf16', float32 -> bfloat16 (RNE, held in float32)."""
    with np.errstate(over="ignore"):
        v32 = np.asarray(values, dtype=np.float64).astype(np.float32)
        if precision == "f16":
            return v32.astype(np.float16)
        if precision == "bf16":
            return float32_to_bfloat16(v32)
        return v32


# ----------------------------------------------------------------------------
# sanitize and the HDR transfer ([webgpu-0.6] inputShader / outputShader call
# sanitize(), HDRForward() and HDRInverse(), whose bodies are not on the pages)
# ----------------------------------------------------------------------------
def sanitize(v, lo: float, hi: float) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    v = np.where(np.isnan(v), 0.0, v)
    return np.minimum(np.maximum(v, lo), hi)


def hdr_forward(x) -> np.ndarray:
    return np.log1p(np.asarray(x, dtype=np.float64))


def hdr_inverse(y) -> np.ndarray:
    return np.expm1(np.asarray(y, dtype=np.float64))


# ----------------------------------------------------------------------------
# Input pass ([webgpu-0.6] inputShader; lane layout as in [web-0.4]
# createInputPackShader): clamp-to-edge read of the tile rectangle, sanitize,
# HDR transfer of the colour, normals mapped from [-1, 1] to [0, 1], the
# 3 * sources channels packed densely into 4-lane blocks, unused lanes 0.
# ----------------------------------------------------------------------------
def pack_input(color, albedo, normal, tile_x: int, tile_y: int, tile_w: int, tile_h: int,
               hdr: bool, input_scale: float, precision: str) -> np.ndarray:
    img_h, img_w = color.shape[:2]
    ys = np.clip(np.arange(tile_y, tile_y + tile_h), 0, img_h - 1)
    xs = np.clip(np.arange(tile_x, tile_x + tile_w), 0, img_w - 1)

    def rect(img):
        return img[ys][:, xs]

    col = rect(color)[..., :3].astype(np.float32)
    if hdr:
        scaled = col * np.float32(input_scale)          # the multiply is float32
        channels = [hdr_forward(sanitize(scaled, 0.0, FLT_MAX))]
    else:
        channels = [sanitize(col, 0.0, 1.0)]
    if albedo is not None:
        channels.append(sanitize(rect(albedo)[..., :3], 0.0, 1.0))
        if normal is not None:
            channels.append(sanitize(rect(normal)[..., :3], -1.0, 1.0) * 0.5 + 0.5)
    elif normal is not None:
        raise ValueError("a normal image needs an albedo image")
    logical = np.concatenate(channels, axis=-1)
    out = np.zeros((tile_h, tile_w, stored(logical.shape[-1])), np_storage(precision))
    out[..., :logical.shape[-1]] = round_to(logical, precision)
    return out


# ----------------------------------------------------------------------------
# 3x3 convolution, stride 1, zero padding 1, bias, optional ReLU
# ([web-0.4] createConvShader: the accumulator starts at the bias, taps outside
# the image are skipped, ReLU is max(acc, 0)).  Weights are OHWI over logical
# input channels.  Out-of-range lanes are stored as 0.
# ----------------------------------------------------------------------------
def conv3x3(x: np.ndarray, cin: int, w_ohwi: np.ndarray, b: np.ndarray, relu: bool,
            precision: str, out_precision: str | None = None) -> np.ndarray:
    out_precision = out_precision or precision
    h, w = x.shape[:2]
    cout = w_ohwi.shape[0]
    assert w_ohwi.shape == (cout, 3, 3, cin), (w_ohwi.shape, cin)
    wq = round_to(w_ohwi, precision).astype(np.float64)
    xp = np.zeros((h + 2, w + 2, cin), np.float64)
    xp[1:h + 1, 1:w + 1] = x[..., :cin].astype(np.float64)
    acc = np.empty((h * w, cout), np.float64)
    acc[...] = np.asarray(b, np.float64)
    for ky in range(3):
        for kx in range(3):
            # sum over input channels of W[o][ky][kx][i] * X[y+ky-1][x+kx-1][i]
            shifted = np.ascontiguousarray(xp[ky:ky + h, kx:kx + w, :]).reshape(h * w, cin)
            acc += shifted @ wq[:, ky, kx, :].T
    acc = acc.reshape(h, w, cout)
    if relu:
        acc = np.maximum(acc, 0.0)
    out = np.zeros((h, w, stored(cout)), np_storage(out_precision))
    out[..., :cout] = round_to(acc, out_precision)
    return out


# ----------------------------------------------------------------------------
# 2x2 max-pool, stride 2 ([web-0.4] createMaxPoolShader): the max over the four
# inputs of each window.  Even sizes only (the network never sees odd ones).
# ----------------------------------------------------------------------------
def pool2x2(x: np.ndarray) -> np.ndarray:
    h, w, c = x.shape
    if h % 2 or w % 2:
        raise ValueError("pool2x2 needs even height and width")
    return x.reshape(h // 2, 2, w // 2, 2, c).max(axis=(1, 3))


# ----------------------------------------------------------------------------
# Nearest 2x upsample + channel concat ([web-0.4] createTiledDecoderShader /
# createFusedDecoderShader: the upsampled source is read at (x/2, y/2); input
# blocks of the first source come before those of the second, each source
# keeping its own 4-lane blocks).
# ----------------------------------------------------------------------------
def upsample_concat(low: np.ndarray, c_low: int, skip: np.ndarray, c_skip: int) -> np.ndarray:
    if c_low % 4:
        raise ValueError("the upsampled source must fill whole 4-lane blocks")
    h, w = skip.shape[:2]
    if low.shape[0] * 2 != h or low.shape[1] * 2 != w:
        raise ValueError("low-resolution source must be half the skip size")
    up = low[np.arange(h) // 2][:, np.arange(w) // 2][..., :stored(c_low)]
    return np.concatenate([up, skip[..., :stored(c_skip)]], axis=-1)


# ----------------------------------------------------------------------------
# The network (reading of the missing modelSpec; see the module docstring).
# Each row: (name, upsampled-or-plain source, skip source or None, cout,
# 2x2 pool after the conv, ReLU).  Channel counts follow the OIDN-style UNet.
# ----------------------------------------------------------------------------
UNET_LAYERS = (
    ("enc_conv0",  "input",      None,    32, False, True),
    ("enc_conv1",  "enc_conv0",  None,    32, True,  True),   # -> pool1
    ("enc_conv2",  "enc_conv1",  None,    48, True,  True),   # -> pool2
    ("enc_conv3",  "enc_conv2",  None,    64, True,  True),   # -> pool3
    ("enc_conv4",  "enc_conv3",  None,    80, True,  True),   # -> pool4
    ("enc_conv5a", "enc_conv4",  None,    96, False, True),
    ("enc_conv5b", "enc_conv5a", None,    96, False, True),
    ("dec_conv4a", "enc_conv5b", "enc_conv3", 112, False, True),
    ("dec_conv4b", "dec_conv4a", None,   112, False, True),
    ("dec_conv3a", "dec_conv4b", "enc_conv2",  96, False, True),
    ("dec_conv3b", "dec_conv3a", None,    96, False, True),
    ("dec_conv2a", "dec_conv3b", "enc_conv1",  64, False, True),
    ("dec_conv2b", "dec_conv2a", None,    64, False, True),
    ("dec_conv1a", "dec_conv2b", "input",  64, False, True),
    ("dec_conv1b", "dec_conv1a", None,    32, False, True),
    ("dec_conv0",  "dec_conv1b", None,     3, False, False),
)


def unet_layer_shapes(in_channels: int):
    """[(cin_logical, cout)] in table order; decoder cin = c_upsampled + c_skip."""
    if in_channels not in (3, 6, 9):
        raise ValueError("input channels must be 3, 6 or 9")
    couts = {"input": in_channels}
    shapes = []
    for name, src, skip, cout, _pool, _relu in UNET_LAYERS:
        cin = couts[src] + (couts[skip] if skip else 0)
        shapes.append((cin, cout))
        couts[name] = cout
    return shapes


def unet_forward_packed(weights, biases, packed: np.ndarray, in_channels: int,
                        precision: str) -> np.ndarray:
    """Network on one packed tile; returns the RGBA float32 network output (lane 3 = 0)."""
    th, tw = packed.shape[:2]
    if th % TILE_ALIGN or tw % TILE_ALIGN:
        raise ValueError("tile sizes must be multiples of 16")
    values = {"input": packed}
    chans = {"input": in_channels}
    last = len(UNET_LAYERS) - 1
    for i, (name, src, skip, cout, pool, relu) in enumerate(UNET_LAYERS):
        if skip is None:
            x, cin = values[src], chans[src]
        else:
            x = upsample_concat(values[src], chans[src], values[skip], chans[skip])
            cin = chans[src] + chans[skip]
        y = conv3x3(x, cin, weights[i], biases[i], relu, precision,
                    "f32" if i == last else precision)
        values[name] = pool2x2(y) if pool else y
        chans[name] = cout
    return values[UNET_LAYERS[last][0]]


# ----------------------------------------------------------------------------
# Output pass ([webgpu-0.6] outputShader): inside the tile's output rectangle,
# sanitize the network RGB (the network may emit negatives or NaNs), undo the
# HDR transfer and the input scale, take alpha from the input colour.
# ----------------------------------------------------------------------------
def unpack_output(net: np.ndarray, in_off_x: int, in_off_y: int, color: np.ndarray,
                  out_x: int, out_y: int, out_w: int, out_h: int, hdr: bool,
                  input_scale: float, out: np.ndarray) -> None:
    raw = net[in_off_y:in_off_y + out_h, in_off_x:in_off_x + out_w, :3]
    d = sanitize(raw, 0.0, FLT_MAX if hdr else 1.0)
    rgb = hdr_inverse(d) / np.float64(np.float32(input_scale)) if hdr else d
    out[out_y:out_y + out_h, out_x:out_x + out_w, :3] = rgb.astype(np.float32)
    out[out_y:out_y + out_h, out_x:out_x + out_w, 3] = color[out_y:out_y + out_h,
                                                              out_x:out_x + out_w, 3]


# ----------------------------------------------------------------------------
# Tile grid ([webgpu-0.6] recordDenoiseExecution: overlap from the receptive
# field aligned to the tile alignment, maxTileSize 0 meaning the whole image
# aligned up; planTileGrid itself is not on the pages).  Reading: per axis of
# extent E with tile limit T and overlap O, one tile when alignUp(E) fits,
# otherwise n = ceil(E / (T - 2O)) output spans of S = alignUp(ceil(E / n))
# pixels, each input span S + 2O wide (capped at alignUp(E)) and shifted to
# stay inside [0, alignUp(E)).
# ----------------------------------------------------------------------------
def align_up(v: int, a: int = TILE_ALIGN) -> int:
    return -(-v // a) * a


def _plan_axis(extent: int, tile: int, overlap: int):
    ea = align_up(extent)
    if ea <= tile:
        return [(0, ea, 0, extent)]
    step = tile - 2 * overlap
    if step <= 0:
        raise ValueError("tile size must exceed twice the overlap")
    n = -(-extent // step)
    span = align_up(-(-extent // n))
    size = min(span + 2 * overlap, ea)
    spans = []
    for i in range(n):
        o0 = i * span
        if o0 >= extent:
            break
        o1 = min(extent, o0 + span)
        lo = min(max(0, o0 - overlap), ea - size)
        spans.append((lo, size, o0, o1 - o0))
    return spans


def plan_tiles(width: int, height: int, max_tile: int = 0, overlap: int = -1):
    """List of (in_x, in_y, in_w, in_h, out_x, out_y, out_w, out_h), row-major."""
    if width <= 0 or height <= 0:
        raise ValueError("image dimensions must be positive")
    if overlap < 0:
        overlap = DEFAULT_OVERLAP
    if overlap % TILE_ALIGN:
        raise ValueError("overlap must be a multiple of 16")
    if max_tile < 0 or max_tile % TILE_ALIGN:
        raise ValueError("max tile size must be 0 or a positive multiple of 16")
    tile = max_tile if max_tile > 0 else align_up(max(width, height))
    xs = _plan_axis(width, tile, overlap)
    ys = _plan_axis(height, tile, overlap)
    return [(x[0], y[0], x[1], y[1], x[2], y[2], x[3], y[3]) for y in ys for x in xs]


def unet_forward(weights, biases, color, albedo, normal, hdr: bool, input_scale: float,
                 max_tile: int, overlap: int, precision: str) -> np.ndarray:
    """Tiled denoise ([webgpu-0.6] recordDenoiseExecution): for each planned
    tile, input pass -> network -> output pass into the tile's output rect."""
    img_h, img_w = color.shape[:2]
    in_channels = 3 * (1 + (albedo is not None) + (normal is not None))
    out = np.full((img_h, img_w, 4), np.nan, np.float32)
    for (ix, iy, iw, ih, ox, oy, ow, oh) in plan_tiles(img_w, img_h, max_tile, overlap):
        packed = pack_input(color, albedo, normal, ix, iy, iw, ih, hdr, input_scale, precision)
        net = unet_forward_packed(weights, biases, packed, in_channels, precision)
        unpack_output(net, ox - ix, oy - iy, color, ox, oy, ow, oh, hdr, input_scale, out)
    return out


def unet_flops_per_pixel(in_channels: int) -> int:
    """2 * MACs per level-0 network pixel over logical channels."""
    flops = 0.0
    level = 0
    for (_name, _src, skip, cout, pool, _relu), (cin, _) in zip(UNET_LAYERS,
                                                                 unet_layer_shapes(in_channels)):
        if skip is not None:          # a decoder conv runs at its skip's (finer) level
            level -= 1
        flops += 2 * 9 * cin * cout / 4 ** level
        if pool:
            level += 1
    return int(round(flops))


def max_rel_error(got, ref) -> float:
    """max_i |g_i - o_i| / max_j |o_j| over finite reference entries."""
    g = np.asarray(got, np.float64)
    o = np.asarray(ref, np.float64)
    scale = np.max(np.abs(o))
    if scale == 0:
        return float(np.max(np.abs(g - o)))
    return float(np.max(np.abs(g - o)) / scale)
