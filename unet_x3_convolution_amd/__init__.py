"""Python binding of liboidn_mi355x (the MI355X OIDN-style UNet denoiser).

Argument marshalling only: every call goes through the C ABI declared in
include/oidn_mi355x.h, and every step of the hot path runs in the library's
HIP kernels.  Tensor arguments may be torch tensors (their data_ptr() is
passed) or raw integer device addresses; `stream` defaults to torch's current
stream.  A non-zero status raises OidnError with the library's message.
There is no fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboidn_mi355x.so")

OIDN_OK = 0
OIDN_E_INVALID = -1
OIDN_E_UNSUPPORTED = -2
OIDN_E_WORKSPACE = -3
OIDN_E_HIP = -4

OIDN_F32 = 0
OIDN_F16 = 1
OIDN_BF16 = 2

OIDN_RELU = 1
OIDN_POOL2X2 = 2

OIDN_TRANSFER_PU = 0
OIDN_TRANSFER_LOG = 1

OIDN_TILE_ALIGN = 16
OIDN_DEFAULT_OVERLAP = 96
OIDN_NOALLOC_SCRATCH_MB = 64

EXPORTS = (
    "oidn_last_error", "oidn_version", "oidn_conv3x3_weights_bytes",
    "oidn_conv3x3_pack_weights", "oidn_conv3x3_pack_weights_host", "oidn_conv3x3", "oidn_conv3x3_upcat", "oidn_pool2x2",
    "oidn_upsample_concat", "oidn_pack_input", "oidn_unpack_output", "oidn_plan_tiles",
    "oidn_conv3x3_pair", "oidn_conv3x3_kernel", "oidn_unet_layer_count", "oidn_unet_layer_info", "oidn_unet_layer_kernel",
    "oidn_unet_weights_bytes",
    "oidn_unet_pack_weights", "oidn_unet_packed_workspace_bytes", "oidn_unet_forward_packed",
    "oidn_unet_workspace_bytes", "oidn_unet_tile_batch", "oidn_unet_input_layout",
    "oidn_unet_forward",
    "oidn_unet_forward_timed", "oidn_unet_forward_noalloc", "oidn_unet_noalloc_scratch_bytes",
    "oidn_calibrate_mfma", "oidn_calibrate_read", "oidn_event_create", "oidn_event_destroy", "oidn_event_elapsed_ms",
)


class OidnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"oidn status {code}: {message}")
        self.code = code


class oidn_tile(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("in_x", "in_y", "in_w", "in_h", "out_x", "out_y", "out_w", "out_h")]

    def as_tuple(self):
        return tuple(getattr(self, n) for n, _ in self._fields_)


_lib = None
_vp, _i, _u, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "oidn_last_error": ([], ctypes.c_char_p),
    "oidn_version": ([], _i),
    "oidn_conv3x3_weights_bytes": ([_i, _i, _i, _i, ctypes.POINTER(_sz)], _i),
    "oidn_conv3x3_pack_weights": ([_vp, _vp, _i, _i, _i, _i, _vp, _vp], _i),
    "oidn_conv3x3_pack_weights_host": ([_vp, _vp, _i, _i, _i, _i, _vp], _i),
    "oidn_conv3x3": ([_vp, _i, _i, _i, _vp, _vp, _i, _i, _i, _u, _vp], _i),
    "oidn_conv3x3_upcat": ([_vp, _i, _vp, _i, _i, _i, _vp, _vp, _i, _i, _i, _u, _vp], _i),
    "oidn_pool2x2": ([_vp, _i, _i, _i, _vp, _i, _vp], _i),
    "oidn_upsample_concat": ([_vp, _i, _vp, _i, _i, _i, _vp, _i, _vp], _i),
    "oidn_pack_input": ([_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _i, _vp], _i),
    "oidn_unpack_output": ([_vp, _i, _i, _i, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp,
                            _vp], _i),
    "oidn_plan_tiles": ([_i, _i, _i, _i, ctypes.POINTER(oidn_tile), _i, ctypes.POINTER(_i)], _i),
    "oidn_unet_layer_count": ([], _i),
    "oidn_unet_layer_info": ([_i, _i, ctypes.POINTER(_i), ctypes.POINTER(_i), ctypes.POINTER(_i),
                              ctypes.POINTER(_i), ctypes.POINTER(_u),
                              ctypes.POINTER(ctypes.c_char_p)], _i),
    "oidn_unet_layer_kernel": ([_i, _i, _i, _i, _i, _i, ctypes.c_char_p, _i, ctypes.POINTER(_i)], _i),
    "oidn_conv3x3_pair": ([_vp, _i, _i, _i, _vp, _vp, _vp, _i, _i, _u, _vp], _i),
    "oidn_conv3x3_kernel": ([_i, _i, _i, _i, _i, _i, _i, _u, ctypes.c_char_p, _i,
                             ctypes.POINTER(_i)], _i),
    "oidn_unet_weights_bytes": ([_i, _i, ctypes.POINTER(_sz)], _i),
    "oidn_unet_pack_weights": ([ctypes.POINTER(_vp), ctypes.POINTER(_vp), _i, _i, _vp, _vp], _i),
    "oidn_unet_packed_workspace_bytes": ([_i, _i, _i, _i, ctypes.POINTER(_sz)], _i),
    "oidn_unet_forward_packed": ([_vp, _i, _vp, _i, _i, _vp, _sz, _vp, _i, _vp], _i),
    "oidn_unet_workspace_bytes": ([_i, _i, _i, _i, _i, _i, ctypes.POINTER(_sz)], _i),
    "oidn_unet_tile_batch": ([_i, _i, _i, _i, _i, _i, ctypes.POINTER(_i)], _i),
    "oidn_unet_input_layout": ([_i, _i, _i, _i, _i, _i, ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                ctypes.POINTER(_i), ctypes.POINTER(_i)], _i),
    "oidn_unet_forward": ([_vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp, _i,
                           _vp], _i),
    "oidn_unet_forward_timed": ([_vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp,
                                 _i, _vp, ctypes.POINTER(_vp), _i], _i),
    "oidn_unet_forward_noalloc": ([_vp, _i, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _i, _vp, _i,
                                   _vp], _i),
    "oidn_unet_noalloc_scratch_bytes": ([ctypes.POINTER(_sz)], _i),
    "oidn_calibrate_mfma": ([_i, ctypes.c_long, _i, _vp, ctypes.POINTER(ctypes.c_longlong), _vp], _i),
    "oidn_calibrate_read": ([_vp, _sz, _vp, _vp], _i),
    "oidn_event_create": ([ctypes.POINTER(_vp)], _i),
    "oidn_event_destroy": ([_vp], _i),
    "oidn_event_elapsed_ms": ([_vp, _vp, ctypes.POINTER(_f)], _i),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OidnError(OIDN_E_HIP, f"{LIB_PATH} is not built; run __graft_entry__.build()")
        # torch ships its own HIP runtime with the same soname; loading torch
        # first makes the library bind to that one instead of mapping a second
        # runtime (which would see no device and could not use torch's memory).
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        _check_single_hip_runtime()
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check_single_hip_runtime():
    try:
        maps = open("/proc/self/maps").read()
    except OSError:
        return
    runtimes = {line.split()[-1] for line in maps.splitlines()
                if "libamdhip64" in line and line.split()[-1].startswith("/")}
    if len(runtimes) > 1:
        raise OidnError(OIDN_E_HIP, "two HIP runtimes are loaded in this process: "
                        + ", ".join(sorted(runtimes)))


def last_error() -> str:
    return lib().oidn_last_error().decode()


def _check(rc: int):
    if rc != OIDN_OK:
        raise OidnError(rc, last_error())


def _p(t):
    """Device address of a tensor (or int / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ convs
def oidn_conv3x3_weights_bytes(cin0: int, cin1: int, cout: int, dtype: int) -> int:
    n = _sz()
    _check(lib().oidn_conv3x3_weights_bytes(cin0, cin1, cout, dtype, ctypes.byref(n)))
    return n.value


def oidn_conv3x3_pack_weights(w_ohwi, bias, cin0: int, cin1: int, cout: int, dtype: int,
                              d_packed, stream=None):
    """w_ohwi, bias: host numpy float32 arrays (C-contiguous)."""
    import numpy as np
    w = np.ascontiguousarray(w_ohwi, dtype=np.float32)
    b = np.ascontiguousarray(bias, dtype=np.float32)
    if w.size != cout * 9 * (cin0 + cin1) or b.size != cout:
        raise OidnError(OIDN_E_INVALID, "weight or bias size does not match the shape")
    _check(lib().oidn_conv3x3_pack_weights(w.ctypes.data, b.ctypes.data, cin0, cin1, cout, dtype,
                                           _p(d_packed), _s(stream)))


def oidn_conv3x3_pack_weights_host(w_ohwi, bias, cin0: int, cin1: int, cout: int, dtype: int):
    """Packed bytes (numpy uint8) of the device layout, built on the host."""
    import numpy as np
    w = np.ascontiguousarray(w_ohwi, dtype=np.float32)
    b = np.ascontiguousarray(bias, dtype=np.float32)
    if w.size != cout * 9 * (cin0 + cin1) or b.size != cout:
        raise OidnError(OIDN_E_INVALID, "weight or bias size does not match the shape")
    out = np.zeros(oidn_conv3x3_weights_bytes(cin0, cin1, cout, dtype), np.uint8)
    _check(lib().oidn_conv3x3_pack_weights_host(w.ctypes.data, b.ctypes.data, cin0, cin1, cout,
                                                dtype, out.ctypes.data))
    return out


def oidn_conv3x3(x, h: int, w: int, cin: int, w_packed, y, cout: int, in_dtype: int,
                 out_dtype: int, flags: int, stream=None):
    _check(lib().oidn_conv3x3(_p(x), h, w, cin, _p(w_packed), _p(y), cout, in_dtype, out_dtype,
                              flags, _s(stream)))


def oidn_conv3x3_upcat(low, c_low: int, skip, c_skip: int, h: int, w: int, w_packed, y,
                       cout: int, in_dtype: int, out_dtype: int, flags: int, stream=None):
    _check(lib().oidn_conv3x3_upcat(_p(low), c_low, _p(skip), c_skip, h, w, _p(w_packed), _p(y),
                                    cout, in_dtype, out_dtype, flags, _s(stream)))


def oidn_conv3x3_pair(x, h: int, w: int, cin: int, wa_packed, wb_packed, y, cout: int,
                      out_dtype: int, flags: int, stream=None):
    _check(lib().oidn_conv3x3_pair(_p(x), h, w, cin, _p(wa_packed), _p(wb_packed), _p(y), cout,
                                   out_dtype, flags, _s(stream)))


# ------------------------------------------------------------ elementwise
def oidn_pool2x2(x, h: int, w: int, c: int, y, dtype: int, stream=None):
    _check(lib().oidn_pool2x2(_p(x), h, w, c, _p(y), dtype, _s(stream)))


def oidn_upsample_concat(low, c_low: int, skip, c_skip: int, h: int, w: int, z, dtype: int,
                         stream=None):
    _check(lib().oidn_upsample_concat(_p(low), c_low, _p(skip), c_skip, h, w, _p(z), dtype,
                                      _s(stream)))


def oidn_pack_input(color, albedo, normal, img_w: int, img_h: int, tile_x: int, tile_y: int,
                    tile_w: int, tile_h: int, hdr: bool, transfer: int, input_scale: float,
                    packed, dtype: int, stream=None):
    _check(lib().oidn_pack_input(_p(color), _p(albedo), _p(normal), img_w, img_h, tile_x, tile_y,
                                 tile_w, tile_h, int(hdr), transfer, input_scale, _p(packed),
                                 dtype, _s(stream)))


def oidn_unpack_output(net_rgba, tile_w: int, tile_h: int, in_off_x: int, in_off_y: int, color,
                       img_w: int, img_h: int, out_x: int, out_y: int, out_w: int, out_h: int,
                       hdr: bool, transfer: int, input_scale: float, out_rgba, stream=None):
    _check(lib().oidn_unpack_output(_p(net_rgba), tile_w, tile_h, in_off_x, in_off_y, _p(color),
                                    img_w, img_h, out_x, out_y, out_w, out_h, int(hdr), transfer,
                                    input_scale, _p(out_rgba), _s(stream)))


# ---------------------------------------------------------------- tiles
def oidn_plan_tiles(w: int, h: int, max_tile: int, overlap: int):
    """List of (in_x, in_y, in_w, in_h, out_x, out_y, out_w, out_h)."""
    count = _i()
    _check(lib().oidn_plan_tiles(w, h, max_tile, overlap, None, 0, ctypes.byref(count)))
    arr = (oidn_tile * max(count.value, 1))()
    _check(lib().oidn_plan_tiles(w, h, max_tile, overlap, arr, count.value, ctypes.byref(count)))
    return [arr[i].as_tuple() for i in range(count.value)]


# ----------------------------------------------------------------- UNet
def oidn_unet_layer_count() -> int:
    return lib().oidn_unet_layer_count()


def oidn_unet_layer_info(in_channels: int, layer: int):
    """(name, cin0, cin1, cout, level, flags)."""
    c0, c1, co, lv, fl, nm = _i(), _i(), _i(), _i(), _u(), ctypes.c_char_p()
    _check(lib().oidn_unet_layer_info(in_channels, layer, ctypes.byref(c0), ctypes.byref(c1),
                                      ctypes.byref(co), ctypes.byref(lv), ctypes.byref(fl),
                                      ctypes.byref(nm)))
    return nm.value.decode(), c0.value, c1.value, co.value, lv.value, fl.value


def oidn_conv3x3_kernel(h: int, w: int, cin0: int, cin1: int, cout: int, in_dtype: int,
                        out_dtype: int, flags: int):
    """(kernel instance name, workgroups) of one conv (cin1 > 0: decoder conv)."""
    buf = ctypes.create_string_buffer(128)
    nb = _i()
    _check(lib().oidn_conv3x3_kernel(h, w, cin0, cin1, cout, in_dtype, out_dtype, flags, buf, 128,
                                     ctypes.byref(nb)))
    return buf.value.decode(), nb.value


def oidn_unet_layer_kernel(in_channels: int, layer: int, tw: int, th: int, dtype: int,
                           batch: int = 1):
    """(kernel instance name, workgroups) of a layer on `batch` tw x th tiles
    per launch."""
    buf = ctypes.create_string_buffer(128)
    nb = _i()
    _check(lib().oidn_unet_layer_kernel(in_channels, layer, tw, th, batch, dtype, buf, 128,
                                        ctypes.byref(nb)))
    return buf.value.decode(), nb.value


def unet_layer_shapes(in_channels: int):
    """[(cin_logical, cout)] of the library's layer table."""
    out = []
    for i in range(oidn_unet_layer_count()):
        _, c0, c1, co, _, _ = oidn_unet_layer_info(in_channels, i)
        out.append((c0 + c1, co))
    return out


def oidn_unet_weights_bytes(in_channels: int, dtype: int) -> int:
    n = _sz()
    _check(lib().oidn_unet_weights_bytes(in_channels, dtype, ctypes.byref(n)))
    return n.value


def oidn_unet_pack_weights(weights, biases, in_channels: int, dtype: int, d_weights, stream=None):
    """weights[i]: host float32 OHWI array of layer i; biases[i]: host float32 array."""
    import numpy as np
    ws = [np.ascontiguousarray(w, dtype=np.float32) for w in weights]
    bs = [np.ascontiguousarray(b, dtype=np.float32) for b in biases]
    n = oidn_unet_layer_count()
    if len(ws) != n or len(bs) != n:
        raise OidnError(OIDN_E_INVALID, f"expected {n} weight and bias arrays")
    for i, ((cin, cout), w, b) in enumerate(zip(unet_layer_shapes(in_channels), ws, bs)):
        if w.shape != (cout, 3, 3, cin) or b.shape != (cout,):
            raise OidnError(OIDN_E_INVALID, f"layer {i}: expected weights {(cout, 3, 3, cin)}")
    wp = (_vp * n)(*[w.ctypes.data for w in ws])
    bp = (_vp * n)(*[b.ctypes.data for b in bs])
    _check(lib().oidn_unet_pack_weights(wp, bp, in_channels, dtype, _p(d_weights), _s(stream)))


def oidn_unet_packed_workspace_bytes(in_channels: int, tw: int, th: int, dtype: int) -> int:
    n = _sz()
    _check(lib().oidn_unet_packed_workspace_bytes(in_channels, tw, th, dtype, ctypes.byref(n)))
    return n.value


def oidn_unet_forward_packed(d_weights, in_channels: int, packed_in, tw: int, th: int, workspace,
                             ws_bytes: int, net_out_rgba, dtype: int, stream=None):
    _check(lib().oidn_unet_forward_packed(_p(d_weights), in_channels, _p(packed_in), tw, th,
                                          _p(workspace), ws_bytes, _p(net_out_rgba), dtype,
                                          _s(stream)))


def oidn_unet_workspace_bytes(in_channels: int, w: int, h: int, max_tile: int, overlap: int,
                              dtype: int) -> int:
    n = _sz()
    _check(lib().oidn_unet_workspace_bytes(in_channels, w, h, max_tile, overlap, dtype,
                                           ctypes.byref(n)))
    return n.value


def oidn_unet_tile_batch(in_channels: int, w: int, h: int, max_tile: int, overlap: int,
                         dtype: int) -> int:
    n = _i()
    _check(lib().oidn_unet_tile_batch(in_channels, w, h, max_tile, overlap, dtype, ctypes.byref(n)))
    return n.value


def oidn_unet_input_layout(in_channels: int, w: int, h: int, max_tile: int, overlap: int,
                           dtype: int):
    """(offset, tile_stride, lanes, taps) of the packed network input that
    oidn_unet_forward leaves in its workspace."""
    off, stride, lanes, taps = _sz(), _sz(), _i(), _i()
    _check(lib().oidn_unet_input_layout(in_channels, w, h, max_tile, overlap, dtype,
                                        ctypes.byref(off), ctypes.byref(stride),
                                        ctypes.byref(lanes), ctypes.byref(taps)))
    return off.value, stride.value, lanes.value, bool(taps.value)


def oidn_unet_forward(d_weights, in_channels: int, color, albedo, normal, w: int, h: int,
                      hdr: bool, transfer: int, input_scale: float, max_tile: int, overlap: int,
                      workspace, ws_bytes: int, out_rgba, dtype: int, stream=None):
    _check(lib().oidn_unet_forward(_p(d_weights), in_channels, _p(color), _p(albedo), _p(normal),
                                   w, h, int(hdr), transfer, input_scale, max_tile, overlap,
                                   _p(workspace), ws_bytes, _p(out_rgba), dtype, _s(stream)))


def oidn_unet_forward_timed(d_weights, in_channels: int, color, albedo, normal, w: int, h: int,
                            hdr: bool, transfer: int, input_scale: float, max_tile: int,
                            overlap: int, workspace, ws_bytes: int, out_rgba, dtype: int, events,
                            stream=None):
    ev = (_vp * len(events))(*events)
    _check(lib().oidn_unet_forward_timed(_p(d_weights), in_channels, _p(color), _p(albedo),
                                         _p(normal), w, h, int(hdr), transfer, input_scale,
                                         max_tile, overlap, _p(workspace), ws_bytes,
                                         _p(out_rgba), dtype, _s(stream), ev, len(events)))


def oidn_unet_forward_noalloc(d_weights, in_channels: int, color, albedo, normal, w: int, h: int,
                              hdr: bool, transfer: int, input_scale: float, max_tile: int,
                              overlap: int, out_rgba, dtype: int, stream=None):
    _check(lib().oidn_unet_forward_noalloc(_p(d_weights), in_channels, _p(color), _p(albedo),
                                           _p(normal), w, h, int(hdr), transfer, input_scale,
                                           max_tile, overlap, _p(out_rgba), dtype, _s(stream)))


def oidn_unet_noalloc_scratch_bytes() -> int:
    n = _sz()
    _check(lib().oidn_unet_noalloc_scratch_bytes(ctypes.byref(n)))
    return n.value


def oidn_calibrate_mfma(dtype: int, iters: int, blocks: int, sink, stream=None) -> int:
    """Launches the MFMA stream; returns its FLOPs."""
    n = ctypes.c_longlong()
    _check(lib().oidn_calibrate_mfma(dtype, iters, blocks, _p(sink), ctypes.byref(n), _s(stream)))
    return n.value


def oidn_calibrate_read(buf, nbytes: int, sink, stream=None):
    _check(lib().oidn_calibrate_read(_p(buf), nbytes, _p(sink), _s(stream)))


def oidn_event_create() -> int:
    e = _vp()
    _check(lib().oidn_event_create(ctypes.byref(e)))
    return e.value


def oidn_event_destroy(event: int):
    _check(lib().oidn_event_destroy(event))


def oidn_event_elapsed_ms(start: int, end: int) -> float:
    ms = _f()
    _check(lib().oidn_event_elapsed_ms(start, end, ctypes.byref(ms)))
    return ms.value
