"""Helpers for the GPU parity tests: host <-> device copies and packing
through the C ABI.  Tolerances follow the contract: max_i |g - o| / max |o|
within 1e-5 (fp32 storage) or 2e-2 (fp16 storage, fp32 accumulate).  bf16
storage has no stated bound: the fp16 one scaled by the ratio of the two
formats' unit roundoffs, 2^-8 / 2^-11 = 8, since both sides round every
stored value the same way and differ only where fp32 and float64 sums round
to different neighbours."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import unet_x3_convolution_amd as U  # noqa: E402

TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 8 * 2e-2}
DT = {"f32": U.OIDN_F32, "f16": U.OIDN_F16, "bf16": U.OIDN_BF16}


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    U.lib()  # loud failure if the HIP library is missing
    return torch


def dev(a):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def empty(shape, np_dtype, fill=None):
    torch = torch_cuda()
    tdt = {np.float16: torch.float16, np.float32: torch.float32, np.uint8: torch.uint8}[np_dtype]
    t = torch.empty(shape, dtype=tdt, device="cuda")
    if fill is not None:
        t.fill_(fill)
    return t


def host(t):
    torch = torch_cuda()
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()   # exact
    return t.cpu().numpy()


def to_dev(a, precision):
    """Stored values (the oracle's storage arrays) to a device tensor of the
    precision's storage type; bf16 values are exact in both."""
    if precision == "bf16":
        torch = torch_cuda()
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).cuda()
    return dev(np.asarray(a, {"f16": np.float16, "f32": np.float32}[precision]))


def alloc(shape, precision, fill=None):
    """Device buffer of the precision's storage type."""
    if precision == "bf16":
        torch = torch_cuda()
        t = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        if fill is not None:
            t.fill_(fill)
        return t
    return empty(shape, {"f16": np.float16, "f32": np.float32}[precision], fill)


def packed_conv(w, b, cin0, cin1, cout, precision):
    dtype = DT[precision]
    buf = empty((U.oidn_conv3x3_weights_bytes(cin0, cin1, cout, dtype),), np.uint8)
    U.oidn_conv3x3_pack_weights(w, b, cin0, cin1, cout, dtype, buf)
    return buf


def packed_unet(ws, bs, in_channels, precision):
    dtype = DT[precision]
    buf = empty((U.oidn_unet_weights_bytes(in_channels, dtype),), np.uint8)
    U.oidn_unet_pack_weights(ws, bs, in_channels, dtype, buf)
    return buf


def rel_err(got, ref):
    g = np.asarray(got, np.float64)
    o = np.asarray(ref, np.float64)
    scale = np.max(np.abs(o))
    return float(np.max(np.abs(g - o)) / scale) if scale > 0 else float(np.max(np.abs(g - o)))


def ulp_diff_f16(a, b):
    """|difference| in units of fp16 ordering (0 = identical bits)."""
    def key(x):
        i = np.asarray(x, np.float16).view(np.int16).astype(np.int32)
        return np.where(i < 0, -(i & 0x7FFF), i)
    return np.abs(key(a) - key(b))


def ulp_diff_bf16(a, b):
    """|difference| in units of bf16 ordering, for float32 arrays holding
    bf16 values (0 = identical bits)."""
    def key(x):
        i = (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.int32)
        return np.where(i >= 0x8000, -(i & 0x7FFF), i)
    return np.abs(key(a) - key(b))


def ulp_diff(a, b, precision):
    return ulp_diff_bf16(a, b) if precision == "bf16" else ulp_diff_f16(a, b)


def say(*args):
    print(*args, flush=True)
