"""The no-alloc denoise entry point (oidn_unet_forward_noalloc, workspace in
the library's static device array) against oidn_unet_forward with a caller
workspace, through the C ABI: the same bits, on calls in a row with shrinking
inputs (the array keeps the previous call's contents), one of them with
fewer tiles per launch than oidn_unet_forward runs."""
import numpy as np
import pytest

import synthetic as S
import unet_x3_convolution_amd as U
from helpers import DT, dev, empty, host, packed_unet, say

pytestmark = pytest.mark.gpu


def _case(w, h, seed):
    r = S.rng(seed)
    color, albedo, normal = S.images(r, w, h)
    ws, bs = S.layer_params(r, U.unet_layer_shapes(9))
    return color, albedo, normal, ws, bs


@pytest.mark.parametrize("precision", ["f16", "bf16"])
def test_noalloc_equals_forward_on_calls_in_a_row(precision):
    F = DT[precision]
    scratch = U.oidn_unet_noalloc_scratch_bytes()
    assert scratch == U.OIDN_NOALLOC_SCRATCH_MB << 20
    # (w, h, max_tile, overlap): 12 tiles of 224 x 224 whose batch of 12 does
    # not fit the array (fewer per launch), one whole 512 x 384 tile, then 12
    # tiles of 128 x 112
    cases = [(640, 480, 256, 32), (512, 384, 0, 32), (203, 141, 128, 32)]
    for k, (w, h, mt, ov) in enumerate(cases):
        color, albedo, normal, ws, bs = _case(w, h, seed=40 + k)
        wd = packed_unet(ws, bs, 9, precision)
        ntiles = len(U.oidn_plan_tiles(w, h, mt, ov))
        batch = U.oidn_unet_tile_batch(9, w, h, mt, ov, F)
        nbytes = U.oidn_unet_workspace_bytes(9, w, h, mt, ov, F)
        per_tile = nbytes // batch
        fits = min(batch, scratch // per_tile)
        if k == 0:
            assert fits < batch, (fits, batch)
        d_color, d_albedo, d_normal = dev(color), dev(albedo), dev(normal)
        work = empty((nbytes,), np.uint8)
        ref = empty((h, w, 4), np.float32, fill=float("nan"))
        U.oidn_unet_forward(wd, 9, d_color, d_albedo, d_normal, w, h, True, U.OIDN_TRANSFER_LOG,
                            0.9, mt, ov, work, nbytes, ref, F)
        got = empty((h, w, 4), np.float32, fill=float("nan"))
        U.oidn_unet_forward_noalloc(wd, 9, d_color, d_albedo, d_normal, w, h, True,
                                    U.OIDN_TRANSFER_LOG, 0.9, mt, ov, got, F)
        g, r = host(got), host(ref)
        assert not np.any(np.isnan(g))
        assert np.array_equal(g, r), (w, h, mt)
        say(f"no-alloc {precision} {w}x{h} ({ntiles} tiles, {fits} per launch of {batch}): "
            f"equal to oidn_unet_forward")


def test_noalloc_refuses_a_tile_larger_than_its_array():
    color, albedo, normal, ws, bs = _case(64, 64, seed=3)
    wd = packed_unet(ws, bs, 9, "f16")
    out = empty((1080, 1920, 4), np.float32, fill=5.0)
    big = empty((1080, 1920, 4), np.float32, fill=0.5)
    with pytest.raises(U.OidnError) as e:
        U.oidn_unet_forward_noalloc(wd, 9, big, big, big, 1920, 1080, True, U.OIDN_TRANSFER_LOG,
                                    1.0, 0, 32, out, U.OIDN_F16)
    assert e.value.code == U.OIDN_E_WORKSPACE and "no-alloc" in U.last_error()
    assert np.all(host(out) == 5.0)
