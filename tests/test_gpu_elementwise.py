"""GPU parity of the bandwidth-bound passes (pool, upsample-concat, input
pack, output unpack) against the CPU oracle, through the C ABI."""
import math

import numpy as np
import pytest

import synthetic as S
import unet_x3_convolution_amd as U
from helpers import DT, alloc, dev, empty, host, say, to_dev, ulp_diff, ulp_diff_f16
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("h,w,c,precision", [(6, 10, 12, "f16"), (128, 64, 48, "f16"),
                                             (2, 2, 4, "f32"), (40, 18, 9, "f32"),
                                             (6, 10, 12, "bf16"), (128, 64, 48, "bf16"),
                                             # more output rows than one launch's grid
                                             # holds: the kernel steps over the rest
                                             (70002, 4, 8, "f16"), (65540, 2, 4, "bf16")])
def test_pool_bit_exact(h, w, c, precision):
    r = np.random.default_rng(h * w)
    x = np.zeros((h, w, O.stored(c)), O.np_storage(precision))
    x[..., :c] = O.round_to(r.standard_normal((h, w, c)), precision)
    y = alloc((h // 2, w // 2, O.stored(c)), precision, fill=float("nan"))
    U.oidn_pool2x2(to_dev(x, precision), h, w, c, y, DT[precision])
    assert np.array_equal(host(y), O.pool2x2(x))


@pytest.mark.parametrize("h,w,c_low,c_skip,precision", [(16, 16, 96, 64, "f16"),
                                                        (6, 10, 8, 9, "f16"),
                                                        (4, 2, 4, 3, "f32"),
                                                        (6, 10, 8, 9, "bf16"),
                                                        # rows past one launch's grid
                                                        (140004, 4, 4, 3, "f16"),
                                                        (140002, 2, 8, 9, "f32")])
def test_upsample_concat_bit_exact(h, w, c_low, c_skip, precision):
    r = np.random.default_rng(h + c_low)
    low = O.round_to(r.standard_normal((h // 2, w // 2, c_low)), precision)
    skip = np.zeros((h, w, O.stored(c_skip)), O.np_storage(precision))
    skip[..., :c_skip] = O.round_to(r.standard_normal((h, w, c_skip)), precision)
    z = alloc((h, w, c_low + O.stored(c_skip)), precision, fill=float("nan"))
    U.oidn_upsample_concat(to_dev(low, precision), c_low, to_dev(skip, precision), c_skip, h, w,
                           z, DT[precision])
    assert np.array_equal(host(z), O.upsample_concat(low, c_low, skip, c_skip))


def _gpu_pack(color, albedo, normal, rect, hdr, scale, precision):
    img_h, img_w = color.shape[:2]
    tx, ty, tw, th = rect
    ch = 3 * (1 + (albedo is not None) + (normal is not None))
    out = alloc((th, tw, O.stored(ch)), precision, fill=float("nan"))
    U.oidn_pack_input(dev(color), None if albedo is None else dev(albedo),
                      None if normal is None else dev(normal), img_w, img_h, tx, ty, tw, th, hdr,
                      U.OIDN_TRANSFER_LOG, scale, out, DT[precision])
    return host(out)


@pytest.mark.parametrize("sources", [1, 2, 3])
@pytest.mark.parametrize("precision", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("hdr", [True, False])
def test_pack_matches_oracle(sources, precision, hdr):
    r = S.rng(sources)
    color, albedo, normal = S.images(r, 37, 29)
    if not hdr:
        color[..., :3] = r.uniform(-0.2, 1.2, color[..., :3].shape)
    albedo = albedo if sources > 1 else None
    normal = normal if sources > 2 else None
    scale = 0.5 if hdr else 1.0
    # whole 64-pixel waves only, and 1073 pixels (16 whole waves and a
    # partial one: the LDS store path and the per-lane stores in one launch)
    for rect in [(0, 0, 48, 32), (-5, -3, 16, 48), (20, 10, 32, 32), (3, 2, 37, 29)]:
        got = _gpu_pack(color, albedo, normal, rect, hdr, scale, precision)
        ref = O.pack_input(color, albedo, normal, *rect, hdr, scale, precision)
        assert got.shape == ref.shape
        # layout, zero lanes, albedo, normal and LDR colour: bit-exact
        exact = got.copy()
        if hdr:
            exact[..., :3] = ref[..., :3]
        assert np.array_equal(exact, ref), rect
        if hdr:  # log1p on the device vs float64 on the host: <= 1 ulp of the stored type
            if precision != "f32":
                assert ulp_diff(got[..., :3], ref[..., :3], precision).max() <= 1
            else:
                np.testing.assert_allclose(got[..., :3], ref[..., :3], rtol=3e-7, atol=0)


def test_pack_special_values():
    inf, nan = np.float32(np.inf), np.float32(np.nan)
    color = np.array([[[nan, -1.0, inf, 0.5], [0.0, 1e30, 3.0, 0.25]]], np.float32)
    albedo = np.array([[[nan, 2.0, -3.0, 1.0], [0.5, 0.25, 1.0, 0.0]]], np.float32)
    normal = np.array([[[nan, -5.0, 5.0, 0.0], [-1.0, 0.0, 1.0, 0.0]]], np.float32)
    for precision in ["f16", "bf16", "f32"]:
        got = _gpu_pack(color, albedo, normal, (0, 0, 2, 1), True, 1.0, precision)
        ref = O.pack_input(color, albedo, normal, 0, 0, 2, 1, True, 1.0, precision)
        assert got[0, 0, 0] == 0 and got[0, 0, 1] == 0
        assert np.array_equal(got[..., 3:], ref[..., 3:])
        if precision != "f32":
            assert ulp_diff(got[..., :3], ref[..., :3], precision).max() <= 1
        else:
            np.testing.assert_allclose(got[..., :3], ref[..., :3], rtol=3e-7)
    assert math.isclose(float(got[0, 0, 2]), math.log1p(O.FLT_MAX), rel_tol=1e-6)


@pytest.mark.parametrize("precision", ["f16", "bf16", "f32"])
def test_pack_hdr_transfer_across_the_float_range(precision):
    """The HDR log transfer over every binade of fp32 (and densely where
    1 + x rounds away most of x): the stored channel is the correctly
    rounded log1p or its neighbour in the 16-bit types, and almost always
    the correctly rounded one; within 3e-7 in fp32."""
    r = np.random.default_rng(77)
    h, w = 64, 128
    n = h * w * 3
    wide = np.exp2(r.uniform(-149, 128, n // 2))
    small = np.exp2(r.uniform(-30, -8, n // 4))
    edges = (np.exp2(np.arange(-30.0, 30.0))[:, None] * np.array([1 - 2**-24, 1, 1 + 2**-23])).ravel()
    rest = np.concatenate([edges, [O.FLT_MAX, 0.0, 1.0, 2**-24, 2**-25]])
    tail = r.uniform(0, 4, n - len(wide) - len(small) - len(rest))
    vals = np.concatenate([wide, small, rest, tail]).astype(np.float32)
    vals = np.minimum(vals, np.float32(O.FLT_MAX))
    color = np.ones((h, w, 4), np.float32)
    color[..., :3] = vals.reshape(h, w, 3)
    got = _gpu_pack(color, None, None, (0, 0, w, h), True, 1.0, precision)[..., :3]
    ref = O.pack_input(color, None, None, 0, 0, w, h, True, 1.0, precision)[..., :3]
    if precision == "f32":
        np.testing.assert_allclose(got, ref, rtol=3e-7, atol=0)
        return
    d = ulp_diff(got, ref, precision)
    say(f"{precision}: {np.count_nonzero(d)} of {d.size} one ulp off")
    assert d.max() <= 1
    assert np.count_nonzero(d) <= d.size // 200


@pytest.mark.parametrize("hdr", [True, False])
def test_unpack_matches_oracle(hdr):
    r = S.rng(9)
    color, _, _ = S.images(r, 40, 30)
    net = r.standard_normal((48, 64, 4)).astype(np.float32) * 3
    net[5, 3, :3] = [np.nan, -np.inf, np.inf]   # first pixel read
    rect = (3, 5, 2, 4, 33, 21)  # in_off_x, in_off_y, out_x, out_y, out_w, out_h
    scale = 0.75 if hdr else 1.0
    out = empty((30, 40, 4), np.float32, fill=-7.0)
    U.oidn_unpack_output(dev(net), 64, 48, rect[0], rect[1], dev(color), 40, 30, rect[2], rect[3],
                         rect[4], rect[5], hdr, U.OIDN_TRANSFER_LOG, scale, out)
    got = host(out)
    ref = np.full((30, 40, 4), -7.0, np.float32)
    O.unpack_output(net, rect[0], rect[1], color, rect[2], rect[3], rect[4], rect[5], hdr, scale, ref)
    inside = np.zeros((30, 40), bool)
    inside[rect[3]:rect[3] + rect[5], rect[2]:rect[2] + rect[4]] = True
    assert np.all(got[~inside] == -7.0)
    assert np.array_equal(got[..., 3], ref[..., 3])
    g, o = got[inside][:, :3], ref[inside][:, :3]
    finite = np.isfinite(o)
    assert np.array_equal(np.isfinite(g), finite)
    np.testing.assert_allclose(g[finite], o[finite], rtol=2e-6, atol=0)
    say(f"unpack hdr={hdr}: ok")
