"""GPU parity of the 3x3 conv kernels (fp32 VALU and fp16 MFMA) against the
CPU oracle, through the C ABI, plus the conv invariants on the GPU."""
import numpy as np
import pytest

import synthetic as S
import unet_x3_convolution_amd as U
from helpers import DT, TOL, alloc, dev, empty, host, packed_conv, rel_err, say, to_dev, ulp_diff_f16
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def run_conv(x_np, cin, w, b, cout, precision, flags, out_precision=None):
    out_precision = out_precision or precision
    h, wd = x_np.shape[:2]
    pk = packed_conv(w, b, cin, 0, cout, precision)
    oh, ow = (h // 2, wd // 2) if flags & U.OIDN_POOL2X2 else (h, wd)
    y = alloc((oh, ow, O.stored(cout)), out_precision, fill=float("nan"))
    U.oidn_conv3x3(to_dev(x_np, precision), h, wd, cin, pk, y, cout, DT[precision],
                   DT[out_precision], flags)
    return host(y)


def oracle_conv(x_np, cin, w, b, cout, precision, flags, out_precision=None):
    y = O.conv3x3(x_np, cin, w, b, bool(flags & U.OIDN_RELU), precision, out_precision)
    return O.pool2x2(y) if flags & U.OIDN_POOL2X2 else y


def check(got, ref, cout, precision, label):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert not np.any(np.isnan(got)), f"{label}: unwritten outputs"
    assert np.all(got[..., cout:] == 0), f"{label}: pad lanes not zero"
    err = rel_err(got[..., :cout], ref[..., :cout])
    extra = ""
    if got.dtype == np.float16:
        extra = f" max_ulp={int(ulp_diff_f16(got, ref).max())}"
    say(f"{label}: max_rel_err={err:.3e}{extra}")
    assert err <= TOL[precision], (label, err)


def test_config1_single_conv_fp32():
    """64x64, 9 (12 stored) -> 32 channels, fp32, He-normal weights, seed 0."""
    r = S.rng(0)
    x = S.uniform_activation(r, 64, 64, 9, 12)
    w = S.he_normal(r, 32, 9)
    b = S.bias(r, 32)
    got = run_conv(x, 9, w, b, 32, "f32", U.OIDN_RELU)
    check(got, oracle_conv(x, 9, w, b, 32, "f32", U.OIDN_RELU), 32, "f32", "config1")


F16_CASES = [
    # h, w, cin, cout, flags, out precision
    (64, 64, 9, 32, U.OIDN_RELU, "f16"),
    (37, 23, 12, 3, 0, "f32"),                       # ragged tile edges, final-layer shape
    (16, 16, 32, 32, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),
    (50, 34, 48, 80, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),
    (18, 30, 76, 64, U.OIDN_RELU, "f16"),
    (33, 17, 5, 20, U.OIDN_RELU, "f16"),             # cout not a multiple of 16
    (24, 20, 160, 112, U.OIDN_RELU, "f16"),          # five K chunks, 7 output fragments
    (8, 8, 256, 128, U.OIDN_RELU, "f16"),            # channel limits
    (1, 1, 4, 4, 0, "f16"),
    (2, 2, 8, 16, U.OIDN_RELU | U.OIDN_POOL2X2, "f32"),
    (70, 3, 96, 96, U.OIDN_RELU, "f16"),
    (512, 1024, 32, 32, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),   # 32-row tiles, all fragments
    (520, 1030, 12, 64, U.OIDN_RELU, "f16"),                    # 32-row tiles, ragged edges
    # 16-byte patch loads (sources a multiple of 8 channels), many 32 x 16 tiles
    (544, 960, 16, 32, U.OIDN_RELU, "f16"),                     # 16-channel chunk, 2 fragments
    (520, 1030, 32, 3, 0, "f32"),                               # 1 fragment, fp32 out, ragged
    (512, 1000, 32, 48, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),   # 3 fragments, pooled, ragged
    (530, 1024, 64, 32, U.OIDN_RELU, "f16"),                    # two chunks per tile
    (544, 512, 32, 64, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),    # 4 fragments
    (546, 1002, 48, 64, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),   # ragged, 32 + 16 chunks, pooled
    (530, 1010, 32, 64, 0, "f32"),                              # ragged, fp32 out, no ReLU
    (544, 520, 96, 64, U.OIDN_RELU, "f16"),                     # three chunks per tile
    # one case per launch plan instance <fragments/wave, rows/wave, row groups>
    (272, 480, 48, 64, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),    # <2, 8, 2>
    (256, 512, 80, 64, U.OIDN_RELU, "f16"),                     # <2, 8, 2>: 3 chunks
    (128, 512, 80, 64, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),    # <1, 8, 1>
    (512, 480, 128, 64, U.OIDN_RELU, "f16"),                    # <4, 8, 4>: 4 chunks
    (272, 480, 96, 96, U.OIDN_RELU, "f16"),                     # <3, 8, 2>
    (256, 256, 64, 64, U.OIDN_RELU, "f16"),                     # <1, 8, 1>
    (256, 256, 32, 32, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),    # <1, 4, 2>
    (128, 256, 64, 128, U.OIDN_RELU, "f16"),                    # <2, 4, 2>, outputs split in two
    (256, 512, 32, 48, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),    # <3, 4, 4>
    (128, 512, 32, 48, U.OIDN_RELU, "f16"),                     # <3, 2, 4>
    (128, 512, 96, 96, U.OIDN_RELU, "f16"),                     # <3, 4, 2>
    (256, 512, 32, 128, U.OIDN_RELU, "f16"),                    # <4, 8, 2>
    (128, 512, 32, 128, U.OIDN_RELU, "f16"),                    # <4, 4, 2>
    (256, 512, 64, 80, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),    # <5, 4, 4>
    (256, 512, 32, 112, U.OIDN_RELU, "f16"),                    # <7, 4, 4>
    # cout inside a fragment pair: 16-byte stores must stop at cout_stored
    (544, 512, 32, 52, U.OIDN_RELU, "f16"),                     # <2, 16, 2>, pair (2, 3) partial
    (272, 480, 96, 84, U.OIDN_RELU, "f16"),                     # <3, 8, 2>, pair (4, 5) partial
    (256, 256, 64, 60, U.OIDN_RELU | U.OIDN_POOL2X2, "f16"),    # <1, 8, 1>
    (512, 480, 128, 60, U.OIDN_RELU, "f16"),                    # <4, 8, 4>, pair (2, 3) partial
]


@pytest.mark.parametrize("h,w,cin,cout,flags,outp", F16_CASES)
def test_conv_f16_matches_oracle(h, w, cin, cout, flags, outp):
    r = np.random.default_rng(1000 + h * 7 + cin)
    x = O.round_to(S.relu_normal_activation(r, h, w, cin, O.stored(cin)), "f16")
    wt = S.he_normal(r, cout, cin)
    b = S.bias(r, cout)
    got = run_conv(x, cin, wt, b, cout, "f16", flags, outp)
    check(got, oracle_conv(x, cin, wt, b, cout, "f16", flags, outp), cout, "f16",
          f"conv f16 {h}x{w} {cin}->{cout} flags={flags} out={outp}")


@pytest.mark.parametrize("h,w,cin,cout,flags,outp", F16_CASES)
def test_conv_bf16_matches_oracle(h, w, cin, cout, flags, outp):
    """The same shapes with bf16 storage (every launch plan instance)."""
    r = np.random.default_rng(2000 + h * 7 + cin)
    x = O.round_to(S.relu_normal_activation(r, h, w, cin, O.stored(cin)), "bf16")
    wt = S.he_normal(r, cout, cin)
    b = S.bias(r, cout)
    outp = "bf16" if outp == "f16" else outp
    got = run_conv(x, cin, wt, b, cout, "bf16", flags, outp)
    check(got, oracle_conv(x, cin, wt, b, cout, "bf16", flags, outp), cout, "bf16",
          f"conv bf16 {h}x{w} {cin}->{cout} flags={flags} out={outp}")


@pytest.mark.parametrize("h,w,cin,cout,flags", [(20, 18, 12, 8, U.OIDN_RELU),
                                                (10, 14, 40, 20, U.OIDN_RELU | U.OIDN_POOL2X2),
                                                (9, 5, 3, 3, 0),
                                                # three input chunks, two fragment groups
                                                # (7 fragments), ragged 16 x 16 tiles
                                                (37, 41, 72, 112, U.OIDN_RELU),
                                                (34, 50, 96, 96, U.OIDN_RELU | U.OIDN_POOL2X2),
                                                (64, 64, 9, 32, 0)])
def test_conv_f32_matches_oracle(h, w, cin, cout, flags):
    r = np.random.default_rng(h + cin)
    x = S.relu_normal_activation(r, h, w, cin, O.stored(cin))
    wt = S.he_normal(r, cout, cin)
    b = S.bias(r, cout)
    got = run_conv(x, cin, wt, b, cout, "f32", flags)
    check(got, oracle_conv(x, cin, wt, b, cout, "f32", flags), cout, "f32",
          f"conv f32 {h}x{w} {cin}->{cout} flags={flags}")


@pytest.mark.parametrize("precision", ["f16", "f32"])
def test_conv_delta_kernel_is_identity_on_gpu(precision):
    r = np.random.default_rng(5)
    c = 48
    x = O.round_to(np.abs(r.standard_normal((21, 19, c))), precision)
    w = np.zeros((c, 3, 3, c), np.float32)
    w[np.arange(c), 1, 1, np.arange(c)] = 1.0
    got = run_conv(x, c, w, np.zeros(c, np.float32), c, precision, U.OIDN_RELU)
    assert np.array_equal(got, x)


def test_conv_zero_padding_counts_on_gpu():
    cin, cout = 32, 16
    h, w = 19, 35
    x = np.ones((h, w, cin), np.float16)
    got = run_conv(x, cin, np.ones((cout, 3, 3, cin), np.float32), np.zeros(cout, np.float32),
                   cout, "f16", 0).astype(np.float64)
    rows = np.array([2] + [3] * (h - 2) + [2])
    cols = np.array([2] + [3] * (w - 2) + [2])
    expected = np.outer(rows, cols) * cin
    for o in range(cout):
        assert np.array_equal(got[..., o], expected)


def test_fused_pool_equals_conv_then_pool_bit_exact():
    r = np.random.default_rng(6)
    h, w, cin, cout = 34, 46, 32, 48
    x = O.round_to(S.relu_normal_activation(r, h, w, cin, cin), "f16")
    wt = S.he_normal(r, cout, cin)
    b = S.bias(r, cout)
    fused = run_conv(x, cin, wt, b, cout, "f16", U.OIDN_RELU | U.OIDN_POOL2X2)
    full = run_conv(x, cin, wt, b, cout, "f16", U.OIDN_RELU)
    y = empty((h // 2, w // 2, cout), np.float16)
    U.oidn_pool2x2(dev(full), h, w, cout, y, U.OIDN_F16)
    assert np.array_equal(fused, host(y))


UPCAT_CASES = [
    # h, w (output), c_low, c_skip, cout, precision
    (16, 16, 96, 64, 112, "f16"),
    (32, 48, 64, 9, 64, "f16"),
    (20, 12, 8, 5, 16, "f16"),
    (18, 26, 112, 48, 96, "f16"),
    (12, 10, 16, 9, 8, "f32"),
    (34, 46, 96, 64, 112, "f32"),                               # 6 input chunks, 2 fragment groups
    (30, 18, 64, 9, 64, "f32"),
    (512, 1024, 64, 9, 64, "f16"),                              # 32-row tiles
    (544, 960, 64, 16, 64, "f16"),                              # <4, 8, 4>: 16-channel skip, 3 chunks
    (546, 1002, 96, 32, 64, "f16"),                             # <4, 8, 4>, ragged, 4 chunks
    (514, 1026, 32, 16, 32, "f16"),                             # ragged
    (272, 480, 112, 48, 96, "f16"),                             # <3, 8, 2>: 2 row groups
    # one ragged case for every other instance an upsampled source can reach
    (238, 242, 96, 48, 24, "f16"),                              # <1, 4, 2>
    (130, 242, 112, 64, 120, "f16"),                            # <2, 4, 2>
    (466, 242, 48, 32, 56, "f16"),                              # <2, 8, 2>
    (466, 242, 64, 9, 40, "f16"),                               # <3, 4, 4>
    (226, 966, 32, 16, 40, "f16"),                              # <3, 8, 4>
    (466, 242, 32, 16, 120, "f16"),                             # <4, 8, 2>
    (466, 242, 96, 48, 72, "f16"),                              # <5, 4, 4>
    (466, 242, 48, 32, 104, "f16"),                             # <7, 4, 4>
]


# every fp16 case again with bf16 storage
UPCAT_CASES += [c[:5] + ("bf16",) for c in UPCAT_CASES if c[5] == "f16"]


@pytest.mark.parametrize("h,w,c_low,c_skip,cout,precision", UPCAT_CASES)
def test_decoder_conv_matches_oracle(h, w, c_low, c_skip, cout, precision):
    r = np.random.default_rng(h * w + c_low)
    low = O.round_to(S.relu_normal_activation(r, h // 2, w // 2, c_low, c_low), precision)
    skip = O.round_to(S.relu_normal_activation(r, h, w, c_skip, O.stored(c_skip)), precision)
    wt = S.he_normal(r, cout, c_low + c_skip)
    b = S.bias(r, cout)
    pk = packed_conv(wt, b, c_low, c_skip, cout, precision)
    y = alloc((h, w, O.stored(cout)), precision, fill=float("nan"))
    U.oidn_conv3x3_upcat(to_dev(low, precision), c_low, to_dev(skip, precision), c_skip, h, w, pk,
                         y, cout, DT[precision], DT[precision], U.OIDN_RELU)
    got = host(y)
    z = O.upsample_concat(low, c_low, skip, c_skip)
    ref = O.conv3x3(z, c_low + c_skip, wt, b, True, precision)
    check(got, ref, cout, precision, f"upcat conv {precision} {h}x{w} [{c_low}|{c_skip}]->{cout}")


def _random_cases(seed, n):
    """Seeded conv shapes across the kernel's regimes: ragged sizes, channel
    counts off the 4-, 8- and 16-lane grids, pooled or fp32 outputs, an
    upsampled source with a skip."""
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        upcat = bool(r.random() < 0.35)
        h = 2 * int(r.integers(1, 150))
        w = 2 * int(r.integers(1, 200))
        cin = 4 * int(r.integers(1, 33)) if upcat else int(r.integers(1, 161))
        cskip = int(r.integers(1, 65)) if upcat else 0
        cin = min(cin, 160 - cskip) if upcat else cin
        cout = int(r.integers(1, 129))
        pool = (not upcat) and bool(r.random() < 0.4)
        outp = "f32" if r.random() < 0.2 else None
        cases.append((h, w, cin, cskip, cout, pool, outp))
    return cases


@pytest.mark.parametrize("precision", ["f16", "bf16"])
@pytest.mark.parametrize("idx", range(12))
def test_conv_random_shapes(precision, idx):
    h, w, cin, cskip, cout, pool, outp = _random_cases(77 if precision == "f16" else 78, 12)[idx]
    outp = outp or precision
    r = np.random.default_rng(idx)
    wt = S.he_normal(r, cout, cin + cskip)
    b = S.bias(r, cout)
    flags = U.OIDN_RELU | (U.OIDN_POOL2X2 if pool else 0)
    name = U.oidn_conv3x3_kernel(h, w, cin, cskip, cout, DT[precision], DT[outp], flags)[0]
    label = f"random conv {precision} {h}x{w} [{cin}|{cskip}]->{cout} pool={pool} out={outp} {name}"
    say(label)
    if cskip:
        low = O.round_to(S.relu_normal_activation(r, h // 2, w // 2, cin, cin), precision)
        skip = O.round_to(S.relu_normal_activation(r, h, w, cskip, O.stored(cskip)), precision)
        pk = packed_conv(wt, b, cin, cskip, cout, precision)
        y = alloc((h, w, O.stored(cout)), outp, fill=float("nan"))
        U.oidn_conv3x3_upcat(to_dev(low, precision), cin, to_dev(skip, precision), cskip, h, w, pk,
                             y, cout, DT[precision], DT[outp], flags)
        got = host(y)
        ref = O.conv3x3(O.upsample_concat(low, cin, skip, cskip), cin + cskip, wt, b, True,
                        precision, outp)
    else:
        x = O.round_to(S.relu_normal_activation(r, h, w, cin, O.stored(cin)), precision)
        got = run_conv(x, cin, wt, b, cout, precision, flags, outp)
        ref = oracle_conv(x, cin, wt, b, cout, precision, flags, outp)
    check(got, ref, cout, precision, label)


def test_conv_ladder_config2():
    """256x256 fp16: 32->48->64->80->96->96, conv+ReLU then 2x2 pool per stage;
    each stage is checked against the oracle on the GPU's own stage input."""
    r = S.rng(0)
    x = O.round_to(S.relu_normal_activation(r, 256, 256, 32, 32), "f16")
    chans = [32, 48, 64, 80, 96, 96]
    flags = U.OIDN_RELU | U.OIDN_POOL2X2
    for i in range(5):
        cin, cout = chans[i], chans[i + 1]
        wt = S.he_normal(r, cout, cin)
        b = S.bias(r, cout)
        got = run_conv(x, cin, wt, b, cout, "f16", flags)
        check(got, oracle_conv(x, cin, wt, b, cout, "f16", flags), cout, "f16",
              f"ladder stage {i} {x.shape[0]}^2 {cin}->{cout}")
        x = got


@pytest.mark.parametrize("cin,full_kernel", [
    (32, "conv3x3_f16_mfma<2, 16, 2, false>"),   # one chunk: 32-row tiles, 2-fragment waves
    (128, "conv3x3_f16_mfma<4, 8, 4, false>"),   # four chunks: 4-fragment waves
])
def test_conv_result_independent_of_launch_plan_bit_exact(cin, full_kernel):
    """Large images run 32-row tiles with all output fragments per
    workgroup, small ones 8-row tiles with the outputs split across four
    workgroups;
    every output is accumulated in the same order either way, so a conv over
    a crop reproduces the interior of the conv over the image."""
    r = np.random.default_rng(7)
    h, w, cout = 544, 960, 64
    x = O.round_to(S.relu_normal_activation(r, h, w, cin, cin), "f16")
    wt = S.he_normal(r, cout, cin)
    b = S.bias(r, cout)
    assert U.oidn_conv3x3_kernel(h, w, cin, 0, cout, U.OIDN_F16, U.OIDN_F16, U.OIDN_RELU)[0] == \
        full_kernel
    assert U.oidn_conv3x3_kernel(40, 52, cin, 0, cout, U.OIDN_F16, U.OIDN_F16, U.OIDN_RELU)[0] == \
        "conv3x3_f16_mfma<1, 2, 4, false>"
    full = run_conv(x, cin, wt, b, cout, "f16", U.OIDN_RELU)
    y0, x0, ch, cw = 101, 333, 40, 52
    crop = run_conv(np.ascontiguousarray(x[y0:y0 + ch, x0:x0 + cw]), cin, wt, b, cout, "f16",
                    U.OIDN_RELU)
    assert np.array_equal(crop[1:-1, 1:-1], full[y0 + 1:y0 + ch - 1, x0 + 1:x0 + cw - 1])
