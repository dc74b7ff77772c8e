"""Identities the fp16 kernels rely on, checked in float64 on the CPU.

The kernels reorganise some sums (never the arithmetic they define); these
tests show each reorganisation is exact in real arithmetic, so that the GPU
results differ from the oracle's plain definitions by rounding only."""
import numpy as np
import pytest


def _conv3x3_f64(x, w_ohwi):
    """3x3 conv, stride 1, zero padding 1, no bias: out[y][x][o] =
    sum over ky, kx, i of W[o][ky][kx][i] * X[y + ky - 1][x + kx - 1][i]."""
    h, wd, cin = x.shape
    xp = np.zeros((h + 2, wd + 2, cin))
    xp[1:h + 1, 1:wd + 1] = x
    out = np.zeros((h, wd, w_ohwi.shape[0]))
    for ky in range(3):
        for kx in range(3):
            out += xp[ky:ky + h, kx:kx + wd] @ w_ohwi[:, ky, kx, :].T
    return out


def _row_subpixel_conv(low, w_ohwi):
    """The decoder kernels' form of conv3x3(nearest_upsample_2x(low)): an
    output row y = 2 Y + py reads low-resolution rows Y - 1 (weights W0) and
    Y (W1 + W2) if py = 0, Y (W0 + W1) and Y + 1 (W2) if py = 1; columns keep
    their three taps on the upsampled columns x + kx - 1, i.e. low-resolution
    column (x + kx - 1) // 2.  Rows and columns outside the image are zero."""
    lh, lw, cin = low.shape
    h, wd = 2 * lh, 2 * lw
    cout = w_ohwi.shape[0]
    combos = {0: [(-1, w_ohwi[:, 0]), (0, w_ohwi[:, 1] + w_ohwi[:, 2])],
              1: [(0, w_ohwi[:, 0] + w_ohwi[:, 1]), (1, w_ohwi[:, 2])]}
    out = np.zeros((h, wd, cout))
    for y in range(h):
        Y, py = divmod(y, 2)
        for dy, wrow in combos[py]:          # wrow: cout x 3 (kx) x cin
            ly = Y + dy
            if not 0 <= ly < lh:
                continue
            for x in range(wd):
                for kx in range(3):
                    ux = x + kx - 1
                    if not 0 <= ux < wd:
                        continue
                    out[y, x] += wrow[:, kx, :] @ low[ly, ux // 2]
    return out


@pytest.mark.parametrize("lh,lw,cin,cout", [(1, 1, 3, 2), (3, 4, 5, 3), (4, 7, 8, 4)])
def test_row_subpixel_equals_conv_of_upsampled(lh, lw, cin, cout):
    r = np.random.default_rng(lh * 100 + lw * 10 + cin)
    low = r.standard_normal((lh, lw, cin))
    w = r.standard_normal((cout, 3, 3, cin))
    up = np.repeat(np.repeat(low, 2, axis=0), 2, axis=1)
    ref = _conv3x3_f64(up, w)
    got = _row_subpixel_conv(low, w)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_row_subpixel_work():
    """Per output pixel and channel pair the upsampled source costs 2 x 3 = 6
    multiply-adds instead of 9; the network's decoder layers (c_low of
    96, 112, 96, 64) therefore need 211,980 FLOP per input pixel instead of
    250,812 at 9 input channels (the count the bench reports TFLOP/s on)."""
    layers = [  # cin0, cin1, cout, level for every conv of the 9-channel UNet
        (9, 0, 32, 0), (32, 0, 32, 0), (32, 0, 48, 1), (48, 0, 64, 2), (64, 0, 80, 3),
        (80, 0, 96, 4), (96, 0, 96, 4), (96, 64, 112, 3), (112, 0, 112, 3), (112, 48, 96, 2),
        (96, 0, 96, 2), (96, 32, 64, 1), (64, 0, 64, 1), (64, 9, 64, 0), (64, 0, 32, 0),
        (32, 0, 3, 0)]
    full = sum(2 * 9 * (c0 + c1) * co / 4 ** lvl for c0, c1, co, lvl in layers)
    red = sum(2 * ((6 * c0 + 9 * c1) if c1 else 9 * c0) * co / 4 ** lvl
              for c0, c1, co, lvl in layers)
    assert full == 250812 and red == 211980


def _tap_chunk_conv(x9, w_ohwi):
    """The tap-chunk form of a conv over a 9-channel input: channels 0..7 keep
    their three column taps; channel 8's three taps come from one 'centre
    pixel' group whose lanes hold channel 8 at columns x - 1, x, x + 1 (zero
    outside the image), weighted by W[.][ky][kx][8] for kx = 0, 1, 2."""
    h, wd, _ = x9.shape
    taps = np.zeros((h, wd, 3))
    taps[:, 1:, 0] = x9[:, :-1, 8]
    taps[:, :, 1] = x9[:, :, 8]
    taps[:, :-1, 2] = x9[:, 1:, 8]
    out = _conv3x3_f64(np.concatenate([x9[..., :8], np.zeros((h, wd, 1))], axis=2),
                       np.concatenate([w_ohwi[..., :8], np.zeros(w_ohwi.shape[:3] + (1,))], axis=3))
    # centre-pixel group: rows ky = 0..2 at the centre column only
    tp = np.zeros((h + 2, wd, 3))
    tp[1:h + 1] = taps
    for ky in range(3):
        out += tp[ky:ky + h] @ w_ohwi[:, ky, :, 8].T
    return out


def test_tap_chunk_equals_plain_conv():
    r = np.random.default_rng(11)
    x9 = r.standard_normal((5, 7, 9))
    w = r.standard_normal((4, 3, 3, 9))
    assert np.allclose(_tap_chunk_conv(x9, w), _conv3x3_f64(x9, w), rtol=1e-12, atol=1e-12)
