"""GPU parity of the fused conv pair y = convB(relu(convA(x))) (32-channel
intermediate kept on chip) against the CPU oracle's two convs, and bit-exact
against two separate conv launches, through the C ABI."""
import numpy as np
import pytest

import synthetic as S
import unet_x3_convolution_amd as U
from helpers import DT, TOL, dev, empty, host, packed_conv, rel_err, say
from oracle import oracle as O

pytestmark = pytest.mark.gpu

R, P = U.OIDN_RELU, U.OIDN_POOL2X2
PAIR_CASES = [
    # h, w, cin, cout, convB flags, output precision
    (544, 960, 16, 32, R | P, "f16"),     # enc_conv0 -> enc_conv1 shape (16-channel chunk)
    (520, 1030, 64, 3, 0, "f32"),         # dec_conv1b -> dec_conv0 shape, ragged, fp32 out
    (33, 47, 32, 32, R, "f16"),           # odd sizes, tile edges everywhere
    (64, 62, 16, 16, R | P, "f16"),       # one output fragment, pooled
    (1, 1, 8, 4, 0, "f32"),               # degenerate 1 x 1
    (16, 30, 64, 32, R, "f16"),           # exactly one tile
    (18, 62, 96, 32, R, "f16"),           # three 32-channel chunks
    (96, 120, 8, 20, R, "f16"),           # 8-channel source, cout inside a fragment pair
    (64, 90, 32, 28, R | P, "f16"),       # cout inside a fragment pair, pooled
]


def run_pair(x, cin, wa, ba, wb, bb, cout, flags, outp):
    h, w = x.shape[:2]
    pa = packed_conv(wa, ba, cin, 0, 32, "f16")
    pb = packed_conv(wb, bb, 32, 0, cout, "f16")
    oh, ow = (h // 2, w // 2) if flags & P else (h, w)
    y = empty((oh, ow, O.stored(cout)), O.np_storage(outp), fill=float("nan"))
    U.oidn_conv3x3_pair(dev(x), h, w, cin, pa, pb, y, cout, DT[outp], flags)
    return host(y), pa, pb


@pytest.mark.parametrize("h,w,cin,cout,flags,outp", PAIR_CASES)
def test_pair_matches_oracle_and_two_launches(h, w, cin, cout, flags, outp):
    r = np.random.default_rng(3000 + h + cin)
    x = O.round_to(S.relu_normal_activation(r, h, w, cin, O.stored(cin)), "f16")
    wa, ba = S.he_normal(r, 32, cin), S.bias(r, 32)
    wb, bb = S.he_normal(r, cout, 32), S.bias(r, cout)
    got, pa, pb = run_pair(x, cin, wa, ba, wb, bb, cout, flags, outp)
    assert not np.any(np.isnan(got)), "unwritten outputs"
    mid = O.conv3x3(x, cin, wa, ba, True, "f16")
    ref = O.conv3x3(mid, 32, wb, bb, bool(flags & R), "f16", outp)
    if flags & P:
        ref = O.pool2x2(ref)
    assert np.all(got[..., cout:] == 0), "pad lanes not zero"
    err = rel_err(got[..., :cout], ref[..., :cout])
    say(f"pair {h}x{w} {cin}->32->{cout} flags={flags} out={outp}: max_rel_err={err:.3e}")
    assert err <= TOL["f16"], err
    # the same two convs as separate launches: identical bits
    m = empty((h, w, 32), np.float16, fill=float("nan"))
    U.oidn_conv3x3(dev(x), h, w, cin, pa, m, 32, U.OIDN_F16, U.OIDN_F16, R)
    oh, ow = (h // 2, w // 2) if flags & P else (h, w)
    y2 = empty((oh, ow, O.stored(cout)), O.np_storage(outp), fill=float("nan"))
    U.oidn_conv3x3(m, h, w, 32, pb, y2, cout, U.OIDN_F16, DT[outp], flags)
    assert np.array_equal(got, host(y2))


@pytest.mark.parametrize("cin,cout", [(12, 32), (48, 32), (32, 48)])
def test_pair_rejects_unsupported_shapes(cin, cout):
    x = empty((8, 8, O.stored(cin)), np.float16)
    pa = empty((U.oidn_conv3x3_weights_bytes(cin, 0, 32, U.OIDN_F16),), np.uint8)
    pb = empty((U.oidn_conv3x3_weights_bytes(32, 0, cout, U.OIDN_F16),), np.uint8)
    y = empty((8, 8, O.stored(cout)), np.float16)
    with pytest.raises(U.OidnError) as e:
        U.oidn_conv3x3_pair(x, 8, 8, cin, pa, pb, y, cout, U.OIDN_F16, R)
    assert e.value.code == U.OIDN_E_UNSUPPORTED
