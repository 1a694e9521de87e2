"""Pins for the MX-fp4 oracle (oracle/mx.py) from the format's definition
(OCP Microscaling Formats v1.0: e8m0 shared scale 2^(floor(log2 amax) - 2),
e2m1 elements rounded to nearest even with saturation), never against the
HIP path:

  * hand-derived e2m1 roundings, ties included, and the code encoding;
  * the rounding against a brute-force nearest-value search in Python floats
    on a dense grid;
  * the scale rule against math.frexp, the zero block, the clamp of tiny
    blocks, the round-trip bound;
  * the layer's residual product against explicit per-block loops (exact in
    fp64 at these sizes), and the rank branch and bias against NumPy.
"""

import math

import numpy as np
import pytest

from oracle import mx
from synth import make_random_layer

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("v,val,code", [
    (0.0, 0.0, 0), (0.25, 0.0, 0), (0.3, 0.5, 1), (0.75, 1.0, 2), (1.25, 1.0, 2), (1.3, 1.5, 3),
    (1.75, 2.0, 4), (2.5, 2.0, 4), (2.6, 3.0, 5), (3.5, 4.0, 6), (5.0, 4.0, 6), (5.5, 6.0, 7),
    (6.9, 6.0, 7), (7.99, 6.0, 7), (-0.75, -1.0, 10), (-5.0, -4.0, 14), (-7.0, -6.0, 15),
    (-0.2, -0.0, 8), (-0.25, -0.0, 8), (-0.0, -0.0, 8), (-0.26, -0.5, 9),   # sign kept at zero
])
def test_e2m1_hand_cases(v, val, code):
    c, q = mx.e2m1_round(np.array([v]))
    assert q[0] == val and np.signbit(q[0]) == np.signbit(val) and c[0] == code


def test_e2m1_rounding_matches_brute_force():
    def ref(v):
        m = abs(v)
        best = None
        for i, e in enumerate(mx.E2M1):
            d = abs(m - e)
            # nearest; on a tie the even mantissa (even index) wins
            if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
                best = (d, i)
        i = best[1]
        if m > 6.0:
            i = 7
        neg = math.copysign(1.0, v) < 0
        return mx.E2M1[i] * (-1 if neg else 1), i + (8 if neg else 0)
    grid = np.concatenate([np.arange(-8.0, 8.0, 1.0 / 64), [-0.0]])
    c, q = mx.e2m1_round(grid)
    for v, cc, qq in zip(grid, c, q):
        rv, rc = ref(float(v))
        assert qq == rv and cc == rc, v


def test_scale_rule_matches_frexp():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((50, 64)) * np.exp(rng.uniform(-20, 20, (50, 1)))).astype(np.float32)
    _, s = mx.quantize_blocks(x)
    for r in range(50):
        for b in range(2):
            amax = float(np.abs(x[r, 32 * b:32 * b + 32]).max())
            _, e = math.frexp(amax)           # amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1
            assert s[r, b] == (e - 1) - 2 + 127


def test_zero_block_tiny_block_and_round_trip_bound():
    x = np.zeros((3, 64), dtype=np.float32)
    x[1, :32] = np.float32(2.0 ** -140) * np.arange(1, 33)
    x[2, 32:] = np.linspace(-100, 77, 32)
    c, s = mx.quantize_blocks(x)
    assert s[0, 0] == 127 and s[0, 1] == 127 and not c[0].any()
    assert s[1, 0] == 0                       # clamped: the scale floor is 2^-127
    d = mx.dequantize_blocks(c, s)
    scale = np.ldexp(1.0, s[2, 1].astype(np.int64) - 127)
    assert np.all(np.abs(d[2, 32:] - x[2, 32:]) <= 2.0 * scale)
    assert np.abs(d[2, 32:]).max() <= 6.0 * scale


def test_residual_product_matches_block_loops():
    rng = np.random.default_rng(4)
    lay = make_random_layer(401, 5, 128, 6, r=2, outlier_channels=1)
    R = (rng.standard_normal((128, 6)) * 0.01).astype(np.float32)
    Y = mx.linear(lay["X"], lay["lam"], R)
    ca, sa = mx.quantize_act(lay["X"], lay["lam"])
    cw, sw = mx.quantize_weight(R)
    val = lambda c: (-1 if c & 8 else 1) * mx.E2M1[c & 7]
    for m in range(5):
        for n in range(6):
            acc = 0.0
            for b in range(4):
                blk = sum(val(int(ca[m, 32 * b + i])) * val(int(cw[32 * b + i, n])) for i in range(32))
                acc += blk * 2.0 ** (int(sa[m, b]) + int(sw[b, n]) - 254)
            assert Y[m, n] == acc


def test_rank_branch_and_bias():
    lay = make_random_layer(402, 7, 128, 9, r=3, outlier_channels=1)
    R = np.zeros((128, 9), dtype=np.float32)
    Y = mx.linear(lay["X"], lay["lam"], R, lay["L1"][0], lay["L2"][0], lay["bias"][0])
    xh = mx.smoothed(lay["X"], lay["lam"]).astype(np.float64)
    L1 = (lay["L1"][0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    L2 = (lay["L2"][0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    b = (lay["bias"][0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.allclose(Y, xh @ L1 @ L2 + b, rtol=1e-12, atol=1e-15)
