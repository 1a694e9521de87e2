"""Pins for the asymmetric-activation oracle (oracle/asym.py), never against
the HIP path:

  * a group worked by hand (scale, zero point and every code);
  * special cases: a zero group, an all-positive group (zero point 0), an
    all-negative group (zero point 15), a constant group;
  * the code against a brute-force search for the nearest of the group's 16
    levels, and the round-trip bound;
  * the partial sums against the zero-point identity
    sum (q - z) w = sum q w - z sum w, computed by a separate route;
  * the layer output against dequantize-then-multiply in fp64.
"""

import numpy as np
import pytest

from oracle import asym
from synth import make_random_layer


def bits_bf16(vals):
    """bf16 bit patterns of values exactly representable in bf16."""
    v = np.asarray(vals, dtype=np.float32)
    b = v.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0)
    return (b >> 16).astype(np.uint16)


ONE_F16 = np.uint16(0x3C00)


def quant_row(vals, group=64):
    X = bits_bf16(np.asarray(vals, dtype=np.float32)[None, :])
    lam = np.full(X.shape[1], ONE_F16, dtype=np.uint16)
    xh = asym.smoothed(X, lam)
    q, z, s16 = asym.quantize(xh, group)
    return xh, q, z, s16


def test_hand_worked_group():
    # lo = -1, hi = 2: range 3, 3/15 = 0.2 -> fp16 0.199951171875 (0x3266);
    # inv = fl32(1 / 0.199951171875) = 5.0012207...; z = rint(5.0012) = 5
    vals = np.zeros(64, dtype=np.float32)
    vals[:5] = [-1.0, 2.0, 0.0, 0.5, 1.0]
    _, q, z, s16 = quant_row(vals)
    assert s16[0, 0] == 0x3266
    assert z[0, 0] == 5
    # 2 -> rint(10.0024) + 5 = 15; -1 -> -5 + 5 = 0; 0 -> 5; 0.5 -> rint(2.5006) = 3 -> 8;
    # 1 -> rint(5.0012) = 5 -> 10
    assert list(q[0, :5]) == [0, 15, 5, 8, 10]
    assert np.all(q[0, 5:] == 5)
    d = asym.stored_codes(q, z)
    assert list(d[0, :5]) == [-5, 10, 0, 3, 5]


def test_special_groups():
    # zero group
    _, q, z, s16 = quant_row(np.zeros(64))
    assert s16[0, 0] == 0 and z[0, 0] == 0 and not q.any()
    # all positive: lo = 0, so z = 0 and q = rint(x / s), the largest 15
    pos = np.linspace(0.25, 4.0, 64).astype(np.float32)
    pos = (pos.view(np.uint32) & 0xFFFF0000).view(np.float32)
    _, q, z, s16 = quant_row(pos)
    assert z[0, 0] == 0 and q.max() == 15 and q.min() >= 0
    # all negative: hi = 0, -lo / s is about 15, so z = 15 and the stored values are <= 0
    _, q, z, s16 = quant_row(-pos)
    assert z[0, 0] == 15
    d = asym.stored_codes(q, z)
    assert d.max() <= 0 and d.min() == -15
    # constant group c: range [0, c], s = fp16(c / 15), every code 15 (or the level next to c)
    _, q, z, s16 = quant_row(np.full(64, 3.0))
    assert z[0, 0] == 0 and np.all(q == 15)


def test_codes_are_the_nearest_level():
    rng = np.random.default_rng(11)
    for trial in range(40):
        scale = np.exp(rng.uniform(-6, 6))
        shift = rng.uniform(-1, 1) * scale
        vals = (rng.standard_normal(64) * scale + shift).astype(np.float32)
        vals = (vals.view(np.uint32) & 0xFFFF0000).view(np.float32)
        xh, q, z, s16 = quant_row(vals)
        s = float(s16.view(np.float16)[0, 0])
        zz = int(z[0, 0])
        levels = (np.arange(16) - zz) * s
        deq = (q[0].astype(np.int64) - zz) * s
        for x, dv in zip(xh[0].astype(np.float64), deq):
            best = np.min(np.abs(levels - x))
            # nearest level up to the rounding of x / s in fp32
            assert abs(dv - x) <= best + 1e-6 * s, (trial, x, dv, best)
        lo, hi = min(0.0, float(xh.min())), max(0.0, float(xh.max()))
        slack = max(0.0, (hi - lo) - 15 * s)          # what fp16 rounding of s leaves uncovered
        assert np.all(np.abs(deq - xh[0]) <= 0.5 * s + slack + 1e-6 * s)


def test_partials_match_zero_point_identity():
    lay = make_random_layer(903, 9, 256, 21, r=0, outlier_channels=2)
    X, lam, qw = lay["X"], lay["lam"], lay["qw"][0]
    P = asym.partials(X, lam, qw)
    q, z, _ = asym.quantize(asym.smoothed(X, lam))
    qi, wi = q.astype(np.int64), qw.astype(np.int64)
    for g in range(4):
        sl = slice(64 * g, 64 * g + 64)
        ref = qi[:, sl] @ wi[sl, :] - z[:, g:g + 1].astype(np.int64) * wi[sl, :].sum(axis=0)[None, :]
        assert np.array_equal(P[:, :, g], ref)


@pytest.mark.parametrize("group", [64, 128])
def test_linear_matches_dequantized_product(group):
    lay = make_random_layer(904, 7, 256, 13, r=3, outlier_channels=1)
    X, lam = lay["X"], lay["lam"]
    qw = lay["qw"][0]
    G = 256 // group
    sw = lay["sw"][0][:G]
    Y = asym.linear(X, lam, qw, sw, lay["L1"][0], lay["L2"][0], lay["bias"][0], group=group)
    xh = asym.smoothed(X, lam)
    q, z, s16 = asym.quantize(xh, group)
    sx = s16.view(np.float16).astype(np.float64)
    A = (q.astype(np.float64).reshape(7, G, group) - z[:, :, None]) * sx[:, :, None]
    W = qw.astype(np.float64).reshape(G, group, 13) * sw.view(np.float16).astype(np.float64)[:, None, :]
    L1 = (lay["L1"][0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    L2 = (lay["L2"][0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    b = (lay["bias"][0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = A.reshape(7, 256) @ W.reshape(256, 13) + xh.astype(np.float64) @ L1 @ L2 + b
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
