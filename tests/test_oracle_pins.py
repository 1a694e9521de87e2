"""Pins for the CPU oracle: checks against what the pages and mathematics fix,
never against the oracle itself or the HIP path.

Sources of truth used here:
  * library conversions (numpy float16, torch bfloat16) for the number formats;
  * hand-derived quantizer cases (tests/golden/quantizer_cases.json);
  * invariants of symmetric absmax/7 quantization (range, |q| = 7 at the
    absmax, round-trip bound, sign symmetry, power-of-two invariance,
    group and token independence);
  * numpy integer / fp64 matrix products for the grouped contraction, the
    rank branch and the two reductions the method must satisfy: rank 0 is
    plain W4A4 and an all-zero residual leaves only the low-rank product
    (Deflating the Hessian, abstract: W ~ L1*L2 + Q(R)).
"""

import json
import os

import numpy as np
import pytest

from synth import bf16_bits_to_f32, f16_bits_to_f32, f64_to_bf16_bits, make_random_layer

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_cases.json")


# ------------------------------------------------------------------ formats
def test_f16_to_f32_matches_numpy_for_every_pattern(oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_to_f32_matches_torch_for_every_pattern(oracle):
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    got = np.array([oracle.bf16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f16_probe_values():
    rng = np.random.default_rng(7)
    v = []
    # every finite fp16 value, the exact midpoints between neighbours, and
    # the float32 neighbours of each midpoint
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    mids = ((h[:-1].astype(np.float64) + h[1:].astype(np.float64)) / 2).astype(np.float32)
    v += [h, mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))]
    # random magnitudes across and beyond the fp16 range
    e = rng.uniform(-30, 18, 20000)
    v.append((2.0 ** e * rng.uniform(1, 2, e.size)).astype(np.float32))
    v.append(np.array([65504, 65519.99, 65520, 65536, 1e10, 2 ** -24, 2 ** -25, 3 * 2 ** -26,
                       2 ** -14, 2 ** -14 - 2 ** -25], dtype=np.float32))
    allv = np.concatenate(v)
    return np.concatenate([allv, -allv])


def test_f32_to_f16_rne_matches_numpy(oracle):
    vals = _f16_probe_values()
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(float(x)) for x in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


# ------------------------------------------------------------- quantizer
def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_quantizer_hand_derived_cases(oracle, case):
    X = np.array(case["X_bf16"], dtype=np.uint16)[None, :]
    lam = np.array(case["lam_f16"], dtype=np.uint16)
    q, sx = oracle.quantize(X, lam)
    assert int(sx[0, 0]) == case["s_f16"]
    assert q[0].tolist() == case["codes"]


def _random_x(seed, M, K, scale=1.0, outliers=3):
    lay = make_random_layer(seed, M, K, 16, outlier_channels=outliers, x_scale=scale)
    return lay["X"], lay["lam"]


def _deq_scale(sx):
    return f16_bits_to_f32(sx).astype(np.float64)


@pytest.mark.parametrize("seed,group,K", [(0, 64, 320), (1, 64, 320), (2, 64, 320),
                                          (0, 128, 384), (1, 128, 384)])
def test_quantizer_invariants(oracle, seed, group, K):
    X, lam = _random_x(seed, 37, K)
    q, sx, xh = oracle.quantize(X, lam, want_xh=True, group=group)
    M, K = X.shape
    G = K // group
    assert sx.shape == (M, G)
    s = _deq_scale(sx)
    # codes of symmetric absmax/7 quantization lie in [-7, 7]
    assert q.min() >= -7 and q.max() <= 7
    # xh is x divided by lambda, to fp32 rounding of the reciprocal product
    ref_xh = bf16_bits_to_f32(X).astype(np.float64) / f16_bits_to_f32(lam).astype(np.float64)
    assert np.allclose(xh, ref_xh, rtol=2.5e-7, atol=0)
    for g in range(G):
        blk = xh[:, group * g:group * (g + 1)].astype(np.float64)
        qb = q[:, group * g:group * (g + 1)].astype(np.float64)
        amax = np.abs(blk).max(axis=1)
        # the scale is absmax/7 to fp16 precision (relative 2^-11)
        assert np.all(np.abs(s[:, g] - amax / 7) <= amax / 7 * 2.0 ** -11)
        # the absmax element maps to +-7
        am = np.abs(blk).argmax(axis=1)
        assert np.all(np.abs(qb[np.arange(M), am]) == 7)
        # round trip: |xh - q*s| <= s * (1/2 + 2^-20)
        assert np.all(np.abs(blk - qb * s[:, g:g + 1]) <= s[:, g:g + 1] * (0.5 + 2.0 ** -20))


def test_quantizer_sign_symmetry(oracle):
    X, lam = _random_x(5, 23, 256)
    q1, s1 = oracle.quantize(X, lam)
    q2, s2 = oracle.quantize(X ^ np.uint16(0x8000), lam)
    assert np.array_equal(s1, s2)
    assert np.array_equal(q2, -q1)


@pytest.mark.parametrize("j", [-3, 2, 5])
def test_quantizer_power_of_two_invariance(oracle, j):
    X, lam = _random_x(6, 19, 192)
    Xs = f64_to_bf16_bits(bf16_bits_to_f32(X).astype(np.float64) * 2.0 ** j)  # exact
    q1, s1 = oracle.quantize(X, lam)
    q2, s2 = oracle.quantize(Xs, lam)
    assert np.array_equal(q1, q2)
    a, b = _deq_scale(s1), _deq_scale(s2)
    normal = (a >= 2.0 ** -14) & (b >= 2.0 ** -14)
    assert normal.mean() > 0.9
    assert np.array_equal(b[normal], a[normal] * 2.0 ** j)
    # scaling lambda by the same power of two undoes it exactly
    lam_s = (f16_bits_to_f32(lam).astype(np.float64) * 2.0 ** j).astype(np.float16).view(np.uint16)
    q3, s3 = oracle.quantize(Xs, lam_s)
    assert np.array_equal(q3, q1) and np.array_equal(s3, s1)


def test_quantizer_groups_and_tokens_are_independent(oracle):
    X, lam = _random_x(8, 9, 256)
    q1, s1 = oracle.quantize(X, lam)
    X2 = X.copy()
    X2[4, 64:128] = f64_to_bf16_bits(np.linspace(-100, 100, 64))  # one group of one token
    q2, s2 = oracle.quantize(X2, lam)
    changed = np.ones_like(s1, dtype=bool)
    changed[4, 1] = False
    assert np.array_equal(s1[changed], s2[changed])
    keep = np.ones_like(q1, dtype=bool)
    keep[4, 64:128] = False
    assert np.array_equal(q1[keep], q2[keep])
    assert not np.array_equal(q1[4, 64:128], q2[4, 64:128])


def test_group128_equals_group64_when_halves_share_absmax(oracle):
    # Where both 64-channel halves of every 128-group have the same absmax
    # (the second half is the first, negated and reversed), a 128-wide group
    # has the scale of each of its halves, so group-128 and group-64 give
    # the same codes and the same scales (repeated).
    X, lam = _random_x(9, 11, 256)
    x = bf16_bits_to_f32(X).astype(np.float64)
    lamf = f16_bits_to_f32(lam).astype(np.float64)
    lam2 = lam.copy()
    for j in range(0, 256, 128):
        x[:, j + 64:j + 128] = -x[:, j:j + 64][:, ::-1]
        lam2[j + 64:j + 128] = lam[j:j + 64][::-1]      # the same divisor for the mirrored channel
    Xm = f64_to_bf16_bits(x)
    assert np.all(lamf > 0)
    q64, s64 = oracle.quantize(Xm, lam2, group=64)
    q128, s128 = oracle.quantize(Xm, lam2, group=128)
    assert np.array_equal(q64, q128)
    assert np.array_equal(s64[:, 0::2], s128) and np.array_equal(s64[:, 1::2], s128)
    # and in general the two differ: a group-128 scale covers both halves
    q64r, s64r = oracle.quantize(X, lam, group=64)
    _, s128r = oracle.quantize(X, lam, group=128)
    assert np.array_equal(s128r.view(np.uint16), np.maximum(s64r[:, 0::2], s64r[:, 1::2]))


def test_pack_act_hand_example(oracle):
    q = np.array([[1, -1, 7, -8, 0, 3, -3, 0]], dtype=np.int8)
    # byte j: code 2j in the low nibble, 2j+1 in the high nibble
    assert oracle.pack_act(q).tolist() == [[0xF1, 0x87, 0x30, 0x0D]]


# ------------------------------------------------------ integer contraction
def test_group_partials_match_numpy_integer_matmul(oracle):
    rng = np.random.default_rng(11)
    M, K, N = 21, 320, 37
    qa = rng.integers(-8, 8, (M, K), dtype=np.int8)
    qw = rng.integers(-8, 8, (K, N), dtype=np.int8)
    P = oracle.group_partials(qa, qw)
    for g in range(K // 64):
        ref = qa[:, 64 * g:64 * (g + 1)].astype(np.int64) @ qw[64 * g:64 * (g + 1)].astype(np.int64)
        assert np.array_equal(P[:, :, g], ref)
    W = oracle.group_partials(qa, qw, 3, 7, 10, 20)
    assert np.array_equal(W, P[3:10, 10:30])


def test_group128_partials_are_sums_of_group64_partials(oracle):
    rng = np.random.default_rng(12)
    M, K, N = 13, 384, 29
    qa = rng.integers(-8, 8, (M, K), dtype=np.int8)
    qw = rng.integers(-8, 8, (K, N), dtype=np.int8)
    P64 = oracle.group_partials(qa, qw, group=64)
    P128 = oracle.group_partials(qa, qw, group=128)
    assert P128.shape == (M, N, K // 128)
    assert np.array_equal(P128, P64[:, :, 0::2] + P64[:, :, 1::2])
    for g in range(K // 128):
        ref = qa[:, 128 * g:128 * (g + 1)].astype(np.int64) @ qw[128 * g:128 * (g + 1)].astype(np.int64)
        assert np.array_equal(P128[:, :, g], ref)
    # the closed-form extreme doubles with the group width
    assert np.all(oracle.group_partials(np.full((2, 128), -8, np.int8), np.full((128, 3), -8, np.int8),
                                        group=128) == 128 * 64)


def test_group_partials_closed_form_extremes(oracle):
    qa = np.full((3, 128), 7, np.int8)
    qw = np.full((128, 5), -8, np.int8)
    assert np.all(oracle.group_partials(qa, qw) == -7 * 8 * 64)
    qa[:] = -8
    assert np.all(oracle.group_partials(qa, qw) == 64 * 64)


# --------------------------------------------------------------- rank branch
def test_lowrank_down_matches_numpy(oracle):
    lay = make_random_layer(3, 13, 192, 8, r=5)
    _, _, xh = oracle.quantize(lay["X"], lay["lam"], want_xh=True)
    U = oracle.lowrank_down(xh, lay["L1"][0])
    ref = xh.astype(np.float64) @ bf16_bits_to_f32(lay["L1"][0]).astype(np.float64)
    assert np.allclose(U, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------- linear, fp64
def _dense_reference(oracle, lay, b=0, rank=True, zero_w=False):
    """Y from dense fp64 products of the dequantized matrices (numpy)."""
    group = lay["group"]
    q, sx, xh = oracle.quantize(lay["X"], lay["lam"], want_xh=True, group=group)
    A = q.astype(np.float64) * np.repeat(_deq_scale(sx), group, axis=1)
    qw = np.zeros_like(lay["qw"][b]) if zero_w else lay["qw"][b]
    W = qw.astype(np.float64) * np.repeat(f16_bits_to_f32(lay["sw"][b]).astype(np.float64), group, axis=0)
    Y = A @ W + bf16_bits_to_f32(lay["bias"][b]).astype(np.float64)[None, :]
    if rank and lay["L1"].shape[2]:
        L1 = bf16_bits_to_f32(lay["L1"][b]).astype(np.float64)
        L2 = bf16_bits_to_f32(lay["L2"][b]).astype(np.float64)
        Y = Y + (xh.astype(np.float64) @ L1) @ L2
    return Y


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("group", [64, 128])
def test_linear_equals_dense_dequantized_form(oracle, group):
    lay = make_random_layer(21, 17, 384, 29, r=4, outlier_channels=2, group=group)
    Y = oracle.linear(lay["X"], lay["lam"], lay["qw"][0], lay["sw"][0], lay["L1"][0],
                      lay["L2"][0], lay["bias"][0], group=group)
    assert _rel(Y, _dense_reference(oracle, lay)) < 1e-13


@pytest.mark.parametrize("group", [64, 128])
def test_rank_zero_is_plain_w4a4(oracle, group):
    lay = make_random_layer(22, 11, 256, 19, r=0, group=group)
    Y = oracle.linear(lay["X"], lay["lam"], lay["qw"][0], lay["sw"][0], None, None, lay["bias"][0],
                      group=group)
    assert _rel(Y, _dense_reference(oracle, lay, rank=False)) < 1e-13


@pytest.mark.parametrize("group", [64, 128])
def test_zero_residual_is_pure_low_rank(oracle, group):
    lay = make_random_layer(23, 12, 256, 21, r=4, group=group)
    zw = np.zeros_like(lay["qw"][0])
    Y = oracle.linear(lay["X"], lay["lam"], zw, lay["sw"][0], lay["L1"][0], lay["L2"][0],
                      lay["bias"][0], group=group)
    q, sx, xh = oracle.quantize(lay["X"], lay["lam"], want_xh=True, group=group)
    L1 = bf16_bits_to_f32(lay["L1"][0]).astype(np.float64)
    L2 = bf16_bits_to_f32(lay["L2"][0]).astype(np.float64)
    ref = xh.astype(np.float64) @ L1 @ L2 + bf16_bits_to_f32(lay["bias"][0]).astype(np.float64)
    assert _rel(Y, ref) < 1e-13


def test_bias_only(oracle):
    lay = make_random_layer(24, 5, 64, 9, r=0)
    Y = oracle.linear(lay["X"], lay["lam"], np.zeros_like(lay["qw"][0]), lay["sw"][0],
                      None, None, lay["bias"][0])
    assert np.array_equal(Y, np.broadcast_to(bf16_bits_to_f32(lay["bias"][0]).astype(np.float64), Y.shape))


def test_linear_row_subset_and_batch(oracle):
    lay = make_random_layer(25, 14, 128, 10, r=3, batch=2)
    full = oracle.linear_batched(lay)
    rows = np.array([13, 0, 7])
    sub = oracle.linear_batched(lay, rows=rows)
    assert np.array_equal(sub, full[:, rows])
    for b in range(2):
        assert _rel(full[b], _dense_reference(oracle, lay, b=b)) < 1e-13
