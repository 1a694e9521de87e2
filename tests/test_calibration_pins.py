"""Pins for the calibration oracle (oracle/calibration.py): checks against
what the pages and linear algebra fix, never against the oracle itself or
the HIP path.

  * the deflated Hessian annihilates the protected subspace, Hperp L1 = 0
    (Deflating the Hessian, Figure 1 caption);
  * eliminating the output-side factor in closed form is least squares:
    the closed-form L2 equals NumPy's lstsq solution of Xh L1 L2 ~ Xh E,
    which never forms H, and its residual equals tr(E^T Hperp E)
    (abstract: eliminating the output-side factor yields the deflated
    Hessian; rit.work explainer: the output factor is recomputed in closed
    form on the finished residual);
  * H = Xh^T Xh entry by entry from explicit loops, symmetry, positive
    semi-definiteness, and Hperp's r null directions;
  * deflation depends on span(L1) only, an error inside span(L1) costs
    nothing, and rank 0 leaves H unchanged.
"""

import numpy as np
import pytest

from oracle import calibration as cal
from synth import f64_to_bf16_bits, f64_to_f16_bits, make_full_weight, make_random_layer


def _setup(seed=0, M=256, K=128, N=48, r=4):
    lay = make_random_layer(seed, M, K, N, r=r, outlier_channels=3)
    xh = cal.smoothed_activations(lay["X"], lay["lam"])
    H = cal.hessian(lay["X"], lay["lam"])
    L1 = cal.bf16_matrix(lay["L1"][0])
    W = make_full_weight(lay, 0)
    E = cal.residual_error(W, lay["qw"][0], lay["sw"][0], lay["group"])
    return lay, xh, H, L1, E


def test_smoothing_is_exact_for_power_of_two_lambda():
    rng = np.random.default_rng(5)
    X = f64_to_bf16_bits(rng.standard_normal((8, 64)))
    e = rng.integers(-6, 7, 64)
    lam = f64_to_f16_bits(2.0 ** e)
    x = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(cal.smoothed_activations(X, lam), x * 2.0 ** (-e)[None, :])


def test_smoothing_within_two_roundings_of_the_quotient():
    rng = np.random.default_rng(6)
    X = f64_to_bf16_bits(rng.standard_normal((16, 64)) * 3)
    lam = f64_to_f16_bits(np.exp(rng.uniform(-1, 1, 64)))
    x = (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q = x / lam.view(np.float16).astype(np.float64)[None, :]
    got = cal.smoothed_activations(X, lam)
    assert np.all(np.abs(got - q) <= 2.0 ** -22 * np.abs(q))


def test_hessian_entries_from_explicit_loops():
    lay, xh, H, _, _ = _setup(M=40, K=64)
    rows = [[float(v) for v in row] for row in xh]
    for i, j in [(0, 0), (3, 17), (17, 3), (63, 63), (10, 50)]:
        s = 0.0
        for m in range(len(rows)):
            s += rows[m][i] * rows[m][j]
        assert H[i, j] == pytest.approx(s, rel=1e-12, abs=1e-300)
    assert np.array_equal(H, H.T)
    assert np.all(np.diag(H) >= 0)


def test_hessian_is_positive_semidefinite():
    _, _, H, _, _ = _setup()
    ev = np.linalg.eigvalsh(H)
    assert ev.min() >= -1e-12 * ev.max()


@pytest.mark.parametrize("r", [1, 4, 8])
def test_deflated_hessian_annihilates_l1(r):
    _, _, H, L1, _ = _setup(seed=r, r=r)
    _, _, _, Hp = cal.deflate(H, L1)
    assert np.linalg.norm(Hp @ L1) <= 1e-12 * np.linalg.norm(H) * np.linalg.norm(L1)
    assert np.linalg.norm(L1.T @ Hp) <= 1e-12 * np.linalg.norm(H) * np.linalg.norm(L1)


def test_deflated_hessian_is_psd_with_r_null_directions():
    r = 4
    _, _, H, L1, _ = _setup(r=r)              # M = 256 >= K = 128: H is definite
    _, _, _, Hp = cal.deflate(H, L1)
    ev = np.linalg.eigvalsh((Hp + Hp.T) / 2)
    top = np.linalg.eigvalsh(H).max()
    assert ev.min() >= -1e-11 * top
    assert np.sum(np.abs(ev) <= 1e-11 * top) == r
    assert np.linalg.eigvalsh(H).min() > 1e-6 * top


def test_deflation_depends_only_on_the_span_of_l1():
    _, _, H, L1, E = _setup(seed=3)
    T = np.random.default_rng(9).standard_normal((4, 4)) + 3 * np.eye(4)
    _, _, _, Hp = cal.deflate(H, L1)
    _, _, _, Hq = cal.deflate(H, L1 @ T)
    assert np.allclose(Hp, Hq, rtol=0, atol=1e-10 * np.abs(H).max())
    # and L2 transforms contravariantly: (L1 T)(T^-1 L2) = L1 L2
    L2 = cal.closed_form_l2(H, L1, E)
    L2t = cal.closed_form_l2(H, L1 @ T, E)
    assert np.allclose(L1 @ L2, (L1 @ T) @ L2t, rtol=1e-9, atol=1e-14)


def test_closed_form_l2_is_least_squares():
    _, xh, H, L1, E = _setup(seed=4)
    L2_ls, *_ = np.linalg.lstsq(xh @ L1, xh @ E, rcond=None)
    L2 = cal.closed_form_l2(H, L1, E)
    assert np.allclose(L2, L2_ls, rtol=1e-8, atol=1e-8 * np.abs(L2_ls).max())
    # the minimum of ||Xh E - Xh L1 L2||^2 over L2 is tr(E^T Hperp E)
    res = np.linalg.norm(xh @ E - xh @ L1 @ L2_ls) ** 2
    _, _, _, Hp = cal.deflate(H, L1)
    assert cal.deflated_error(Hp, E) == pytest.approx(res, rel=1e-8)
    # and any other L2 does worse
    worse = np.linalg.norm(xh @ E - xh @ L1 @ (L2_ls * 1.01)) ** 2
    assert worse > res


def test_error_inside_the_span_of_l1_costs_nothing():
    _, _, H, L1, _ = _setup(seed=5)
    Z = np.random.default_rng(1).standard_normal((4, 48))
    E = L1 @ Z
    assert np.allclose(cal.closed_form_l2(H, L1, E), Z, rtol=1e-9, atol=1e-9)
    _, _, _, Hp = cal.deflate(H, L1)
    assert abs(cal.deflated_error(Hp, E)) <= 1e-12 * np.einsum("kn,kn->", E, H @ E)


def test_rank_zero_leaves_the_hessian_unchanged():
    _, xh, H, _, E = _setup(seed=6)
    HL1, C, Cinv, Hp = cal.deflate(H, np.zeros((H.shape[0], 0)))
    assert HL1.shape == (H.shape[0], 0) and C.shape == (0, 0)
    assert np.array_equal(Hp, H)
    assert cal.deflated_error(Hp, E) == pytest.approx(np.linalg.norm(xh @ E) ** 2, rel=1e-10)


def test_residual_error_of_the_weight_recipe():
    # a weight drawn without rounding noise: its residual error is the
    # low-rank product up to the bf16 rounding of W (half an ulp of |W|)
    lay = make_random_layer(7, 8, 128, 32, r=4)
    W = make_full_weight(lay, 0, noise=0.0)
    E = cal.residual_error(W, lay["qw"][0], lay["sw"][0], lay["group"])
    low = cal.bf16_matrix(lay["L1"][0]) @ cal.bf16_matrix(lay["L2"][0])
    Wf = cal.bf16_matrix(W)
    assert np.all(np.abs(E - low) <= 2.0 ** -8 * np.abs(Wf) + 1e-30)
