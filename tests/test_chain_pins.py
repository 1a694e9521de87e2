"""Pins for the fused-chain oracle (oracle/chain.py), against library
routines and the pinned C oracle, never against the HIP path:

  * the exponential built from basic operations against NumPy's fp64 exp
    (relative error below 2^-21 over its whole range);
  * the fp32 GELU against the tanh form evaluated in fp64 with NumPy's
    tanh; its limits (0 at 0, y for large y, ~0 for very negative y);
  * the fp32-input quantizer against the C oracle's quantizer on inputs that
    are bf16 values (the two must agree bit for bit: the C oracle is pinned
    by tests/test_oracle_pins.py);
  * the down layer's output from codes against the C oracle's linear when
    the hidden activation is a bf16 tensor and the activation the identity
    (the chain then reduces to an ordinary layer).
"""

import numpy as np
import pytest

from oracle import chain
from synth import f64_to_bf16_bits, f64_to_f16_bits, make_random_layer


def test_exp_matches_numpy_over_its_range():
    x = np.linspace(-87.0, 88.0, 200001).astype(np.float32)
    got = chain.exp_f32_basic(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    assert np.all(np.abs(got - ref) <= 2.0 ** -21 * ref)
    assert chain.exp_f32_basic(np.float32(0.0)) == np.float32(1.0)


def test_gelu_matches_the_tanh_form():
    y = np.linspace(-12.0, 12.0, 100001).astype(np.float32)
    yd = y.astype(np.float64)
    ref = 0.5 * yd * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (yd + 0.044715 * yd ** 3)))
    got = chain.gelu_tanh_f32(y).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0 ** -19 * np.abs(yd) + 1e-30)


def test_gelu_limits():
    assert chain.gelu_tanh_f32(np.float32(0.0)) == 0.0
    big = np.array([20.0, 100.0, 3.0e4], dtype=np.float32)
    assert np.array_equal(chain.gelu_tanh_f32(big), big)
    neg = chain.gelu_tanh_f32(np.array([-20.0, -100.0, -3.0e4], dtype=np.float32))
    assert np.all(np.abs(neg) < 1e-30) and np.all(neg <= 0)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp32_quantizer_equals_c_oracle_on_bf16_inputs(oracle, seed):
    lay = make_random_layer(300 + seed, 37, 256, 8, r=0, outlier_channels=3)
    x = lay["X"]
    a = (x.astype(np.uint32) << 16).view(np.float32)
    q, s16, _ = chain.quantize_f32(a, lay["lam"])
    qc, sc = oracle.quantize(x, lay["lam"])
    assert np.array_equal(q, qc)
    assert np.array_equal(s16, sc)


def test_fp32_quantizer_zero_and_saturated_groups():
    lam = f64_to_f16_bits(np.ones(128))
    a = np.zeros((3, 128), dtype=np.float32)
    a[1, :64] = 1.0e6                      # amax / 7 above 65504: the scale saturates
    a[2, 64:] = np.linspace(-7, 7, 64)
    q, s16, _ = chain.quantize_f32(a, lam)
    assert s16[0, 0] == 0 and s16[0, 1] == 0 and not q[0].any()
    assert s16[1, 0] == 0x7BFF and np.all(q[1, :64] == 7)
    assert s16[2, 1] == np.float16(1.0).view(np.uint16)
    assert np.array_equal(q[2, 64:], np.clip(np.rint(np.linspace(-7, 7, 64).astype(np.float32)), -8, 7))


def test_identity_chain_reduces_to_the_plain_layer(oracle):
    # a bf16 hidden tensor through the identity: the chain's down layer is
    # the ordinary linear of that tensor
    lay = make_random_layer(311, 24, 192, 40, r=4, outlier_channels=2)
    a = (lay["X"].astype(np.uint32) << 16).view(np.float32)
    q, s16, U = chain.hidden(a, lay["lam"], lay["L1"][0], "identity")
    Y = chain.down_output(q, s16, U, lay["qw"][0], lay["sw"][0], lay["L2"][0], lay["bias"][0])
    ref = oracle.linear(lay["X"], lay["lam"], lay["qw"][0], lay["sw"][0], lay["L1"][0], lay["L2"][0],
                        lay["bias"][0])
    assert np.allclose(Y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
