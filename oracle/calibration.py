"""CPU oracle for the calibration steps of the method (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  Plain NumPy in float64; it shares nothing with the HIP
library.

What it computes (Deflating the Hessian, shd-paper.top paper page: abstract
and Figure 1 caption; H-SVDQuant explainer, rit.work, section on Hessian
deflation).  The pages print no formulas for these steps; the readings
below are the plainest ones the text supports:

  * Hessian of the layer's output error: H = Xh^T Xh over the calibration
    tokens, with Xh the smoothed activations exactly as the inference path
    forms them (x * fl32(1/lambda), rounded to fp32).  The activation-noise
    surrogate term of the pages is not included (its weight set to 0).
  * For a fixed input-side factor L1 (K x r) and a residual error
    E = W - deq(Q(R)) (K x N), the output-side factor that minimises
    ||Xh E - Xh L1 L2||_F^2 has the closed form
        L2* = C^-1 L1^T H E,   C = L1^T H L1   (r x r).
  * Eliminating L2 that way leaves the error tr(E^T Hperp E) with the
    deflated Hessian
        Hperp = H - H L1 C^-1 L1^T H,
    which satisfies Hperp L1 = 0 (Figure 1 caption): errors inside span(L1)
    cost nothing, because the low-rank branch absorbs them.
"""

from __future__ import annotations

import numpy as np


def smoothed_activations(X_bits: np.ndarray, lam_bits: np.ndarray) -> np.ndarray:
    """Xh = fl32(x * fl32(1 / lambda)) as float64 (the inference path's
    smoothing: bf16 x, fp16 lambda, fp32 reciprocal and product)."""
    x = (X_bits.astype(np.uint32) << 16).view(np.float32)
    lam = lam_bits.view(np.float16).astype(np.float32)
    inv = np.float32(1.0) / lam
    return (x * inv[None, :]).astype(np.float64)


def hessian(X_bits: np.ndarray, lam_bits: np.ndarray) -> np.ndarray:
    """H = Xh^T Xh (K x K, float64)."""
    xh = smoothed_activations(X_bits, lam_bits)
    return xh.T @ xh


def hessian_abs(X_bits: np.ndarray, lam_bits: np.ndarray) -> np.ndarray:
    """|Xh|^T |Xh|: the magnitude each entry of H is summed from (rounding
    bounds of H are proportional to it)."""
    xa = np.abs(smoothed_activations(X_bits, lam_bits))
    return xa.T @ xa


def dequantized_residual(qw: np.ndarray, sw_bits: np.ndarray, group: int) -> np.ndarray:
    """deq(Q(R))[k, n] = qw[k, n] * sw[k // group, n] (float64)."""
    sw = sw_bits.view(np.float16).astype(np.float64)
    return qw.astype(np.float64) * np.repeat(sw, group, axis=0)


def residual_error(W_bits: np.ndarray, qw: np.ndarray, sw_bits: np.ndarray, group: int) -> np.ndarray:
    """E = W - deq(Q(R)) for a bf16 weight W (K x N)."""
    W = (W_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return W - dequantized_residual(qw, sw_bits, group)


def bf16_matrix(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def deflate(H: np.ndarray, L1: np.ndarray):
    """The deflation of H by span(L1): returns (H L1, C, C^-1, Hperp).

    C = L1^T H L1 is inverted with a library solve; r = 0 gives Hperp = H."""
    H = np.asarray(H, dtype=np.float64)
    L1 = np.asarray(L1, dtype=np.float64)
    r = L1.shape[1]
    HL1 = H @ L1
    if r == 0:
        return HL1, np.zeros((0, 0)), np.zeros((0, 0)), H.copy()
    C = L1.T @ HL1
    Cinv = np.linalg.solve(C, np.eye(r))
    Hperp = H - HL1 @ Cinv @ HL1.T
    return HL1, C, Cinv, Hperp


def closed_form_l2(H: np.ndarray, L1: np.ndarray, E: np.ndarray) -> np.ndarray:
    """L2* = (L1^T H L1)^-1 L1^T H E (r x N)."""
    HL1, C, _, _ = deflate(H, L1)
    return np.linalg.solve(C, HL1.T @ E)


def deflated_error(Hperp: np.ndarray, E: np.ndarray) -> float:
    """tr(E^T Hperp E): the output error left after the best L2."""
    return float(np.einsum("kn,kn->", E, Hperp @ E))
