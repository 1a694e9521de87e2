"""CPU oracle for the fused two-layer chain (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  Plain NumPy; it shares nothing with the HIP library.

The chain Y = down(act(up(X))) of a diffusion-transformer MLP, with the down
layer's input quantized from the fp32 activation of the up layer's output
(never rounded to bf16).  What the oracle fixes:

  * the activation: GELU in its tanh form, 0.5 y (1 + tanh(z)) with
    z = sqrt(2/pi) (y + 0.044715 y^3), evaluated in fp32 as y / (1 + e(-2z))
    where e is the exponential built from basic operations stated in
    include/hsq.h (each operation rounded once), so that the fp32 result is
    a defined function of y;
  * the quantizer of the layer's input (Deflating the Hessian: W4A4,
    group-64; the formula block of include/hsq.h) applied to that fp32
    activation: xh = fl32(a * fl32(1/lambda)), s = fp16(fl32(amax/7))
    saturating at 65504, code = clamp(rint(fl32(xh / s)), -8, 7) against the
    stored fp16 s (reciprocal-multiply), zero groups give scale and codes 0;
  * the rank-r branch of the down layer on the smoothed, unquantized xh, and
    the down layer's output from the codes, scales and U (fp64).
"""

from __future__ import annotations

import numpy as np

F = np.float32


def exp_f32_basic(x):
    """exp in fp32 from basic operations (the definition in include/hsq.h)."""
    x = np.asarray(x, dtype=F)
    x = np.minimum(np.maximum(x, F(-87.0)), F(88.0))
    n = np.rint(x * F(1.44269504))
    r = (x - n * F(0.693145751953125)) - n * F(1.428606765330187e-06)
    p = np.full_like(r, F(1.388888888888889e-03))
    for c in (8.333333333333333e-03, 4.166666666666666e-02, 1.666666666666667e-01, 0.5, 1.0, 1.0):
        p = p * r + F(c)
    two_n = ((n.astype(np.int32) + 127) << 23).view(F)
    return (p * two_n).astype(F)


def gelu_tanh_f32(y):
    y = np.asarray(y, dtype=F)
    y3 = (y * y) * y
    z = F(0.7978845608) * (y + F(0.044715) * y3)
    return (y / (F(1.0) + exp_f32_basic(F(-2.0) * z))).astype(F)


def activation(y, act: str):
    if act == "identity":
        return np.asarray(y, dtype=F)
    if act == "gelu_tanh":
        return gelu_tanh_f32(y)
    raise ValueError(act)


def quantize_f32(a, lam_bits, group: int = 64):
    """Codes (int8), fp16 scale bits (uint16) and the smoothed xh (fp32) of
    an fp32 input a (M x K) with smoothing lambda (fp16 bits)."""
    a = np.asarray(a, dtype=F)
    M, K = a.shape
    G = K // group
    inv = F(1.0) / lam_bits.view(np.float16).astype(F)
    xh = (a * inv[None, :]).astype(F)
    xg = xh.reshape(M, G, group)
    amax = np.abs(xg).max(axis=2)
    with np.errstate(over="ignore"):
        s16 = (amax / F(7.0)).astype(np.float16)
    s16 = np.where(np.isinf(s16), np.float16(65504.0), s16)
    s16 = np.where(amax == 0, np.float16(0.0), s16)
    s = s16.astype(F)
    with np.errstate(divide="ignore"):
        inv_s = np.where(s16 != 0, F(1.0) / s, F(0.0)).astype(F)
    t = (xg * inv_s[:, :, None]).astype(F)
    q = np.clip(np.rint(t), -8, 7).astype(np.int8).reshape(M, K)
    return q, s16.view(np.uint16), xh


def hidden(yhid, lam_bits, L1_bits, act: str, group: int = 64):
    """The down layer's input formed from the up layer's fp32 output:
    (codes, scale bits, U fp64) with U = xh L1 (L1 bf16 bits, K x r)."""
    a = activation(yhid, act)
    q, s16, xh = quantize_f32(a, lam_bits, group)
    L1 = (L1_bits.astype(np.uint32) << 16).view(F).astype(np.float64)
    return q, s16, xh.astype(np.float64) @ L1


def down_output(q, s16, U, qw, sw_bits, L2_bits, bias_bits, group: int = 64):
    """Y = sum_g P_g sx sw + U L2 + b in fp64 from the codes (M x K), the
    scales (M x K/group) and U (M x r) of the down layer's input."""
    M, K = q.shape
    G = K // group
    sx = s16.view(np.float16).astype(np.float64)
    sw = sw_bits.view(np.float16).astype(np.float64)
    Y = np.zeros((M, qw.shape[1]))
    for g in range(G):
        P = q[:, g * group:(g + 1) * group].astype(np.int64) @ qw[g * group:(g + 1) * group].astype(np.int64)
        Y += P.astype(np.float64) * sx[:, g:g + 1] * sw[g][None, :]
    if U.shape[1]:
        L2 = (L2_bits.astype(np.uint32) << 16).view(F).astype(np.float64)
        Y += U @ L2
    if bias_bits is not None:
        Y += (bias_bits.astype(np.uint32) << 16).view(F).astype(np.float64)[None, :]
    return Y
