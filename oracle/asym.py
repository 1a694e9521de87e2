"""CPU oracle for the asymmetric-activation variant of the layer (test
infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  Plain NumPy; it shares nothing with the HIP library.

DiRotQ notes (papernotes.org), experimental setup: its INT W4A4 setting
quantizes activations asymmetrically in groups of 64 channels per token
and the weights symmetrically.  The page prints no formula; the reading
taken here is the usual min-max uniform quantizer with 16 levels, its
range widened to contain 0 (so that 0 is a level and the zero point is an
integer in [0, 15]), with the same smoothing, fp16 scale and fp32 rounding
steps as the symmetric quantizer of the layer:

  xh  = fl32(X * fl32(1 / lambda))
  lo  = min(0, min over the group of xh),  hi = max(0, max over the group)
  s   = 0 if hi == lo, else f16_rne(fl32(fl32(hi - lo) / 15)), saturated at 65504
  inv = fl32(1 / s)  (0 if s == 0)
  z   = clamp(rint(fl32(-lo * inv)), 0, 15)              zero point
  q   = clamp(rint(fl32(xh * inv)) + z, 0, 15)           4-bit code
  deq = (q - z) * s

Weights stay symmetric int4 with fp16 group scales, so the residual
product per group is s * sw * sum (q - z) qw, an exact integer sum times
two scales; the rank branch and the bias are those of the layer.
"""

from __future__ import annotations

import numpy as np


def smoothed(X_bits, lam_bits):
    """fl32(X * fl32(1 / lambda)) from bf16 X and fp16 lambda bit patterns."""
    x = (np.asarray(X_bits).astype(np.uint32) << 16).view(np.float32)
    inv = np.float32(1.0) / np.asarray(lam_bits).view(np.float16).astype(np.float32)
    return (x * inv[None, :]).astype(np.float32)


def quantize(xh, group=64):
    """Codes q (uint8, M x K, in [0, 15]), zero points z (uint8, M x K/group)
    and scale bit patterns s16 (uint16, M x K/group) of fp32 xh."""
    xh = np.asarray(xh, dtype=np.float32)
    M, K = xh.shape
    xg = xh.reshape(M, K // group, group)
    lo = np.minimum(xg.min(axis=2), np.float32(0.0))
    hi = np.maximum(xg.max(axis=2), np.float32(0.0))
    rng = (hi - lo).astype(np.float32)
    with np.errstate(over="ignore"):
        s = (rng / np.float32(15.0)).astype(np.float32).astype(np.float16)
    s = np.where(np.isinf(s), np.float16(65504.0), s)
    s = np.where(rng == 0, np.float16(0.0), s)
    s32 = s.astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(s32 != 0, np.float32(1.0) / s32, np.float32(0.0)).astype(np.float32)
    z = np.clip(np.rint((-lo * inv).astype(np.float32)), 0, 15)
    t = (xg * inv[:, :, None]).astype(np.float32)
    q = np.clip(np.rint(t) + z[:, :, None], 0, 15)
    return q.reshape(M, K).astype(np.uint8), z.astype(np.uint8), s.view(np.uint16)


def stored_codes(q, z, group=64):
    """q - z (int8, in [-15, 15]): the value each code stands for in units
    of its group's scale."""
    M, K = q.shape
    d = q.reshape(M, K // group, group).astype(np.int16) - z[:, :, None].astype(np.int16)
    return d.reshape(M, K).astype(np.int8)


def partials(X_bits, lam_bits, qw, group=64, rows=None):
    """P[m, n, g] = sum over channel k of group g of (q - z)[m, k] * qw[k, n]
    (int64), qw: K x N int8 weight codes."""
    xh = smoothed(X_bits, lam_bits)
    if rows is not None:
        xh = xh[rows]
    q, z, _ = quantize(xh, group)
    d = stored_codes(q, z, group).astype(np.int64)
    M, K = d.shape
    G = K // group
    qw = np.asarray(qw).astype(np.int64)
    P = np.empty((M, qw.shape[1], G), dtype=np.int64)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        P[:, :, g] = d[:, sl] @ qw[sl, :]
    return P


def linear(X_bits, lam_bits, qw, sw_bits, L1_bits=None, L2_bits=None, bias_bits=None, group=64,
           rows=None):
    """Y (fp64) = sum_g P * s * sw + (xh L1) L2 + b for the chosen rows."""
    xh = smoothed(X_bits, lam_bits)
    if rows is not None:
        xh = xh[rows]
    q, z, s16 = quantize(xh, group)
    d = stored_codes(q, z, group).astype(np.int64)
    M, K = d.shape
    G = K // group
    qw = np.asarray(qw).astype(np.int64)
    sx = s16.view(np.float16).astype(np.float64)
    sw = np.asarray(sw_bits).view(np.float16).astype(np.float64)
    Y = np.zeros((M, qw.shape[1]), dtype=np.float64)
    for g in range(G):
        sl = slice(g * group, (g + 1) * group)
        P = (d[:, sl] @ qw[sl, :]).astype(np.float64)
        Y += P * sx[:, g:g + 1] * sw[g][None, :]
    if L1_bits is not None and np.asarray(L1_bits).shape[-1]:
        L1 = (np.asarray(L1_bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        L2 = (np.asarray(L2_bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        Y += (xh.astype(np.float64) @ L1) @ L2
    if bias_bits is not None:
        Y += (np.asarray(bias_bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)[None, :]
    return Y
