"""CPU oracle for the MX-fp4 format variant of the layer (test infrastructure
only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  Plain NumPy; it shares nothing with the HIP library.

The variant keeps the method's layer, Y = Q(Xh) Q(R) + (Xh L1) L2 + b with
the same smoothing Xh = x * fl32(1/lambda), and swaps the 4-bit format: both
operands of the residual product are MX-fp4 (OCP Microscaling Formats v1.0,
the format gfx950's scaled MFMA consumes) instead of int4 with fp16 group-64
scales.  Per block of 32 consecutive values along the reduction dimension:

  * shared scale 2^X with X = floor(log2(amax)) - 2 (2 is the exponent of
    e2m1's largest normal, 6), stored as the e8m0 byte X + 127, clamped to
    [0, 254]; a block of zeros gets the byte 127 (scale 1);
  * elements: v = value / 2^X rounded to the nearest e2m1 value
    {0, 0.5, 1, 1.5, 2, 3, 4, 6} (ties to the even mantissa), magnitudes
    above 6 saturating to 6; the 4-bit code is the index of the magnitude in
    that list plus 8 when v's sign bit is set.  e2m1 is sign-magnitude, so a
    negative value whose magnitude rounds to 0 becomes -0 (code 8), as an
    IEEE-754 round-to-nearest-even conversion keeps the sign of a zero
    result; -0 and +0 contribute the same 0 to every product.

The activations are blocked along K per token, the residual along K per
output column.  The product is sum over blocks of 2^(Xa + Xw) times the
exact sum of the 32 element products, evaluated here in fp64.
"""

from __future__ import annotations

import numpy as np

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BLOCK = 32


def e2m1_round(v):
    """Nearest e2m1 magnitude of |v| (ties to even mantissa), saturating at
    6, with v's sign bit; returns (code 0..15, value)."""
    v = np.asarray(v, dtype=np.float64)
    m = np.abs(v)
    q = np.where(m < 2.0, np.rint(m * 2.0) / 2.0,
                 np.where(m < 4.0, np.rint(m), np.rint(m / 2.0) * 2.0))
    q = np.minimum(q, 6.0)
    idx = np.searchsorted(E2M1, q)
    neg = np.signbit(v)                      # the sign bit is kept, also when the magnitude rounds to 0
    code = idx + np.where(neg, 8, 0)
    return code.astype(np.uint8), np.where(neg, -q, q)


def quantize_blocks(x):
    """MX-fp4 along the last axis (a multiple of 32) of fp32 values x:
    (codes uint8 [..., n], scale bytes uint8 [..., n/32])."""
    x = np.asarray(x, dtype=np.float32)
    shp = x.shape
    xb = x.reshape(shp[:-1] + (shp[-1] // BLOCK, BLOCK))
    amax = np.abs(xb).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(amax.astype(np.float64)))
    X = np.where(amax > 0, e - 2, 0)
    sbyte = np.clip(X + 127, 0, 254).astype(np.int64)
    scale = np.ldexp(1.0, sbyte - 127)
    code, _ = e2m1_round(xb.astype(np.float64) / scale[..., None])
    return code.reshape(shp), sbyte.astype(np.uint8)


def dequantize_blocks(code, sbyte):
    code = np.asarray(code)
    mag = E2M1[code & 7]
    val = np.where(code & 8, -mag, mag)
    shp = code.shape
    vb = val.reshape(shp[:-1] + (shp[-1] // BLOCK, BLOCK))
    return (vb * np.ldexp(1.0, sbyte.astype(np.int64) - 127)[..., None]).reshape(shp)


def smoothed(X_bits, lam_bits):
    x = (X_bits.astype(np.uint32) << 16).view(np.float32)
    inv = np.float32(1.0) / lam_bits.view(np.float16).astype(np.float32)
    return (x * inv[None, :]).astype(np.float32)


def quantize_act(X_bits, lam_bits):
    """Codes (M x K) and scale bytes (M x K/32) of the smoothed activations."""
    return quantize_blocks(smoothed(X_bits, lam_bits))


def quantize_weight(R):
    """Codes (K x N) and scale bytes (K/32 x N) of a residual R (K x N, fp32),
    blocked along K per column."""
    c, s = quantize_blocks(np.asarray(R, dtype=np.float32).T)
    return c.T.copy(), s.T.copy()


def linear(X_bits, lam_bits, R, L1_bits=None, L2_bits=None, bias_bits=None, rows=None):
    """Y (fp64) of the MX-fp4 layer: deq(Q(Xh)) deq(Q(R)) + (Xh L1) L2 + b."""
    xh = smoothed(X_bits, lam_bits)
    if rows is not None:
        xh = xh[rows]
    ca, sa = quantize_blocks(xh)
    cw, sw = quantize_weight(R)
    Y = dequantize_blocks(ca, sa) @ dequantize_blocks(cw.T, sw.T).T
    if L1_bits is not None and L1_bits.shape[-1]:
        L1 = (L1_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        L2 = (L2_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        Y += (xh.astype(np.float64) @ L1) @ L2
    if bias_bits is not None:
        Y += (bias_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)[None, :]
    return Y
