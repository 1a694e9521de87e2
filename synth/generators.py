"""Seeded synthetic layers.

Every tensor is drawn from
``numpy.random.default_rng(SeedSequence([261011315, cfg, layer, tensor]))``
in float64 and cast once, with round-to-nearest-even, to its storage type.
Half-precision tensors are returned as their uint16 bit patterns (bf16 or
fp16), int4 weight codes as int8 values in [-8, 7].

Shapes are those of the linear layers the pages evaluate (PixArt-Sigma,
SANA-1.6B, FLUX.1, Qwen3-8B); the activations imitate what reaches a DiT/LLM
linear layer: channel-varying spread plus a few outlier channels.  No
dataset, prompt or trained weight is used.

Layer dictionaries hold, with ``B`` = number of projections sharing X:
  X    (M, K)     uint16 bf16 bits    activations, row-major
  lam  (K,)       uint16 fp16 bits    smoothing factors (x is divided by them)
  qw   (B, K, N)  int8                residual codes, in x out
  sw   (B, G, N)  uint16 fp16 bits    residual scale per K group (G = K / group)
  L1   (B, K, r)  uint16 bf16 bits    input-side low-rank factor
  L2   (B, r, N)  uint16 bf16 bits    output-side low-rank factor
  bias (B, N)     uint16 bf16 bits
  group           int                 channels per quantization group (64 or 128)
"""

from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, Optional

import numpy as np

ROOT_SEED = 261011315
GROUP = 64          # default group width; 128 is the other one the library supports


# ---------------------------------------------------------------- conversions
def f64_to_bf16_bits(a) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits), ties to even.

    The value is scaled so that its 8 significant bits sit left of the binary
    point, rounded once with ``rint`` (ties to even) and scaled back; the
    result is exact in float32, whose top 16 bits are the bf16 pattern.
    """
    a = np.asarray(a, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite value")
    mant, expo = np.frexp(a)
    r = np.ldexp(np.rint(np.ldexp(mant, 8)), expo - 8)
    tiny = np.abs(a) < 2.0 ** -126  # bf16 subnormal range: fixed quantum 2^-133
    if np.any(tiny):
        r = np.where(tiny, np.ldexp(np.rint(np.ldexp(a, 133)), -133), r)
    f32 = r.astype(np.float32)
    if not np.all(np.isfinite(f32)):
        raise ValueError("value overflows bf16")
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def f64_to_f16_bits(a) -> np.ndarray:
    """float64 -> IEEE binary16 bit patterns, round to nearest even."""
    a = np.asarray(a, dtype=np.float64)
    h = a.astype(np.float16)
    if not np.all(np.isfinite(h)):
        raise ValueError("value overflows fp16")
    return h.view(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def f16_bits_to_f32(b) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


# ---------------------------------------------------------------- layer specs
@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    cfg: int          # workload index used in the seed (1..5)
    layer: int        # layer index used in the seed
    M: int
    K: int
    N: int
    r: int = 4
    batch: int = 1
    x_recipe: str = "smoke"
    x_rows: int = 0   # rows drawn before slicing to M (0: M)
    description: str = ""
    group: int = GROUP

    @property
    def G(self) -> int:
        return self.K // self.group

    @property
    def ops(self) -> int:
        """Integer MACs x 2 of the residual contraction (the counted work)."""
        return 2 * self.M * self.N * self.K * self.batch


LAYERS: Dict[str, LayerSpec] = {
    s.name: s
    for s in [
        LayerSpec("tiny", 1, 0, 64, 256, 256, x_recipe="smoke",
                  description="tiny smoke layer 64x256 -> 256"),
        LayerSpec("pixart_up", 2, 0, 4096, 1152, 4608, x_recipe="dit",
                  description="PixArt-Sigma MLP up-projection, 4096 tokens, 1152 -> 4608"),
        LayerSpec("sana_qkv", 3, 0, 4096, 2240, 2240, batch=3, x_recipe="dit",
                  description="SANA-1.6B attention Q/K/V, 4096 tokens, 3 x (2240 -> 2240)"),
        LayerSpec("flux_up", 4, 0, 4608, 3072, 12288, x_recipe="flux",
                  description="FLUX.1 joint-token MLP up, 4608 tokens, 3072 -> 12288"),
        LayerSpec("flux_down", 4, 1, 4608, 12288, 3072, x_recipe="flux",
                  description="FLUX.1 joint-token MLP down, 4608 tokens, 12288 -> 3072"),
        LayerSpec("qwen3_up", 5, 0, 2048, 4096, 12288, x_recipe="llm", x_rows=2048,
                  description="Qwen3-8B gate/up projection, 4096 -> 12288"),
        LayerSpec("qwen3_down", 5, 1, 2048, 12288, 4096, x_recipe="llm", x_rows=2048,
                  description="Qwen3-8B down projection, 12288 -> 4096"),
    ]
}


def layer_spec(name: str, M: Optional[int] = None, group: Optional[int] = None) -> LayerSpec:
    s = LAYERS[name]
    if M is not None and M != s.M:
        if s.x_rows and M > s.x_rows:
            raise ValueError(f"{name}: M={M} exceeds the {s.x_rows} drawn rows")
        s = dataclasses.replace(s, M=M)
    if group is not None and group != s.group:
        if group not in (64, 128) or s.K % group:
            raise ValueError(f"{name}: group {group} does not divide K = {s.K}")
        s = dataclasses.replace(s, group=group)
    return s


def _rng(cfg: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([ROOT_SEED, cfg, layer, tensor]))


# tensor ids inside one (cfg, layer)
_T_X, _T_OUTLIER, _T_STD, _T_LAM = 0, 1, 2, 3
_T_PROJ = 100  # + 10 * projection + {0 qw, 1 sw, 2 L1, 3 L2, 4 bias}


def _n_outliers(K: int, frac: float) -> int:
    return int(round(frac * K))


def _draw_x(spec: LayerSpec) -> np.ndarray:
    """float64 activations, before the bf16 cast."""
    c, l = spec.cfg, spec.layer
    rows = spec.x_rows or spec.M
    K = spec.K
    if spec.x_recipe == "smoke":
        x = _rng(c, l, _T_X).standard_normal((rows, K))
        idx = _rng(c, l, _T_OUTLIER).choice(K, 4, replace=False)
        x[:, idx] *= 20.0
    elif spec.x_recipe in ("dit", "flux"):
        std = np.exp(_rng(c, l, _T_STD).uniform(np.log(0.3), np.log(3.0), K))
        idx = _rng(c, l, _T_OUTLIER).choice(K, _n_outliers(K, 0.01), replace=False)
        g = _rng(c, l, _T_X)
        z = g.standard_normal((rows, K))
        if spec.x_recipe == "flux":
            # heavy-tailed outlier channels (Student-t, nu = 3)
            z[:, idx] = g.standard_t(3.0, (rows, idx.size))
        x = z * std
        x[:, idx] *= 30.0
        if spec.x_recipe == "flux" and rows > 4096:
            x[4096:, :] *= 5.0  # text tokens after the 4096 image tokens
    elif spec.x_recipe == "llm":
        x = _rng(c, l, _T_X).standard_normal((rows, K))
        idx = _rng(c, l, _T_OUTLIER).choice(K, _n_outliers(K, 0.005), replace=False)
        x[:, idx] *= 50.0
    else:
        raise ValueError(spec.x_recipe)
    return x


def _draw_projection(spec: LayerSpec, b: int):
    c, l = spec.cfg, spec.layer
    K, N, r, G = spec.K, spec.N, spec.r, spec.G
    t = _T_PROJ + 10 * b
    qw = _rng(c, l, t + 0).integers(-8, 8, size=(K, N), dtype=np.int8)
    sw = f64_to_f16_bits(np.exp(_rng(c, l, t + 1).uniform(np.log(1e-3), np.log(1e-2), (G, N))))
    L1 = f64_to_bf16_bits(_rng(c, l, t + 2).normal(0.0, 0.02, (K, r)))
    L2 = f64_to_bf16_bits(_rng(c, l, t + 3).normal(0.0, 0.02, (r, N)))
    if spec.x_recipe == "smoke":
        bias = np.zeros(N, dtype=np.uint16)
    else:
        bias = f64_to_bf16_bits(_rng(c, l, t + 4).normal(0.0, 0.02, N))
    return qw, sw, L1, L2, bias


def _sqrt_balanced_lambda(x_bf16: np.ndarray, qw: np.ndarray, sw: np.ndarray, group: int) -> np.ndarray:
    """lambda_j = fp16(sqrt(a_j / w_j)); a_j = max_m |X[m, j]|,
    w_j = max over projections and n of |qw[j, n] * sw[j // group, n]|."""
    a = np.abs(bf16_bits_to_f32(x_bf16)).max(axis=0).astype(np.float64)
    B, K, N = qw.shape
    w = np.zeros(K, dtype=np.float64)
    swf = f16_bits_to_f32(sw).astype(np.float64)  # (B, G, N)
    for b in range(B):
        for g in range(K // group):
            blk = np.abs(qw[b, g * group:(g + 1) * group, :].astype(np.float64)) * swf[b, g][None, :]
            w[g * group:(g + 1) * group] = np.maximum(w[g * group:(g + 1) * group], blk.max(axis=1))
    lam = np.sqrt(np.where((a > 0) & (w > 0), a / np.where(w > 0, w, 1.0), 1.0))
    lam = np.clip(lam, 2.0 ** -14, 60000.0)
    return f64_to_f16_bits(lam)


def make_layer(name: str, M: Optional[int] = None, group: Optional[int] = None) -> dict:
    """All tensors of one named layer (see ``LAYERS``), deterministic; `group`
    overrides its quantization group width (64 or 128)."""
    spec = layer_spec(name, M, group)
    x64 = _draw_x(spec)
    X_all = f64_to_bf16_bits(x64)
    del x64
    projs = [_draw_projection(spec, b) for b in range(spec.batch)]
    qw = np.stack([p[0] for p in projs])
    sw = np.stack([p[1] for p in projs])
    L1 = np.stack([p[2] for p in projs])
    L2 = np.stack([p[3] for p in projs])
    bias = np.stack([p[4] for p in projs])
    if spec.x_recipe == "smoke":
        lam = f64_to_f16_bits(np.exp(_rng(spec.cfg, spec.layer, _T_LAM).uniform(
            np.log(0.5), np.log(2.0), spec.K)))
    else:
        lam = _sqrt_balanced_lambda(X_all, qw, sw, spec.group)  # from all drawn rows
    X = np.ascontiguousarray(X_all[: spec.M])
    return dict(spec=spec, X=X, lam=lam, qw=qw, sw=sw, L1=L1, L2=L2, bias=bias, group=spec.group)


def make_random_layer(seed: int, M: int, K: int, N: int, r: int = 4, batch: int = 1,
                      outlier_channels: int = 0, outlier_scale: float = 20.0,
                      x_scale: float = 1.0, zero_bias: bool = False, group: int = GROUP) -> dict:
    """A generic seeded layer for edge-case tests (ragged M/N, other ranks).

    Same distributions as the smoke layer: X ~ N(0, x_scale^2) with optional
    outlier channels, lambda log-uniform in [0.5, 2], codes uniform in
    [-8, 7], weight scales log-uniform in [1e-3, 1e-2], L1/L2/bias
    ~ N(0, 0.02^2)."""
    if group not in (64, 128) or K % group:
        raise ValueError("K must be a multiple of the group width (64 or 128)")
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, 1000 + seed, M, K, N, r, batch]))
    x = rng.standard_normal((M, K)) * x_scale
    if outlier_channels:
        idx = rng.choice(K, outlier_channels, replace=False)
        x[:, idx] *= outlier_scale
    G = K // group
    qw = rng.integers(-8, 8, size=(batch, K, N), dtype=np.int8)
    sw = f64_to_f16_bits(np.exp(rng.uniform(np.log(1e-3), np.log(1e-2), (batch, G, N))))
    L1 = f64_to_bf16_bits(rng.normal(0.0, 0.02, (batch, K, r)))
    L2 = f64_to_bf16_bits(rng.normal(0.0, 0.02, (batch, r, N)))
    if zero_bias:
        bias = np.zeros((batch, N), dtype=np.uint16)
    else:
        bias = f64_to_bf16_bits(rng.normal(0.0, 0.02, (batch, N)))
    lam = f64_to_f16_bits(np.exp(rng.uniform(np.log(0.5), np.log(2.0), K)))
    spec = LayerSpec(f"random{seed}", 0, 0, M, K, N, r=r, batch=batch, x_recipe="random", group=group)
    return dict(spec=spec, X=f64_to_bf16_bits(x), lam=lam, qw=qw, sw=sw, L1=L1, L2=L2, bias=bias,
                group=group)


def make_full_weight(layer: dict, b: int = 0, noise: float = 1.0) -> np.ndarray:
    """A full-precision (smoothed) weight for projection `b` of `layer`, the
    input of the calibration steps: bf16 bits, shape (K, N), drawn as
    qw * sw + L1 * L2 + e with e uniform in [-noise/2, noise/2] * sw of its
    group, i.e. a weight whose residual codes round it within `noise` steps
    and whose low-rank factor is the layer's own.  A sampling recipe only:
    the calibration arithmetic itself is not done here."""
    spec = layer["spec"]
    K, N = layer["qw"].shape[1:]
    group = layer["group"]
    rng = np.random.default_rng(np.random.SeedSequence(
        [ROOT_SEED, 3000 + spec.cfg, spec.layer, K, N, b, zlib.crc32(spec.name.encode())]))
    swf = np.repeat(f16_bits_to_f32(layer["sw"][b]).astype(np.float64), group, axis=0)   # (K, N)
    base = layer["qw"][b].astype(np.float64) * swf
    low = bf16_bits_to_f32(layer["L1"][b]).astype(np.float64) @ bf16_bits_to_f32(layer["L2"][b]).astype(np.float64)
    e = rng.uniform(-0.5, 0.5, (K, N)) * noise * swf
    return f64_to_bf16_bits(base + low + e)

