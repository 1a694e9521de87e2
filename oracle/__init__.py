"""CPU oracle for the W4A4 + rank-r linear layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``hsq_oracle.c`` (plain C, fp64 results,
OpenMP over rows) through ctypes and shares nothing with the HIP library.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hsq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
GROUP = 64          # the default group width; 128 is the other one supported
GROUPS = (64, 128)

_lib = None


def build(force: bool = True, extra_flags: Sequence[str] = (), out: Optional[str] = None) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    out = out or _LIB
    if force or not os.path.exists(out):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
               *extra_flags, "-o", out + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return out


def _load(path: Optional[str] = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_f16_rne.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16_rne.restype = ctypes.c_uint16
    lib.oracle_quantize_act.argtypes = [P, I, I, P, P, P, P]
    lib.oracle_quantize_act.restype = None
    lib.oracle_quantize_act_g.argtypes = [P, I, I, I, P, P, P, P]
    lib.oracle_quantize_act_g.restype = None
    lib.oracle_pack_act.argtypes = [P, I, I, P]
    lib.oracle_pack_act.restype = None
    lib.oracle_group_partials.argtypes = [P, P, I, I, I, I, I, I, I, P]
    lib.oracle_group_partials.restype = None
    lib.oracle_group_partials_g.argtypes = [P, P, I, I, I, I, I, I, I, I, P]
    lib.oracle_group_partials_g.restype = None
    lib.oracle_lowrank_down.argtypes = [P, I, I, P, I, P]
    lib.oracle_lowrank_down.restype = None
    lib.oracle_linear.argtypes = [P, I, I, I, P, P, P, P, P, I, P, P, I, P]
    lib.oracle_linear.restype = None
    lib.oracle_linear_g.argtypes = [P, I, I, I, I, P, P, P, P, P, I, P, P, I, P]
    lib.oracle_linear_g.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I
    lib.oracle_set_num_threads.argtypes = [I]
    lib.oracle_set_num_threads.restype = None
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """Thin ctypes front end; every method mirrors one C function."""

    def __init__(self, lib_path: Optional[str] = None):
        self.lib = _load(lib_path)

    # number formats
    def f32_to_f16(self, x: float) -> int:
        return int(self.lib.oracle_f32_to_f16_rne(float(x)))

    def f16_to_f32(self, h: int) -> float:
        return float(self.lib.oracle_f16_to_f32(int(h)))

    def bf16_to_f32(self, b: int) -> float:
        return float(self.lib.oracle_bf16_to_f32(int(b)))

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    # steps 1-4
    def quantize(self, X, lam, want_xh: bool = False, group: int = GROUP):
        X = _c(X, np.uint16)
        lam = _c(lam, np.uint16)
        M, K = X.shape
        if group not in GROUPS or K % group:
            raise ValueError("group must be 64 or 128 and divide K")
        q = np.empty((M, K), np.int8)
        sx = np.empty((M, K // group), np.uint16)
        xh = np.empty((M, K), np.float32) if want_xh else None
        self.lib.oracle_quantize_act_g(_ptr(X), M, K, group, _ptr(lam), _ptr(q), _ptr(sx), _ptr(xh))
        return (q, sx, xh) if want_xh else (q, sx)

    def pack_act(self, q):
        q = _c(q, np.int8)
        M, K = q.shape
        out = np.empty((M, K // 2), np.uint8)
        self.lib.oracle_pack_act(_ptr(q), M, K, _ptr(out))
        return out

    # step 5
    def group_partials(self, qa, qw, m0=0, mc=None, n0=0, nc=None, group: int = GROUP):
        qa = _c(qa, np.int8)
        qw = _c(qw, np.int8)
        M, K = qa.shape
        K2, N = qw.shape
        assert K == K2 and group in GROUPS and K % group == 0
        mc = M - m0 if mc is None else mc
        nc = N - n0 if nc is None else nc
        assert 0 <= m0 and m0 + mc <= M and 0 <= n0 and n0 + nc <= N
        P = np.empty((mc, nc, K // group), np.int32)
        self.lib.oracle_group_partials_g(_ptr(qa), _ptr(qw), M, K, N, group, m0, mc, n0, nc, _ptr(P))
        return P

    def lowrank_down(self, xh, L1):
        xh = _c(xh, np.float32)
        L1 = _c(L1, np.uint16)
        M, K = xh.shape
        r = L1.shape[1] if L1.ndim == 2 else 0
        U = np.empty((M, r), np.float64)
        if r:
            self.lib.oracle_lowrank_down(_ptr(xh), M, K, _ptr(L1), r, _ptr(U))
        return U

    # steps 1-7
    def linear(self, X, lam, qw, sw, L1=None, L2=None, bias=None, rows=None, group: int = GROUP):
        """fp64 Y for one projection; ``rows`` selects output rows (None: all);
        sw is (K/group) x N."""
        X = _c(X, np.uint16)
        lam = _c(lam, np.uint16)
        qw = _c(qw, np.int8)
        sw = _c(sw, np.uint16)
        M, K = X.shape
        N = qw.shape[1]
        assert group in GROUPS and K % group == 0 and sw.shape == (K // group, N)
        r = 0 if L1 is None else int(L1.shape[1])
        L1c = _c(L1, np.uint16) if r else None
        L2c = _c(L2, np.uint16) if r else None
        bc = None if bias is None else _c(bias, np.uint16)
        if rows is None:
            rows_c, nrows = None, M
        else:
            rows_c = _c(rows, np.int32)
            nrows = rows_c.size
            assert np.all((rows_c >= 0) & (rows_c < M))
        Y = np.empty((nrows, N), np.float64)
        self.lib.oracle_linear_g(_ptr(X), M, K, N, group, _ptr(lam), _ptr(qw), _ptr(sw), _ptr(L1c),
                                 _ptr(L2c), r, _ptr(bc), _ptr(rows_c), nrows, _ptr(Y))
        return Y

    def linear_batched(self, layer: dict, rows=None):
        """Y for every projection of a generated layer: (B, rows, N) fp64
        (the layer's "group", 64 when absent)."""
        B = layer["qw"].shape[0]
        r = layer["L1"].shape[2]
        group = int(layer.get("group", GROUP))
        return np.stack([
            self.linear(layer["X"], layer["lam"], layer["qw"][b], layer["sw"][b],
                        layer["L1"][b] if r else None, layer["L2"][b] if r else None,
                        layer["bias"][b], rows=rows, group=group)
            for b in range(B)])
