"""The linear at the largest sizes the C ABI accepts (M*K, M*N and K*N each
below 2^31 - 1), through the launch configuration the library picks.

Inputs of that size cannot be generated, and checked, row by row on the
host, so each case repeats a few seeded base rows (or base weight columns)
on the device (a torch gather: plumbing, no arithmetic of the method).  Two
checks then cover the whole output:
  * a property that holds at any size: the quantizer works per token and
    the contraction per output column, with one fixed order of arithmetic
    for every tile, so every repeated row (column) equals its base row
    (column) bit for bit;
  * the CPU oracle on the base rows (columns): Y within 1e-3 relative
    Frobenius, and a window of the int32 group partial sums at the far
    corner of the output, bit-exact.
A period of 7 (rows) or 5 (columns) puts an addressing error of a power of
two on a different base row or column.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a4_rank_assisted_amd as hsq  # noqa: E402
from synth import make_random_layer  # noqa: E402

DEV = torch.device("cuda:0")
TOL = 1e-3
LIMIT = 2**31 - 1                     # the ABI rejects M*K, M*N or K*N at or above this


def say(msg):
    print(msg, flush=True)


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(DEV)


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def test_largest_token_count_tiled(oracle):
    K, N, P = 65536, 80, 7
    M = (LIMIT - 1) // K               # 32767: the largest M the ABI accepts at this K
    assert M * K < LIMIT <= (M + 1) * K
    base = make_random_layer(1201, P, K, N, r=4, outlier_channels=3)
    say(f"[limits] tiled M={M} K={K} N={N}: X {2 * M * K / 2**30:.2f} GiB")
    idx = torch.arange(M, device=DEV) % P
    X = dev16(base["X"]).index_select(0, idx)
    lam = dev16(base["lam"])
    packed, st = hsq.pack_weights(dev8(base["qw"][0]))
    assert int(st[0].item()) == 0
    sw, L1, L2, b = (dev16(base[k][:1]) for k in ("sw", "L1", "L2", "bias"))
    Y = hsq.w4a4_lowrank_linear(X, lam, packed, sw, L1, L2, b, N=N, y_dtype="f32")[0]
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy()
    del Y
    rows = np.arange(M) % P
    assert np.array_equal(Yh.view(np.int32), Yh[rows].view(np.int32))
    ref = oracle.linear(base["X"], base["lam"], base["qw"][0], base["sw"][0], base["L1"][0], base["L2"][0],
                        base["bias"][0])
    e = rel(Yh[:P].astype(np.float64), ref)
    say(f"    rows repeat bit for bit; base rows fp32 rel {e:.3e}")
    assert e <= TOL
    m0, mc, n0, nc = M - 20, 20, N - 24, 24
    got = hsq.w4a4_group_partials(X, lam, packed, N, m0, mc, n0, nc, kernel="tiled")
    torch.cuda.synchronize()
    q, _ = oracle.quantize(base["X"], base["lam"])
    ref_p = oracle.group_partials(q, base["qw"][0], 0, P, n0, nc)
    assert np.array_equal(got.cpu().numpy(), ref_p[np.arange(m0, m0 + mc) % P])
    del X, got
    torch.cuda.empty_cache()


def test_largest_weight_skinny(oracle):
    M, K, P = 16, 65536, 5
    N = (LIMIT - 1) // K               # 32767: the largest N the ABI accepts at this K
    assert K * N < LIMIT <= K * (N + 1)
    base = make_random_layer(1202, M, K, P, r=4, outlier_channels=3)
    say(f"[limits] skinny M={M} K={K} N={N}: codes {K * N / 2**30:.2f} GiB")
    idx = torch.arange(N, device=DEV) % P
    codes = dev8(base["qw"][0]).index_select(1, idx)
    packed, st = hsq.pack_weights(codes)
    assert int(st[0].item()) == 0
    del codes
    X, lam = dev16(base["X"]), dev16(base["lam"])
    sw = dev16(base["sw"][:1]).index_select(2, idx)
    L1 = dev16(base["L1"][:1])
    L2 = dev16(base["L2"][:1]).index_select(2, idx)
    b = dev16(base["bias"][:1]).index_select(1, idx)
    Y = hsq.w4a4_lowrank_linear(X, lam, packed, sw, L1, L2, b, N=N, y_dtype="f32")[0]
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy()
    cols = np.arange(N) % P
    assert np.array_equal(Yh.view(np.int32), Yh[:, cols].view(np.int32))
    ref = oracle.linear(base["X"], base["lam"], base["qw"][0], base["sw"][0], base["L1"][0], base["L2"][0],
                        base["bias"][0])
    e = rel(Yh[:, :P].astype(np.float64), ref)
    say(f"    columns repeat bit for bit; base columns fp32 rel {e:.3e}")
    assert e <= TOL
    m0, mc, n0, nc = 0, M, N - 21, 21
    got = hsq.w4a4_group_partials(X, lam, packed, N, m0, mc, n0, nc, kernel="skinny")
    torch.cuda.synchronize()
    q, _ = oracle.quantize(base["X"], base["lam"])
    ref_p = oracle.group_partials(q, base["qw"][0], 0, M, 0, P)
    assert np.array_equal(got.cpu().numpy(), ref_p[:, np.arange(n0, n0 + nc) % P])
    del packed, sw, Y, got
    torch.cuda.empty_cache()
