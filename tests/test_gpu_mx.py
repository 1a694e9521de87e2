"""MX-fp4 variant of the layer (hsq_mx_pack_weights, hsq_mx_lowrank_linear)
vs the CPU oracle (oracle/mx.py), through the C ABI, on seeded inputs.

Bars: the packed weight codes and e8m0 scales, and the activation codes and
scales (decoded from the workspace), bit-exact; U relative Frobenius
<= 1e-5; Y fp32 within 1e-3 relative Frobenius of the oracle's fp64 result,
bf16 within 1e-3 of that result rounded to bf16.  The residual is the int4
layer's own dequantized residual qw * sw (exact in fp32), re-quantized to
MX-fp4.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a4_rank_assisted_amd as hsq  # noqa: E402
from oracle import mx  # noqa: E402
from synth import bf16_bits_to_f32, f64_to_bf16_bits, make_layer, make_random_layer  # noqa: E402

DEV = torch.device("cuda:0")
TOL = 1e-3


def say(msg):
    print(msg, flush=True)


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def align(v, a=256):
    return -(-v // a) * a


def residual(lay):
    sw = lay["sw"][0].view(np.float16).astype(np.float32)
    return (lay["qw"][0].astype(np.float32) * np.repeat(sw, lay["group"], axis=0)).astype(np.float32)


def decode_blob(raw, tiles, KS, rows, K):
    """codes [tiles*16 rows][4*KS*32 channels] -> [:rows, :K] and scales
    [rows][K/32] from a blob (codes, then scales)."""
    KS4 = -(-KS // 4)
    b = raw[: tiles * KS * 1024].reshape(tiles, KS, 4, 16, 16)          # t, ks, kb, r, byte
    lo, hi = b & 15, b >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(tiles, KS, 4, 16, 32)      # element 2i low, 2i+1 high
    codes = nib.transpose(0, 3, 1, 2, 4).reshape(tiles * 16, KS * 128)[:rows, :K]
    s = raw[tiles * KS * 1024: tiles * KS * 1024 + tiles * KS4 * 256].reshape(tiles, KS4, 4, 16, 4)  # t, ks4, kb, r, j
    sc = s.transpose(0, 3, 1, 4, 2).reshape(tiles * 16, KS4 * 16)[:rows, : K // 32]
    return codes, sc


def run_case(lay, rows=None):
    M, K = lay["X"].shape
    N = lay["qw"].shape[2]
    r = lay["L1"].shape[2]
    say(f"[mx] M={M} K={K} N={N} r={r}")
    R = residual(lay)
    packed = hsq.mx_pack_weights(torch.from_numpy(R).to(DEV))
    torch.cuda.synchronize()
    KS, NT, MT = -(-K // 128), -(-N // 16), -(-M // 16)
    wc, ws = decode_blob(packed.cpu().numpy(), NT, KS, N, K)
    oc, osc = mx.quantize_weight(R)
    assert np.array_equal(wc, oc.T) and np.array_equal(ws, osc.T)
    X, lam = dev16(lay["X"]), dev16(lay["lam"])
    L1 = dev16(lay["L1"][0]) if r else None
    L2 = dev16(lay["L2"][0]) if r else None
    bias = dev16(lay["bias"][0])
    wsp = torch.zeros(hsq._load().hsq_mx_workspace_bytes(M, K, r), dtype=torch.uint8, device=DEV)
    Y = hsq.mx_lowrank_linear(X, lam, packed, L1, L2, bias, N=N, y_dtype="f32", workspace=wsp)
    Yb = hsq.mx_lowrank_linear(X, lam, packed, L1, L2, bias, N=N, y_dtype="bf16").float()
    torch.cuda.synchronize()
    raw = wsp.cpu().numpy()
    qa_off = 0
    blob = raw[qa_off: qa_off + MT * KS * 1024]
    sa_off = align(qa_off + MT * KS * 1024)
    sc = raw[sa_off: sa_off + MT * (-(-KS // 4)) * 256]
    ac, asc = decode_blob(np.concatenate([blob, sc]), MT, KS, M, K)
    oac, oas = mx.quantize_act(lay["X"], lay["lam"])
    assert np.array_equal(ac, oac) and np.array_equal(asc, oas)
    rows = np.arange(M) if rows is None else rows
    if r:
        u_off = align(sa_off + MT * (-(-KS // 4)) * 256)
        Mpad = MT * 16
        S = -(-KS // 4)                        # U partials: one per four k-steps, summed in order
        Us = raw[u_off: u_off + S * r * Mpad * 4].view(np.float32).reshape(S, r, Mpad)
        U = Us[0].astype(np.float32)
        for sl in range(1, S):
            U = (U + Us[sl]).astype(np.float32)
        U = U[:, :M].T
        xh = mx.smoothed(lay["X"], lay["lam"]).astype(np.float64)
        L1f = (lay["L1"][0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert rel(U.astype(np.float64), xh @ L1f) <= 1e-5
    ref = mx.linear(lay["X"], lay["lam"], R, lay["L1"][0] if r else None, lay["L2"][0] if r else None,
                    lay["bias"][0], rows=rows)
    e32 = rel(Y.cpu().numpy()[rows].astype(np.float64), ref)
    ref_b = bf16_bits_to_f32(f64_to_bf16_bits(ref)).astype(np.float64)
    e16 = rel(Yb.cpu().numpy()[rows].astype(np.float64), ref_b)
    say(f"    codes/scales exact; Y fp32 rel {e32:.3e}, bf16 rel {e16:.3e}")
    assert e32 <= TOL and e16 <= TOL


@pytest.mark.parametrize("M,K,N,r", [
    (5, 192, 33, 0),          # rank 0, ragged N, one row tile, a k-step of one 64-block pad
    (70, 576, 300, 4),        # 18 blocks: the last k-step half padded
    (130, 1024, 130, 7),      # odd rank (scalar L1 reads), ragged rows and columns
    (200, 2048, 256, 32),     # largest rank
])
def test_mx_matches_oracle(M, K, N, r):
    run_case(make_random_layer(700 + M, M, K, N, r=r, outlier_channels=3))


@pytest.mark.parametrize("K,r", [
    (1536, 4),    # 12 k-steps: three whole groups of four
    (1152, 4),    # 9: one k-step past the last group
    (1280, 0),    # 10: two past it, rank 0
    (1408, 2),    # 11: three past it, rank 2
    (256, 4),     # 2: no whole group at all
])
def test_mx_wide_tiles_sampled_rows(K, r):
    # 2100 x 4100 at rank <= 4 runs the 128 x 256 workgroups (17 x 17 of
    # them, the last row and column tiles ragged); sampled rows cover every
    # column
    M, N = 2100, 4100
    rows = np.array(sorted(set([0, 127, 128, M - 1]) |
                           set(np.random.default_rng(K).choice(M, 40, replace=False).tolist())))
    run_case(make_random_layer(900 + K + r, M, K, N, r=r, outlier_channels=3), rows)


def test_mx_pixart_full_size_sampled_rows():
    lay = make_layer("pixart_up")
    rows = np.array(sorted(set([0, 4095]) | set(np.random.default_rng(5).choice(4096, 30, replace=False).tolist())))
    run_case(lay, rows)


def test_mx_degenerate_blocks():
    # a zero token, a zero 32-block, blocks whose scale clamps at the small
    # end, a block of huge values, an all-negative block (signed zeros among
    # its codes), a constant block
    M, K, N = 48, 512, 64
    lay = make_random_layer(711, M, K, N, r=4)
    x = bf16_bits_to_f32(lay["X"]).astype(np.float64)
    x[3, :] = 0.0
    x[7, 32:64] = 0.0
    x[9, 64:96] *= 2.0 ** -60
    x[10, 96:128] *= 2.0 ** -120
    x[11, 128:160] *= 1.0e30
    x[12, 160:192] = -np.abs(x[12, 160:192]) * 0.01
    x[13, 192:224] = 0.75
    lay["X"] = f64_to_bf16_bits(x)
    run_case(lay)
