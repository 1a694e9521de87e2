"""The fused two-layer chain (hsq_w4a4_lowrank_mlp) vs the CPU oracle,
through the C ABI, on seeded inputs.

The up layer's fp32 output before the activation is exported by the same
launch (Y_hidden); the oracle (oracle/chain.py) forms the down layer's input
from it.  Bars:
  * Y_hidden equals the ordinary up layer's fp32 output bit for bit (same
    contraction, same summation order);
  * the down layer's codes and fp16 scales (decoded from the workspace):
    bit-exact;
  * its U: relative Frobenius <= 1e-5 (fp32 sums vs fp64);
  * Y: fp32 within 1e-3 relative Frobenius of the oracle's fp64 output from
    those codes; bf16 within 1e-3 of that output rounded to bf16.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a4_rank_assisted_amd as hsq  # noqa: E402
from oracle import chain  # noqa: E402
from synth import bf16_bits_to_f32, f64_to_bf16_bits, make_layer, make_random_layer  # noqa: E402

DEV = torch.device("cuda:0")
TOL = 1e-3


def say(msg):
    print(msg, flush=True)


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(DEV)


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def align(v, a=256):
    return -(-v // a) * a


def upload(lay):
    packed, st = hsq.pack_weights(dev8(lay["qw"][0]))
    assert int(st[0].item()) == 0
    r = lay["L1"].shape[2]
    return dict(lam=dev16(lay["lam"]), packed=packed, sw=dev16(lay["sw"][0]),
                L1=dev16(lay["L1"][0]) if r else None, L2=dev16(lay["L2"][0]) if r else None,
                bias=dev16(lay["bias"][0]))


def decode_down(ws, M, K, H, r1, r2):
    """codes (M x H), scale bits (M x H/64) and U (M x r2) of the down
    layer's input, from the chain's workspace (up layer's workspace, then
    the down layer's: MT x Gp blocks of codes in MFMA lane order, MT x Gp x
    16 fp16 scales, U slices)."""
    raw = ws.cpu().numpy()
    up_total = hsq.workspace_bytes(M, K, H, r1, 1)
    base = align(up_total)
    MT, Gp = -(-M // 16), -(-H // 64 // 2) * 2
    qbytes = MT * Gp * 1024
    qa = raw[base: base + qbytes].view(np.int8).reshape(MT, Gp, 4, 16, 16)
    codes = qa.transpose(0, 3, 1, 2, 4).reshape(MT * 16, Gp * 64)[:M, :H]
    soff = base + align(qbytes)
    sx = raw[soff: soff + MT * Gp * 32].view(np.uint16).reshape(MT, Gp, 16)
    scales = sx.transpose(0, 2, 1).reshape(MT * 16, Gp)[:M, : H // 64]
    uoff = align(soff + MT * Gp * 32)
    U = raw[uoff: uoff + r2 * MT * 16 * 4].view(np.float32).reshape(r2, MT * 16)[:, :M].T
    return codes, scales, U


def run_case(up_lay, dn_lay, act, rows=None):
    M, K = up_lay["X"].shape
    H = up_lay["qw"].shape[2]
    N = dn_lay["qw"].shape[2]
    r1, r2 = up_lay["L1"].shape[2], dn_lay["L1"].shape[2]
    say(f"[chain] M={M} K={K} H={H} N={N} r={r1}/{r2} act={act}")
    X = dev16(up_lay["X"])
    up, dn = upload(up_lay), upload(dn_lay)
    ws = torch.zeros(hsq.mlp_workspace_bytes(M, K, H, N, r1, r2), dtype=torch.uint8, device=DEV)
    yh = torch.empty((M, H), dtype=torch.float32, device=DEV)
    Y32 = hsq.w4a4_lowrank_mlp(X, up, dn, H=H, N=N, act=act, y_dtype="f32", hidden_out=yh, workspace=ws)
    torch.cuda.synchronize()
    codes, scales, U = decode_down(ws, M, K, H, r1, r2)
    Yb = hsq.w4a4_lowrank_mlp(X, up, dn, H=H, N=N, act=act, y_dtype="bf16").float()
    torch.cuda.synchronize()
    # the pre-activation export is the ordinary layer's fp32 output
    plain = hsq.w4a4_lowrank_linear(X, up["lam"], up["packed"], up["sw"][None], up["L1"][None] if r1 else None,
                                    up["L2"][None] if r1 else None, up["bias"][None], N=H, y_dtype="f32",
                                    kernel="tiled")
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else rows
    yhn = yh.cpu().numpy()[rows]
    assert np.array_equal(yhn.view(np.uint32), plain[0].cpu().numpy()[rows].view(np.uint32))
    q, s16, Uo = chain.hidden(yhn, dn_lay["lam"], dn_lay["L1"][0], act)
    assert np.array_equal(codes[rows], q)
    assert np.array_equal(scales[rows], s16)
    if r2:
        eu = rel(U[rows].astype(np.float64), Uo)
        assert eu <= 1e-5
    ref = chain.down_output(q, s16, Uo, dn_lay["qw"][0], dn_lay["sw"][0], dn_lay["L2"][0], dn_lay["bias"][0])
    e32 = rel(Y32.cpu().numpy()[rows].astype(np.float64), ref)
    ref_b = bf16_bits_to_f32(f64_to_bf16_bits(ref)).astype(np.float64)
    e16 = rel(Yb.cpu().numpy()[rows].astype(np.float64), ref_b)
    say(f"    codes/scales exact; Y fp32 rel {e32:.3e}, bf16 rel {e16:.3e}")
    assert e32 <= TOL and e16 <= TOL


@pytest.mark.parametrize("M,K,H,N,act", [
    (200, 256, 320, 200, "gelu_tanh"),   # H = 5 groups: a pad group in the last 128-column block
    (200, 256, 320, 200, "identity"),
    (40, 192, 256, 136, "gelu_tanh"),    # 40 tokens: the down layer on the skinny contraction
    (130, 512, 384, 72, "gelu_tanh"),    # ragged rows past a 128-row tile
])
def test_chain_matches_oracle(M, K, H, N, act):
    up = make_random_layer(500 + M, M, K, H, r=4, outlier_channels=2)
    dn = make_random_layer(600 + M, M, H, N, r=4, outlier_channels=0)
    run_case(up, dn, act)


@pytest.mark.parametrize("M,K,H,N,r1,r2", [
    (200, 256, 320, 200, 4, 0),      # rank-0 down layer: no U shares, no U reduction
    (130, 512, 384, 72, 0, 4),       # rank-0 up layer
    (40, 192, 256, 136, 0, 0),       # both rank 0, the down layer on the skinny contraction
])
def test_chain_rank_zero_layers(M, K, H, N, r1, r2):
    up = make_random_layer(700 + M + r1, M, K, H, r=r1, outlier_channels=2)
    dn = make_random_layer(800 + M + r2, M, H, N, r=r2, outlier_channels=0)
    run_case(up, dn, "gelu_tanh")


def test_chain_flux_mlp_sampled_rows():
    up = make_layer("flux_up")
    dn = make_layer("flux_down")
    rows = np.array(sorted(set([0, 1, 4095, 4096, 4607]) |
                           set(np.random.default_rng(3).choice(4608, 19, replace=False).tolist())))
    run_case(up, dn, "gelu_tanh", rows)
