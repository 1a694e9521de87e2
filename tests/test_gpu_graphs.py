"""HIP-graph replay of the format variants, the fused chain and the
calibration kernels: each call is captured once and replayed several times,
with eager calls of the same operation on other buffers in between; every
replay must equal the eager result bit for bit (the kernels are
deterministic, and none of these paths records a memset into the graph).
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


def say(msg):
    print(msg, flush=True)


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(DEV)


def replay_matches(run, out, eager_again):
    """Capture run() (which writes `out`), replay it three times with an
    eager call in between, compare every replay with the eager bits."""
    run()
    torch.cuda.synchronize()
    ref = out.view(torch.int32).cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            run()
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int32).cpu().numpy(), ref), f"replay {rep}"
        eager_again()
        torch.cuda.synchronize()


def test_graph_asymmetric_linear():
    lay = make_random_layer(71, 200, 1024, 300, r=4, outlier_channels=2)
    say("[graph] asymmetric linear M=200 K=1024 N=300")
    X, lam = dev16(lay["X"]), dev16(lay["lam"])
    packed, st = hsq.pack_weights(dev8(lay["qw"][0]))
    sw, L1, L2, b = dev16(lay["sw"][:1]), dev16(lay["L1"][:1]), dev16(lay["L2"][:1]), dev16(lay["bias"][:1])
    out = torch.empty((1, 200, 300), dtype=torch.float32, device=DEV)
    ws = torch.empty(hsq.workspace_bytes(200, 1024, 300, 4, 1), dtype=torch.uint8, device=DEV)
    run = lambda: hsq.w4a4_lowrank_linear(X, lam, packed, sw, L1, L2, b, N=300, y_dtype="f32", out=out,
                                          workspace=ws, act_quant="asym")
    X2 = dev16(make_random_layer(72, 200, 1024, 300, r=4)["X"])
    other = lambda: hsq.w4a4_lowrank_linear(X2, lam, packed, sw, L1, L2, b, N=300, y_dtype="f32",
                                            act_quant="asym")
    replay_matches(run, out, other)


def test_graph_mx_linear():
    lay = make_random_layer(73, 200, 1024, 300, r=4, outlier_channels=2)
    say("[graph] MX-fp4 linear M=200 K=1024 N=300")
    swf = lay["sw"][0].view(np.float16).astype(np.float32)
    R = (lay["qw"][0].astype(np.float32) * np.repeat(swf, 64, axis=0)).astype(np.float32)
    packed = hsq.mx_pack_weights(torch.from_numpy(R).to(DEV))
    X, lam = dev16(lay["X"]), dev16(lay["lam"])
    L1, L2, b = dev16(lay["L1"][0]), dev16(lay["L2"][0]), dev16(lay["bias"][0])
    out = torch.empty((200, 300), dtype=torch.float32, device=DEV)
    ws = torch.empty(hsq._load().hsq_mx_workspace_bytes(200, 1024, 4), dtype=torch.uint8, device=DEV)
    run = lambda: hsq.mx_lowrank_linear(X, lam, packed, L1, L2, b, N=300, y_dtype="f32", out=out, workspace=ws)
    X2 = dev16(make_random_layer(74, 200, 1024, 300, r=4)["X"])
    other = lambda: hsq.mx_lowrank_linear(X2, lam, packed, L1, L2, b, N=300, y_dtype="f32")
    replay_matches(run, out, other)


def test_graph_fused_chain():
    up = make_random_layer(75, 130, 512, 384, r=4, outlier_channels=2)
    dn = make_random_layer(76, 130, 384, 72, r=4)
    say("[graph] fused chain M=130 K=512 H=384 N=72")

    def upload(lay):
        packed, st = hsq.pack_weights(dev8(lay["qw"][0]))
        return dict(lam=dev16(lay["lam"]), packed=packed, sw=dev16(lay["sw"][0]), L1=dev16(lay["L1"][0]),
                    L2=dev16(lay["L2"][0]), bias=dev16(lay["bias"][0]))
    u, d = upload(up), upload(dn)
    X = dev16(up["X"])
    out = torch.empty((130, 72), dtype=torch.float32, device=DEV)
    ws = torch.empty(hsq.mlp_workspace_bytes(130, 512, 384, 72, 4, 4), dtype=torch.uint8, device=DEV)
    run = lambda: hsq.w4a4_lowrank_mlp(X, u, d, H=384, N=72, act="gelu_tanh", y_dtype="f32", out=out, workspace=ws)
    X2 = dev16(make_random_layer(77, 130, 512, 384, r=4)["X"])
    other = lambda: hsq.w4a4_lowrank_mlp(X2, u, d, H=384, N=72, act="gelu_tanh", y_dtype="f32")
    replay_matches(run, out, other)


@pytest.mark.parametrize("M,K", [(512, 1152), (300, 4096)])   # token splits; whole blocks
def test_graph_hessian(M, K):
    lay = make_random_layer(78, M, K, 64, r=4)
    say(f"[graph] Hessian M={M} K={K}")
    X, lam = dev16(lay["X"]), dev16(lay["lam"])
    H = torch.empty((K, K), dtype=torch.float32, device=DEV)
    nws = hsq._load().hsq_hessian_workspace_bytes(M, K)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
    run = lambda: hsq.hessian_accumulate(X, lam, H=H, workspace=ws)
    X2 = dev16(make_random_layer(79, M, K, 64, r=4)["X"])
    other = lambda: hsq.hessian_accumulate(X2, lam)
    replay_matches(run, H, other)


def test_graph_pack_weights():
    # the pack call (status clear + pack kernel) captured and replayed: the
    # packed bytes and the status word equal the eager call's on every
    # replay; a replay over codes that were made out of range in between
    # sets the status, and the next clean replay clears it again
    rng = np.random.default_rng(5)
    K, N = 1152, 300
    codes = dev8(rng.integers(-8, 8, (K, N), dtype=np.int8))
    packed = torch.empty(hsq.packed_weight_bytes(K, N), dtype=torch.uint8, device=DEV)
    status = torch.empty(4, dtype=torch.int32, device=DEV)
    ref_packed, ref_status = hsq.pack_weights(codes)
    torch.cuda.synchronize()
    ref = ref_packed.cpu().numpy().copy()
    assert int(ref_status[0].item()) == 0
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            hsq.pack_weights(codes, packed=packed, status=status)
    torch.cuda.synchronize()
    say(f"[graph] pack K={K} N={N}")
    for rep in range(3):
        packed.fill_(0xEE)
        status.fill_(7)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(packed.cpu().numpy(), ref), f"replay {rep}"
        assert int(status[0].item()) == 0, f"replay {rep}"
        hsq.pack_weights(codes)                 # eager work in between
        torch.cuda.synchronize()
    saved = codes[17, 5].item()
    codes[17, 5] = 9                            # out of range: flagged
    g.replay()
    torch.cuda.synchronize()
    assert int(status[0].item()) == 1
    codes[17, 5] = saved
    g.replay()
    torch.cuda.synchronize()
    assert int(status[0].item()) == 0
    assert np.array_equal(packed.cpu().numpy(), ref)
