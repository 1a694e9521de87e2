"""hsq_w4a4_lowrank_linear_noalloc (the layer with its workspace in the
library's static per-device scratch) against hsq_w4a4_lowrank_linear (the
same kernels on a caller-provided workspace), through the C ABI.

The two share their kernels and the workspace layout, so the bar is bit
for bit on the fp32 and bf16 outputs.  Two calls in a row, the second with
a smaller input, check that nothing of the first call's scratch contents
leaks into the second; a size beyond the scratch is rejected before any
launch.
"""

import ctypes

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


def upload(lay):
    B = lay["qw"].shape[0]
    r = lay["L1"].shape[2]
    packed = torch.cat([hsq.pack_weights(torch.from_numpy(lay["qw"][b]).to(DEV))[0] for b in range(B)])
    return dict(X=dev16(lay["X"]), lam=dev16(lay["lam"]), packed=packed, sw=dev16(lay["sw"]),
                L1=dev16(lay["L1"]) if r else None, L2=dev16(lay["L2"]) if r else None,
                bias=dev16(lay["bias"]), B=B, r=r, M=lay["X"].shape[0], K=lay["X"].shape[1],
                N=lay["qw"].shape[2])


def both(u, y_dtype):
    """(noalloc output, workspace-path output) as raw bits."""
    lib = hsq._load()
    P = hsq._ptr
    tdt = torch.float32 if y_dtype == "f32" else torch.bfloat16
    code = hsq.F32 if y_dtype == "f32" else hsq.BF16
    outs = []
    for which in ("noalloc", "plain"):
        out = torch.full((u["B"], u["M"], u["N"]), float("nan"), dtype=tdt, device=DEV)
        args = (P(u["X"]), u["M"], u["K"], u["N"], u["B"], P(u["lam"]), P(u["packed"]), P(u["sw"]),
                P(u["L1"]), P(u["L2"]), u["r"], P(u["bias"]), P(out), code)
        if which == "noalloc":
            st = lib.hsq_w4a4_lowrank_linear_noalloc(*args, hsq._stream())
        else:
            ws = torch.empty(hsq.workspace_bytes(u["M"], u["K"], u["N"], u["r"], u["B"]), dtype=torch.uint8,
                             device=DEV)
            st = lib.hsq_w4a4_lowrank_linear(*args, P(ws), ws.numel(), hsq._stream())
        assert st == hsq.OK, (which, st)
        torch.cuda.synchronize()
        view = torch.int32 if y_dtype == "f32" else torch.int16
        outs.append(out.view(view).cpu().numpy())
    return outs


@pytest.mark.parametrize("y_dtype", ["f32", "bf16"])
def test_noalloc_matches_workspace_entry_two_calls(y_dtype):
    # first call: tiled contraction, two projections, ragged M and N; second
    # call: fewer tokens (the skinny contraction) and a shorter K, so the
    # scratch holds the first call's larger contents when it starts
    big = upload(make_random_layer(4101, 300, 1152, 520, r=4, batch=2, outlier_channels=2))
    small = upload(make_random_layer(4102, 40, 512, 200, r=4, batch=1, outlier_channels=2))
    for name, u in (("big", big), ("small", small)):
        say(f"[noalloc] {name} M={u['M']} K={u['K']} N={u['N']} batch={u['B']} {y_dtype}")
        a, b = both(u, y_dtype)
        assert np.array_equal(a, b), name


def test_noalloc_third_call_long_k_with_splits():
    # a shape whose tiled contraction splits K (partial tiles in the scratch)
    u = upload(make_random_layer(4103, 200, 4096, 300, r=4, batch=1, outlier_channels=2))
    say(f"[noalloc] split-K M={u['M']} K={u['K']} N={u['N']}")
    a, b = both(u, "f32")
    assert np.array_equal(a, b)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    lib = hsq._load()
    A = ctypes.c_void_p(0x100000)
    M, K, N = 32767, 4096, 16            # codes alone: 2048 x 64 KiB = 128 MiB
    assert hsq.workspace_bytes(M, K, N, 4, 1) > hsq.NOALLOC_SCRATCH_BYTES
    st = lib.hsq_w4a4_lowrank_linear_noalloc(A, M, K, N, 1, A, A, A, A, A, 4, A, A, hsq.BF16, None)
    assert st == hsq.E_SCRATCH
