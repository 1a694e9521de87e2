"""Asymmetric activations (hsq_w4a4_*_aq with HSQ_AQ_ASYMMETRIC) vs the CPU
oracle (oracle/asym.py), through the C ABI, on seeded inputs.

Bars: the stored codes q - z and the fp16 scales (decoded from the
workspace the quantize stage wrote) and the int32 partial sums P: bit-exact;
Y fp32 within 1e-3 relative Frobenius of the oracle's fp64 output, bf16
within 1e-3 of that output rounded to bf16.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a4_rank_assisted_amd as hsq  # noqa: E402
from oracle import asym  # noqa: E402
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


class Layer:
    def __init__(self, lay):
        self.lay = lay
        self.group = int(lay.get("group", 64))
        self.B, self.K, self.N = lay["qw"].shape
        self.M = lay["X"].shape[0]
        self.r = lay["L1"].shape[2]
        self.X, self.lam = dev16(lay["X"]), dev16(lay["lam"])
        packed, st = hsq.pack_weights(dev8(lay["qw"][0]))
        assert int(st[0].item()) == 0
        self.packed = packed
        self.sw = dev16(lay["sw"][:1])
        self.L1 = dev16(lay["L1"][:1]) if self.r else None
        self.L2 = dev16(lay["L2"][:1]) if self.r else None
        self.bias = dev16(lay["bias"][:1])

    def codes_scales(self):
        """Codes and scales from the workspace: MT x Gp blocks of 1 KiB (lane
        slot l = row l%16, channels 16*(l/16) .. +15), then MT x SG x 16 fp16."""
        ws = torch.empty(hsq.workspace_bytes(self.M, self.K, self.N, self.r, 1, self.group),
                         dtype=torch.uint8, device=DEV)
        hsq.quantize_stage(self.X, self.lam, self.L1, N=self.N, batch=1, workspace=ws, group=self.group,
                           act_quant="asym")
        torch.cuda.synchronize()
        MT, Gp = -(-self.M // 16), -(-self.K // 64 // 2) * 2
        SG = self.K // self.group if self.group == 128 else Gp
        raw = ws.cpu().numpy()
        qa = raw[: MT * Gp * 1024].view(np.int8).reshape(MT, Gp, 4, 16, 16)
        codes = qa.transpose(0, 3, 1, 2, 4).reshape(MT * 16, Gp * 64)[: self.M, : self.K]
        off = -(-(MT * Gp * 1024) // 256) * 256
        sx = raw[off: off + MT * SG * 16 * 2].view(np.uint16).reshape(MT, SG, 16)
        return codes, sx.transpose(0, 2, 1).reshape(MT * 16, SG)[: self.M, : self.K // self.group]

    def partials(self, m0, mc, n0, nc, kernel):
        P = hsq.w4a4_group_partials(self.X, self.lam, self.packed, self.N, m0, mc, n0, nc, kernel=kernel,
                                    group=self.group, act_quant="asym")
        torch.cuda.synchronize()
        return P.cpu().numpy()

    def linear(self, y_dtype, kernel):
        Y = hsq.w4a4_lowrank_linear(self.X, self.lam, self.packed, self.sw, self.L1, self.L2, self.bias,
                                    N=self.N, y_dtype=y_dtype, kernel=kernel, group=self.group,
                                    act_quant="asym")
        torch.cuda.synchronize()
        return Y[0]


def check_codes(up):
    codes, scales = up.codes_scales()
    q, z, s16 = asym.quantize(asym.smoothed(up.lay["X"], up.lay["lam"]), up.group)
    assert np.array_equal(scales, s16)
    assert np.array_equal(codes, asym.stored_codes(q, z, up.group))
    return q, z


def check_partials(up, m0, mc, n0, nc, kernel):
    got = up.partials(m0, mc, n0, nc, kernel)
    ref = asym.partials(up.lay["X"], up.lay["lam"], up.lay["qw"][0], up.group, rows=np.arange(m0, m0 + mc))
    assert np.array_equal(got.astype(np.int64), ref[:, n0:n0 + nc, :])


def check_linear(up, rows, kernel):
    lay = up.lay
    ref = asym.linear(lay["X"], lay["lam"], lay["qw"][0], lay["sw"][0], lay["L1"][0] if up.r else None,
                      lay["L2"][0] if up.r else None, lay["bias"][0], group=up.group, rows=rows)
    Y32 = up.linear("f32", kernel).cpu().numpy()[rows].astype(np.float64)
    Yb = up.linear("bf16", kernel).float().cpu().numpy()[rows].astype(np.float64)
    e32 = rel(Y32, ref)
    e16 = rel(Yb, bf16_bits_to_f32(f64_to_bf16_bits(ref)).astype(np.float64))
    say(f"    {kernel}: fp32 rel {e32:.3e}  bf16 rel {e16:.3e}")
    assert e32 <= TOL and e16 <= TOL


@pytest.mark.parametrize("M,K,N,r,group", [
    (5, 256, 33, 0, 64),        # rank 0, ragged N, one row tile
    (40, 640, 300, 4, 64),      # the skinny kernel's range; five groups (a pad group)
    (130, 1024, 130, 7, 64),    # ragged rows and columns past a 128 tile, odd rank
    (70, 2304, 200, 4, 128),    # group 128, K split
])
def test_asym_ragged_shapes_match_oracle(M, K, N, r, group):
    up = Layer(make_random_layer(800 + M, M, K, N, r=r, outlier_channels=3, group=group))
    say(f"[asym] M={M} K={K} N={N} r={r} group={group}")
    check_codes(up)
    kernels = ("tiled", "skinny") if M <= 64 else ("tiled",)
    for kernel in kernels:
        check_partials(up, 0, M, 0, N, kernel)
        check_linear(up, np.arange(M), kernel)


def test_asym_edge_groups():
    M, K, N = 48, 512, 64
    lay = make_random_layer(81, M, K, N, r=4)
    x = bf16_bits_to_f32(lay["X"]).astype(np.float64)
    x[3, :] = 0.0                         # a zero token
    x[7, 64:128] = 0.0                    # one zero group
    x[9, 128:192] = np.abs(x[9, 128:192])   # all positive: zero point 0
    x[10, 128:192] = -np.abs(x[10, 128:192])  # all negative: zero point 15
    x[11, 256:320] *= 2.0 ** -40          # scale underflows to zero
    x[13, 0:64] *= 1.0e6                  # scale saturates at 65504
    x[15, 320:384] = 0.75                 # a constant group
    lay["X"] = f64_to_bf16_bits(x)
    up = Layer(lay)
    q, z = check_codes(up)
    assert z[9, 2] == 0 and z[10, 2] == 15
    for kernel in ("tiled", "skinny"):
        check_partials(up, 0, M, 0, N, kernel)
        check_linear(up, np.arange(M), kernel)


@pytest.mark.parametrize("name,M,group", [("pixart_up", None, 64), ("qwen3_up", 16, 64),
                                          ("qwen3_up", 2048, 128)])
def test_asym_full_size(name, M, group):
    up = Layer(make_layer(name, M, group))
    say(f"[asym full] {name} M={up.M} K={up.K} N={up.N} group={group}")
    check_codes(up)
    kernel = "skinny" if up.M <= 64 else "tiled"
    check_partials(up, max(up.M - 40, 0), min(up.M, 40), up.N - 96, 96, kernel)
    rows = np.array(sorted(set([0, up.M - 1]) | set(np.random.default_rng(2).choice(up.M, min(up.M, 24),
                                                                                      replace=False).tolist())))
    check_linear(up, rows, kernel)
