"""Calibration kernels (Hessian, deflation, closed-form L2) vs the CPU oracle,
through the C ABI, on seeded inputs.

Each stage is checked against the oracle's definition applied in float64 to
the inputs that stage received (the previous stage's GPU output), with an
elementwise bound derived from the stage's floating-point arithmetic
(u = 2^-24, gamma_n = n u / (1 - n u), the textbook bound on an n-term fp32
sum whatever its order):
  * H (bf16 products, exact in fp32, summed over M tokens, then two
    roundings by the smoothing factors) vs Xh^T Xh with Xh rounded to fp32
    as the inference path rounds it:
        |dH| <= gamma_{M+4} (|Xh|^T |Xh|)
  * H L1 (fp32, K terms):             |d HL1| <= gamma_{K+1} (|H| |L1|)
  * C^-1 (fp64 from fp32 H L1):       |Cinv C - I| <= 16 (K + r) 2^-53 cond(C)
  * Hperp = H - (HL1 C^-1) HL1^T (B rounded to fp32, r FMAs):
        |dHperp| <= gamma_{r+2} (|H| + |B| |HL1|^T)
  * L2 = C^-1 sum_slices T, T in fp32 over at most K channels of
    E = W - code * sw (one rounding):
        |dL2| <= |C^-1| gamma_{K+2} (|HL1|^T |E|)
End to end, the pages' properties: Hperp L1 ~ 0 (Figure 1 caption), and the
GPU's L2 attains the least-squares minimum of ||Xh E - Xh L1 L2||^2: its
excess over the minimum, tr(dL2^T C dL2) with dL2 = L2 - L2* (exact for a
quadratic), stays below 1e-8 of the low-rank branch's own output energy
tr(L2*^T C L2*) (abstract: the output-side factor is eliminated in closed
form; the fp32 Hessian alone perturbs L2 by about cond(C) * 1e-7).
"""

import functools

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import w4a4_rank_assisted_amd as hsq  # noqa: E402
from oracle import calibration as cal  # noqa: E402
from synth import make_full_weight, make_layer, make_random_layer  # noqa: E402

DEV = torch.device("cuda:0")
U = 2.0 ** -24


def gamma(n):
    return n * U / (1 - n * U)


def say(msg):
    print(msg, flush=True)


def dev16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int8)).to(DEV)


@functools.lru_cache(maxsize=3)
def case(name, M=None, K=None, N=None, r=4, group=64):
    if name == "random":
        lay = make_random_layer(61 + r + M, M, K, N, r=r, outlier_channels=3, group=group)
    else:
        lay = make_layer(name, M)
    say(f"[calib case] {name} M={lay['X'].shape[0]} K={lay['qw'].shape[1]} N={lay['qw'].shape[2]} "
        f"r={lay['L1'].shape[2]} group={lay['group']}")
    return lay


def run_hessian(lay, accumulate_onto=None):
    X, lam = dev16(lay["X"]), dev16(lay["lam"])
    H = None if accumulate_onto is None else accumulate_onto.clone()
    H = hsq.hessian_accumulate(X, lam, H, accumulate=accumulate_onto is not None)
    torch.cuda.synchronize()
    return H


def check_hessian(lay, Hg):
    M = lay["X"].shape[0]
    H = cal.hessian(lay["X"], lay["lam"])
    A = cal.hessian_abs(lay["X"], lay["lam"])
    err = np.abs(Hg.cpu().numpy().astype(np.float64) - H)
    bound = gamma(M + 4) * A
    worst = float((err / np.maximum(bound, 1e-300)).max())
    rel = float(np.linalg.norm(err) / np.linalg.norm(H))
    say(f"    H: rel Frobenius {rel:.2e}, worst err / bound {worst:.2e}")
    assert np.all(err <= bound)
    assert rel <= 1e-5
    return H


@pytest.mark.parametrize("name,M,K,N,r", [
    ("random", 300, 384, 200, 4),      # ragged tokens, one token split
    ("random", 1000, 320, 200, 4),     # K not a multiple of the 128-block, token splits
    ("pixart_up", None, None, None, 4),   # 45 blocks: 12 token splits
    ("qwen3_up", 2048, None, None, 4),    # 528 blocks, no split
])
def test_hessian_matches_oracle(name, M, K, N, r):
    lay = case(name, M, K, N, r)
    check_hessian(lay, run_hessian(lay))


def test_hessian_accumulates():
    a = make_random_layer(71, 200, 256, 64, r=4)
    b = make_random_layer(72, 333, 256, 64, r=4)
    b["lam"] = a["lam"]
    Ha = run_hessian(a)
    Hab = run_hessian(b, accumulate_onto=Ha).cpu().numpy().astype(np.float64)
    ref = cal.hessian(a["X"], a["lam"]) + cal.hessian(b["X"], b["lam"])
    A = cal.hessian_abs(a["X"], a["lam"]) + cal.hessian_abs(b["X"], b["lam"])
    assert np.all(np.abs(Hab - ref) <= gamma(200 + 333 + 8) * A)
    # the symmetric halves agree bit for bit (one block writes both)
    assert np.array_equal(Hab, Hab.T)


def run_deflate(Hg, L1_bits):
    Hp, HL1, Cinv = hsq.deflate_hessian(Hg, dev16(L1_bits))
    torch.cuda.synchronize()
    return (Hp.cpu().numpy().astype(np.float64), HL1.cpu().numpy().astype(np.float64),
            Cinv.cpu().numpy())


def check_deflate(Hg, L1_bits):
    H = Hg.cpu().numpy().astype(np.float64)
    L1 = cal.bf16_matrix(L1_bits)
    K, r = L1.shape
    Hp, HL1, Cinv = run_deflate(Hg, L1_bits)
    # stage 1: H L1
    ref = H @ L1
    assert np.all(np.abs(HL1 - ref) <= gamma(K + 1) * (np.abs(H) @ np.abs(L1)))
    # stage 2: C^-1 of C = L1^T (H L1) formed from the GPU's H L1
    C = L1.T @ HL1
    assert np.abs(Cinv @ C - np.eye(r)).max() <= 16 * (K + r) * 2.0 ** -53 * np.linalg.cond(C)
    # stage 3: the rank-r update
    B = (HL1 @ Cinv).astype(np.float32).astype(np.float64)
    ref_p = H - B @ HL1.T
    bound = gamma(r + 2) * (np.abs(H) + np.abs(B) @ np.abs(HL1).T)
    worst = float((np.abs(Hp - ref_p) / np.maximum(bound, 1e-300)).max())
    assert np.all(np.abs(Hp - ref_p) <= bound)
    # the pages' property: the protected subspace is annihilated (to fp32
    # rounding of the whole chain)
    ann = np.linalg.norm(Hp @ L1) / (np.linalg.norm(H) * np.linalg.norm(L1))
    say(f"    deflation: worst err / bound {worst:.2e}; |Hperp L1| / (|H| |L1|) = {ann:.2e}")
    assert ann <= 64 * gamma(K) * np.linalg.cond(C)
    return Hp, HL1, Cinv


@pytest.mark.parametrize("name,M,K,N,r", [
    ("random", 300, 384, 200, 4),
    ("random", 300, 384, 200, 7),     # odd rank (rank template 8)
    ("random", 600, 512, 200, 32),    # largest rank
    ("pixart_up", None, None, None, 4),
])
def test_deflation_stages_and_annihilation(name, M, K, N, r):
    lay = case(name, M, K, N, r)
    check_deflate(run_hessian(lay), lay["L1"][0])


def test_deflation_in_place():
    lay = case("random", 300, 384, 200, 4)
    Hg = run_hessian(lay)
    Hp, HL1, Cinv = hsq.deflate_hessian(Hg.clone(), dev16(lay["L1"][0]))
    Hq = Hg.clone()
    Hq2, HL1b, Cinvb = hsq.deflate_hessian(Hq, dev16(lay["L1"][0]), Hperp=Hq)
    torch.cuda.synchronize()
    assert torch.equal(Hq2, Hp) and torch.equal(HL1b, HL1) and torch.equal(Cinvb, Cinv)


def run_l2(lay, HL1, Cinv, W_bits):
    K, N = W_bits.shape
    packed, st = hsq.pack_weights(dev8(lay["qw"][0]))
    assert int(st[0].item()) == 0
    L2 = hsq.closed_form_l2(torch.from_numpy(HL1.astype(np.float32)).to(DEV),
                            torch.from_numpy(Cinv).to(DEV), dev16(W_bits), packed,
                            dev16(lay["sw"][0]), group=lay["group"])
    torch.cuda.synchronize()
    return L2.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name,M,K,N,r,group", [
    ("random", 300, 384, 200, 4, 64),
    ("random", 300, 384, 200, 7, 64),
    ("random", 300, 384, 200, 4, 128),   # group-128 residual scales
    ("random", 600, 512, 200, 32, 64),
    ("pixart_up", None, None, None, 4, 64),
    ("qwen3_up", 2048, None, None, 4, 64),
])
def test_closed_form_l2_stage_and_optimality(name, M, K, N, r, group):
    lay = case(name, M, K, N, r, group)
    Hg = run_hessian(lay)
    Hp, HL1, Cinv = run_deflate(Hg, lay["L1"][0])
    W = make_full_weight(lay, 0)
    E = cal.residual_error(W, lay["qw"][0], lay["sw"][0], lay["group"])
    L2g = run_l2(lay, HL1, Cinv, W)
    K = W.shape[0]
    # the stage: from the GPU's HL1 and Cinv
    ref = Cinv @ (HL1.T @ E)
    bound = np.abs(Cinv) @ (gamma(K + 2) * (np.abs(HL1).T @ np.abs(E)))
    worst = float((np.abs(L2g - ref) / np.maximum(bound, 1e-300)).max())
    assert np.all(np.abs(L2g - ref) <= bound)
    # end to end: the GPU's L2 attains the least-squares minimum
    L1 = cal.bf16_matrix(lay["L1"][0])
    H = cal.hessian(lay["X"], lay["lam"])
    C = L1.T @ H @ L1
    L2s = cal.closed_form_l2(H, L1, E)
    d = L2g - L2s
    excess = float(np.einsum("an,ab,bn->", d, C, d))
    energy = float(np.einsum("an,ab,bn->", L2s, C, L2s))
    say(f"    L2: worst err / bound {worst:.2e}; excess / branch energy {excess / energy:.2e}")
    assert excess <= 1e-8 * energy
