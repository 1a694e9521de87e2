"""The C ABI on the host: the library loads, exports every function
include/hsq.h declares, sizes its buffers, and rejects bad arguments before
it enqueues anything (no GPU needed: no call here reaches a launch)."""

import ctypes
import re
import subprocess

import pytest

import w4a4_rank_assisted_amd as hsq

lib = hsq._load()
A = 0x100000  # a 16-byte aligned fake device address: validation rejects before use
P = ctypes.c_void_p


def test_every_declared_function_is_exported():
    names = hsq.header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", hsq.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (hsq_\w+)", out))
    assert set(names) <= exported


def test_constants_match_header():
    text = open(hsq.HEADER).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"#define (HSQ_\w+)\s+(-?\d+)", text))
    assert consts["HSQ_OK"] == hsq.OK and consts["HSQ_E_INVAL"] == hsq.E_INVAL
    assert consts["HSQ_E_SHAPE"] == hsq.E_SHAPE and consts["HSQ_E_ALIGN"] == hsq.E_ALIGN
    assert consts["HSQ_E_WORKSPACE"] == hsq.E_WORKSPACE and consts["HSQ_E_HIP"] == hsq.E_HIP
    assert consts["HSQ_F32"] == hsq.F32 and consts["HSQ_BF16"] == hsq.BF16
    assert consts["HSQ_KERNEL_TILED"] == hsq.KERNEL_TILED
    assert consts["HSQ_KERNEL_SKINNY"] == hsq.KERNEL_SKINNY


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(lib.hsq_status_string(s), bytes)
    assert lib.hsq_layout_version() == 2


# layout version 2: nibbles (column tiles x group pairs x 1 KiB), then the
# int8 operands (column tiles x padded groups x 1 KiB)
@pytest.mark.parametrize("K,N,expect", [
    (64, 16, 1024 + 2 * 1024),            # one 16-column tile, one (padded) group pair
    (128, 16, 1024 + 2 * 1024),
    (192, 17, 2 * 2 * 1024 + 2 * 4 * 1024),   # 2 column tiles x 2 group pairs
    (1152, 4608, 288 * 9 * 1024 + 288 * 18 * 1024),
    (2240, 2240, 140 * 18 * 1024 + 140 * 36 * 1024),  # 35 groups pad to 36
    (63, 16, 0), (0, 16, 0), (64, 0, 0),
])
def test_packed_weight_bytes(K, N, expect):
    assert lib.hsq_packed_weight_bytes(K, N) == expect


def test_workspace_bytes_cover_the_internal_buffers():
    M, K, N, r, b = 4096, 1152, 4608, 4, 1
    ws = lib.hsq_workspace_bytes(M, K, N, r, b)
    codes = (M // 16) * 18 * 1024            # tiled int8 codes, 18 groups
    scales = (M // 16) * 18 * 16 * 2       # fp16 activation scales
    assert ws >= codes + scales + M * r * 4
    assert ws < 2 * (codes + scales) + 16 * M * r * 4
    assert lib.hsq_workspace_bytes(0, K, N, r, b) == 0
    assert lib.hsq_workspace_bytes(M, 100, N, r, b) == 0
    assert lib.hsq_workspace_bytes(M, K, N, 33, b) == 0
    assert lib.hsq_workspace_bytes(M, K, N, r, 0) == 0
    # M = 1 still needs one row tile
    assert lib.hsq_workspace_bytes(1, 64, 16, 0, 1) >= 2 * 1024


def test_workspace_holds_split_k_partials():
    # few output tiles against a long K: the tiled contraction splits K and
    # keeps fp32 partial tiles (128 x 128 per split) in the workspace
    M, K, N = 256, 12288, 4096                # 2 x 32 tiles, 4 splits (of two K halves each)
    codes = (M // 16) * 192 * 1024
    pairs = (192 + 2) * N * 8                 # weight-scale pairs of the tiled contraction
    ws = lib.hsq_workspace_bytes(M, K, N, 4, 1)
    assert ws >= codes + 4 * 2 * 32 * 128 * 128 * 4 + pairs
    assert ws < codes + 5 * 2 * 32 * 128 * 128 * 4 + pairs
    # enough tiles: no partials
    assert lib.hsq_workspace_bytes(4096, 1152, 4608, 4, 1) < 32 << 20


def _linear(**kw):
    a = dict(X=A, M=64, K=256, N=256, batch=1, lam=A, w=A, sw=A, L1=A, L2=A, r=4, bias=A, Y=A,
             ydt=hsq.BF16, ws=A, wsb=1 << 30, kernel=0, stream=None)
    a.update(kw)
    return lib.hsq_w4a4_lowrank_linear_ex(
        a["X"], a["M"], a["K"], a["N"], a["batch"], a["lam"], a["w"], a["sw"], a["L1"], a["L2"],
        a["r"], a["bias"], a["Y"], a["ydt"], a["ws"], a["wsb"], a["kernel"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(X=None), hsq.E_INVAL),
    (dict(lam=None), hsq.E_INVAL),
    (dict(w=None), hsq.E_INVAL),
    (dict(sw=None), hsq.E_INVAL),
    (dict(Y=None), hsq.E_INVAL),
    (dict(ws=None), hsq.E_INVAL),
    (dict(L1=None), hsq.E_INVAL),
    (dict(L2=None), hsq.E_INVAL),
    (dict(M=0), hsq.E_INVAL),
    (dict(N=0), hsq.E_INVAL),
    (dict(K=100), hsq.E_SHAPE),
    (dict(K=0), hsq.E_INVAL),
    (dict(r=33), hsq.E_INVAL),
    (dict(r=-1), hsq.E_INVAL),
    (dict(batch=0), hsq.E_INVAL),
    (dict(batch=17), hsq.E_INVAL),
    (dict(ydt=2), hsq.E_INVAL),
    (dict(kernel=3), hsq.E_INVAL),
    (dict(kernel=hsq.KERNEL_SKINNY, M=65), hsq.E_INVAL),
    (dict(X=A + 2), hsq.E_ALIGN),
    (dict(w=A + 8), hsq.E_ALIGN),
    (dict(Y=A + 4), hsq.E_ALIGN),
    (dict(ws=A + 1), hsq.E_ALIGN),
    (dict(wsb=0), hsq.E_WORKSPACE),
    (dict(wsb=1000), hsq.E_WORKSPACE),
    (dict(M=1 << 20, K=1 << 12), hsq.E_INVAL),  # M*K >= 2^31
    # M*K < 2^31, but the int8 codes padded to 16 rows reach 2^32 bytes,
    # past what the contraction's 32-bit buffer resources address
    (dict(M=1, K=1 << 28, N=1), hsq.E_INVAL),
    (dict(M=3, K=(1 << 28) - 64, N=1), hsq.E_INVAL),
    # the largest token count the GPU limit tests run passes the size checks
    (dict(M=32767, K=65536, N=16, wsb=0), hsq.E_WORKSPACE),
])
def test_linear_rejects_before_launch(kw, code):
    assert _linear(**kw) == code


def test_linear_rank_zero_needs_no_factors():
    # r = 0 with null L1/L2 passes argument checks and stops at the workspace
    assert _linear(r=0, L1=None, L2=None, wsb=0) == hsq.E_WORKSPACE


def test_plain_linear_entry_validates_too():
    assert lib.hsq_w4a4_lowrank_linear(None, 64, 256, 256, 1, A, A, A, A, A, 4, A, A, 1, A,
                                       1 << 30, None) == hsq.E_INVAL


def test_partials_rejects_bad_windows():
    f = lib.hsq_w4a4_group_partials
    assert f(A, 64, 256, 256, A, A, 0, 64, 0, 256, None, A, 1 << 30, 0, None) == hsq.E_INVAL
    assert f(A, 64, 256, 256, A, A, 0, 65, 0, 256, A, A, 1 << 30, 0, None) == hsq.E_SHAPE
    assert f(A, 64, 256, 256, A, A, -1, 4, 0, 256, A, A, 1 << 30, 0, None) == hsq.E_SHAPE
    assert f(A, 64, 256, 256, A, A, 0, 4, 250, 7, A, A, 1 << 30, 0, None) == hsq.E_SHAPE
    assert f(A, 64, 256, 256, A, A, 0, 0, 0, 4, A, A, 1 << 30, 0, None) == hsq.E_SHAPE
    assert f(A, 64, 250, 256, A, A, 0, 4, 0, 4, A, A, 1 << 30, 0, None) == hsq.E_SHAPE
    assert f(A, 64, 256, 256, A, A, 0, 4, 0, 4, A, A, 0, 0, None) == hsq.E_WORKSPACE


def test_quantize_and_pack_reject_before_launch():
    q = lib.hsq_quantize_act
    assert q(None, 4, 64, A, A, 4, A, A, A, None) == hsq.E_INVAL
    assert q(A, 4, 96, A, A, 4, A, A, A, None) == hsq.E_SHAPE
    assert q(A, 4, 64, A, None, 4, A, A, A, None) == hsq.E_INVAL
    assert q(A, 4, 64, A, A, 4, A, A, None, None) == hsq.E_INVAL
    assert q(A, 4, 64, A + 2, A, 4, A, A, A, None) == hsq.E_ALIGN
    assert q(A, 0, 64, A, A, 4, A, A, A, None) == hsq.E_INVAL
    assert q(A, 4, 12288 + 64, A, A, 4, A, A, A, None) == hsq.E_INVAL
    p = lib.hsq_pack_weights
    assert p(None, 64, 16, A, A, None) == hsq.E_INVAL
    assert p(A, 64, 16, A, None, None) == hsq.E_INVAL
    assert p(A, 65, 16, A, A, None) == hsq.E_SHAPE
    assert p(A, 64, 16, A + 1, A, None) == hsq.E_ALIGN
    u = lib.hsq_unpack_weights
    assert u(A, 64, 0, A, None) == hsq.E_INVAL
    assert u(A, 64, 16, A + 3, None) == hsq.E_ALIGN


def test_last_hip_error_is_static_text():
    # no HIP call has failed on this thread (none reach the runtime here)
    assert lib.hsq_last_hip_error() == b"no HIP error"


def test_one_hip_runtime_in_the_process():
    # the binding loads torch before libhsq, so both use one HIP runtime
    maps = open("/proc/self/maps").read()
    hip = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(hip) == 1, hip


def test_group_width_entry_points_validate():
    ws = lib.hsq_workspace_bytes_g
    assert ws(64, 256, 256, 4, 1, 64) == lib.hsq_workspace_bytes(64, 256, 256, 4, 1)
    assert ws(64, 256, 256, 4, 1, 128) > 0
    assert ws(64, 256, 256, 4, 1, 96) == 0          # not a supported width
    assert ws(64, 320, 256, 4, 1, 128) == 0         # 128 does not divide K
    # group-128 scales take half the bytes of group-64 ones
    assert ws(4096, 4096, 12288, 4, 1, 128) < ws(4096, 4096, 12288, 4, 1, 64)
    f = lib.hsq_w4a4_lowrank_linear_g
    args = (A, A, A, A, A, 4, A, A, hsq.BF16, A, 1 << 30, 0, None)
    assert f(A, 64, 256, 256, 1, 96, *args) == hsq.E_INVAL
    assert f(A, 64, 320, 256, 1, 128, *args) == hsq.E_SHAPE
    assert f(None, 64, 256, 256, 1, 128, *args) == hsq.E_INVAL
    assert f(A, 64, 256, 256, 1, 128, A, A, A, A, A, 4, A, A, hsq.BF16, A, 0, 0, None) == hsq.E_WORKSPACE
    q = lib.hsq_w4a4_quantize_stage_g
    assert q(A, 64, 320, 256, 1, 128, A, A, 4, A, 1 << 30, None) == hsq.E_SHAPE
    c = lib.hsq_w4a4_contract_stage_g
    assert c(64, 256, 256, 1, 32, A, A, A, 4, A, A, hsq.BF16, A, 1 << 30, 0, None) == hsq.E_INVAL
    pg = lib.hsq_w4a4_group_partials_g
    assert pg(A, 64, 256, 256, 128, A, A, 0, 65, 0, 256, A, A, 1 << 30, 0, None) == hsq.E_SHAPE


def test_calibration_entry_points_validate():
    ws = lib.hsq_hessian_workspace_bytes
    assert ws(4096, 1152) > 0            # 45 blocks of H: token splits with partial blocks
    assert ws(2048, 4096) == 0           # 528 blocks: none
    assert ws(10, 100) == 0 and ws(0, 128) == 0
    h = lib.hsq_hessian_accumulate
    assert h(None, 64, 128, A, A, 0, None, 0, None) == hsq.E_INVAL
    assert h(A, 64, 96, A, A, 0, None, 0, None) == hsq.E_SHAPE
    assert h(A, 64, 32768, A, A, 0, None, 0, None) == hsq.E_INVAL
    assert h(A, 64, 128, A, A, 2, None, 0, None) == hsq.E_INVAL
    assert h(A, 64, 128, A, A + 4, 0, None, 0, None) == hsq.E_ALIGN
    assert h(A, 1 << 17, 1 << 13, A, A, 0, A, 1 << 40, None) == hsq.E_INVAL   # M * K >= 2^30
    assert h(A, 4096, 1152, A, A, 0, A, 16, None) == hsq.E_WORKSPACE
    d = lib.hsq_deflate_hessian
    assert lib.hsq_deflate_workspace_bytes(1024, 4) > 1024 * 4 * 4
    assert lib.hsq_deflate_workspace_bytes(1024, 0) == 0
    assert d(A, 128, A, 0, A, A, A, A, 1 << 20, None) == hsq.E_INVAL
    assert d(A, 128, A, 33, A, A, A, A, 1 << 20, None) == hsq.E_INVAL
    assert d(A, 96, A, 4, A, A, A, A, 1 << 20, None) == hsq.E_SHAPE
    assert d(A, 128, A, 4, A, A + 8, A, A, 1 << 20, None) == hsq.E_ALIGN
    assert d(A, 128, A, 4, A, A, A, A, 16, None) == hsq.E_WORKSPACE
    l2 = lib.hsq_closed_form_l2
    assert lib.hsq_closed_form_l2_workspace_bytes(1152, 4608, 4) > 0
    assert l2(A, A, 256, 64, 4, 96, A, A, A, A, A, 1 << 20, None) == hsq.E_INVAL
    assert l2(A, A, 192, 64, 4, 128, A, A, A, A, A, 1 << 20, None) == hsq.E_SHAPE
    assert l2(A, A, 256, 0, 4, 64, A, A, A, A, A, 1 << 20, None) == hsq.E_INVAL
    assert l2(A, A, 256, 64, 4, 64, None, A, A, A, A, 1 << 20, None) == hsq.E_INVAL
    assert l2(A, A, 256, 64, 4, 64, A, A, A, A, A, 0, None) == hsq.E_WORKSPACE


def test_format_variant_entry_points_validate():
    # asymmetric activations: the _g checks plus the format argument
    f = lib.hsq_w4a4_lowrank_linear_aq
    args = (A, A, A, A, A, 4, A, A, hsq.BF16, A, 1 << 30, 0, None)
    assert f(A, 64, 256, 256, 1, 64, 2, *args) == hsq.E_INVAL            # no such format
    assert f(A, 64, 256, 256, 1, 64, -1, *args) == hsq.E_INVAL
    assert f(A, 64, 320, 256, 1, 128, 1, *args) == hsq.E_SHAPE           # 128 does not divide K
    assert f(A, 64, 256, 256, 1, 64, 1, A, A, A, A, A, 4, A, A, hsq.BF16, A, 0, 0, None) == hsq.E_WORKSPACE
    assert f(A, 64, 256, 256, 1, 64, 1, A, A, A, None, A, 4, A, A, hsq.BF16, A, 1 << 30, 0, None) == hsq.E_INVAL
    q = lib.hsq_w4a4_quantize_stage_aq
    assert q(A, 64, 256, 256, 1, 64, 3, A, A, 4, A, 1 << 30, None) == hsq.E_INVAL
    assert q(A, 64, 256, 256, 1, 64, 1, A + 8, A, 4, A, 1 << 30, None) == hsq.E_ALIGN
    pq = lib.hsq_w4a4_group_partials_aq
    assert pq(A, 64, 256, 256, 64, 1, A, A, 0, 65, 0, 256, A, A, 1 << 30, 0, None) == hsq.E_SHAPE
    assert pq(A, 64, 256, 256, 64, 5, A, A, 0, 64, 0, 256, A, A, 1 << 30, 0, None) == hsq.E_INVAL
    # MX-fp4
    assert lib.hsq_mx_packed_weight_bytes(63, 16) == 0
    assert lib.hsq_mx_packed_weight_bytes(128, 16) == 1024 + 256     # one code block, one scale block
    assert lib.hsq_mx_packed_weight_bytes(192, 33) == 3 * 2 * 1024 + 3 * 256
    assert lib.hsq_mx_workspace_bytes(64, 256, 4) > 0
    assert lib.hsq_mx_workspace_bytes(64, 100, 4) == 0
    mp = lib.hsq_mx_pack_weights
    assert mp(A, 96, 16, A, None) == hsq.E_SHAPE
    assert mp(None, 128, 16, A, None) == hsq.E_INVAL
    assert mp(A + 4, 128, 16, A, None) == hsq.E_ALIGN
    ml = lib.hsq_mx_lowrank_linear
    assert ml(A, 64, 256, 256, A, A, A, A, 4, A, A, 7, A, 1 << 30, None) == hsq.E_INVAL      # y dtype
    assert ml(A, 64, 256, 256, A, A, None, A, 4, A, A, hsq.BF16, A, 1 << 30, None) == hsq.E_INVAL
    assert ml(A, 64, 250, 256, A, A, A, A, 4, A, A, hsq.BF16, A, 1 << 30, None) == hsq.E_SHAPE
    assert ml(A, 64, 256, 256, A, A, A, A, 4, A, A, hsq.BF16, A, 16, None) == hsq.E_WORKSPACE
    # fused two-layer chain
    mw = lib.hsq_mlp_workspace_bytes
    assert mw(64, 256, 512, 256, 4, 4) > lib.hsq_workspace_bytes(64, 256, 512, 4, 1)
    assert mw(64, 256, 512, 256, 4, 9) == 0          # the down layer's rank is at most 8
    assert mw(64, 256, 500, 256, 4, 4) == 0          # H must be a multiple of 64
    mlp = lib.hsq_w4a4_lowrank_mlp
    up = (A, A, A, A, A, 4, A)
    dn = (A, A, A, A, A, 4, A)
    assert mlp(A, 64, 256, 512, 256, *up[:6], up[6], 9, *dn, A, hsq.BF16, None, A, 1 << 30, None) == hsq.E_INVAL
    assert mlp(A, 64, 256, 512, 256, *up, hsq.ACT_GELU_TANH, *dn, A, 9, None, A, 1 << 30, None) == hsq.E_INVAL
    assert mlp(A, 64, 256, 512, 256, *up, hsq.ACT_GELU_TANH, *dn, A, hsq.BF16, None, A, 16, None) == hsq.E_WORKSPACE
    assert mlp(A, 64, 256, 512, 256, *up, hsq.ACT_GELU_TANH, *dn, A, hsq.BF16, A + 4, A, 1 << 30, None) == hsq.E_ALIGN


def test_noalloc_entry_validates_before_any_device_call():
    # every rejection happens before the scratch address is looked up, so
    # none of these touches a GPU
    f = lib.hsq_w4a4_lowrank_linear_noalloc
    assert f(None, 64, 256, 256, 1, A, A, A, A, A, 4, A, A, hsq.BF16, None) == hsq.E_INVAL
    assert f(A, 64, 100, 256, 1, A, A, A, A, A, 4, A, A, hsq.BF16, None) == hsq.E_SHAPE
    assert f(A + 2, 64, 256, 256, 1, A, A, A, A, A, 4, A, A, hsq.BF16, None) == hsq.E_ALIGN
    assert f(A, 64, 256, 256, 1, A, A, A, A, A, 4, A, A, 2, None) == hsq.E_INVAL
    # codes alone need 2048 x 64 KiB = 128 MiB > the 64 MiB scratch
    assert lib.hsq_workspace_bytes(32767, 4096, 16, 4, 1) > hsq.NOALLOC_SCRATCH_BYTES
    assert f(A, 32767, 4096, 16, 1, A, A, A, A, A, 4, A, A, hsq.BF16, None) == hsq.E_SCRATCH
    text = open(hsq.HEADER).read()
    assert "#define HSQ_NOALLOC_SCRATCH_BYTES (64u << 20)" in text
    assert "#define HSQ_E_SCRATCH    -6" in text
    assert b"static scratch" in lib.hsq_status_string(hsq.E_SCRATCH)


def test_every_header_is_exported_by_its_library():
    # include/hsq.h -> libhsq.so, include/hsq_probe.h -> libhsq_probe.so
    import glob
    import os

    libs = {"hsq.h": hsq.LIB_PATH,
            "hsq_probe.h": os.path.join(os.path.dirname(hsq.LIB_PATH), "libhsq_probe.so")}
    headers = sorted(os.path.basename(h) for h in glob.glob(os.path.join(os.path.dirname(hsq.HEADER), "*.h")))
    assert headers == sorted(libs)
    for h, so in libs.items():
        text = open(os.path.join(os.path.dirname(hsq.HEADER), h)).read()
        names = set(re.findall(r"\b(hsq_[a-z0-9_]+)\s*\(", text))
        assert names, h
        out = subprocess.run(["nm", "-D", "--defined-only", so], capture_output=True, text=True,
                             check=True).stdout
        assert names <= set(re.findall(r"\bT (hsq_\w+)", out)), h


def test_probe_entry_points_validate_without_launching():
    import os

    plib = ctypes.CDLL(os.path.join(os.path.dirname(hsq.LIB_PATH), "libhsq_probe.so"))
    I, S = ctypes.c_int, ctypes.c_size_t
    plib.hsq_probe_mfma.argtypes = [I, I, I, I, P, P]
    plib.hsq_probe_read.argtypes = [P, S, I, P, P]
    plib.hsq_probe_copy.argtypes = [P, S, I, P, P]
    assert plib.hsq_probe_mfma(6, 10, 1, 8, A, None) == -1      # no such mode
    assert plib.hsq_probe_mfma(4, 10, 1, 16, A, None) == -1     # the wide tile takes 8 waves at most
    assert plib.hsq_probe_mfma(0, 10, 1, 17, A, None) == -1     # more than 16 waves
    assert plib.hsq_probe_mfma(0, 0, 1, 8, A, None) == -1
    assert plib.hsq_probe_mfma(0, 10, 1, 8, None, None) == -1
    assert plib.hsq_probe_mfma(0, 10, 1, 8, A + 4, None) == -3
    assert plib.hsq_probe_read(A, 100, 8, A, None) == -1        # not a multiple of 16
    assert plib.hsq_probe_read(None, 1024, 8, A, None) == -1
    assert plib.hsq_probe_copy(A, 1024, 8, A + 8, None) == -3
