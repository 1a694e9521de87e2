"""Python binding of libhsq, the MI355X (gfx950) W4A4 + rank-r linear layer.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI declared in ``include/hsq.h``; PyTorch provides device
memory and the current stream.  Importing this module never falls back to
anything: if ``_lib/libhsq.so`` is missing or cannot be loaded, every call
raises.

Half-precision inputs may be passed as torch.bfloat16 / torch.float16
tensors or as int16 / uint16 tensors holding the bit patterns.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libhsq.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "hsq.h")

OK, E_INVAL, E_SHAPE, E_ALIGN, E_WORKSPACE, E_HIP, E_SCRATCH = 0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 64 << 20
F32, BF16 = 0, 1
KERNEL_AUTO, KERNEL_TILED, KERNEL_SKINNY = 0, 1, 2
ACT_IDENTITY, ACT_GELU_TANH = 0, 1
_ACTS = {"identity": ACT_IDENTITY, "gelu_tanh": ACT_GELU_TANH}
_KERNELS = {"auto": KERNEL_AUTO, "tiled": KERNEL_TILED, "skinny": KERNEL_SKINNY}

_lib = None


class HsqError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = _load().hsq_status_string(status).decode() if _lib is not None else str(status)
        if status == E_HIP and _lib is not None:
            msg += ": " + _lib.hsq_last_hip_error().decode()
        super().__init__(f"{what}: {msg} (status {status})")
        self.status = status


def _load():
    """Load libhsq.so (raises OSError if it is missing: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing; build it with w4a4_rank_assisted_amd.build.build()")
        # torch first: its HIP runtime is then the one libhsq binds to (same
        # soname), so the device pointers and streams torch hands over belong
        # to the runtime the kernels are launched with.  Loaded the other way
        # round, the process would hold two HIP / HSA runtimes.
        import torch  # noqa: F401
        lib = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        sig = {
            "hsq_layout_version": ([], I),
            "hsq_status_string": ([I], ctypes.c_char_p),
            "hsq_last_hip_error": ([], ctypes.c_char_p),
            "hsq_packed_weight_bytes": ([I, I], S),
            "hsq_pack_weights": ([P, I, I, P, P, P], I),
            "hsq_unpack_weights": ([P, I, I, P, P], I),
            "hsq_quantize_act": ([P, I, I, P, P, I, P, P, P, P], I),
            "hsq_workspace_bytes": ([I, I, I, I, I], S),
            "hsq_w4a4_lowrank_linear": ([P, I, I, I, I, P, P, P, P, P, I, P, P, I, P, S, P], I),
            "hsq_w4a4_lowrank_linear_noalloc": ([P, I, I, I, I, P, P, P, P, P, I, P, P, I, P], I),
            "hsq_w4a4_lowrank_linear_ex": ([P, I, I, I, I, P, P, P, P, P, I, P, P, I, P, S, I, P], I),
            "hsq_w4a4_group_partials": ([P, I, I, I, P, P, I, I, I, I, P, P, S, I, P], I),
            "hsq_w4a4_quantize_stage": ([P, I, I, I, I, P, P, I, P, S, P], I),
            "hsq_w4a4_contract_stage": ([I, I, I, I, P, P, P, I, P, P, I, P, S, I, P], I),
            "hsq_workspace_bytes_g": ([I, I, I, I, I, I], S),
            "hsq_w4a4_lowrank_linear_g": ([P, I, I, I, I, I, P, P, P, P, P, I, P, P, I, P, S, I, P], I),
            "hsq_w4a4_quantize_stage_g": ([P, I, I, I, I, I, P, P, I, P, S, P], I),
            "hsq_w4a4_contract_stage_g": ([I, I, I, I, I, P, P, P, I, P, P, I, P, S, I, P], I),
            "hsq_w4a4_group_partials_g": ([P, I, I, I, I, P, P, I, I, I, I, P, P, S, I, P], I),
            "hsq_w4a4_lowrank_linear_aq": ([P, I, I, I, I, I, I, P, P, P, P, P, I, P, P, I, P, S, I, P], I),
            "hsq_w4a4_quantize_stage_aq": ([P, I, I, I, I, I, I, P, P, I, P, S, P], I),
            "hsq_w4a4_group_partials_aq": ([P, I, I, I, I, I, P, P, I, I, I, I, P, P, S, I, P], I),
            "hsq_mx_packed_weight_bytes": ([I, I], S),
            "hsq_mx_pack_weights": ([P, I, I, P, P], I),
            "hsq_mx_workspace_bytes": ([I, I, I], S),
            "hsq_mx_lowrank_linear": ([P, I, I, I, P, P, P, P, I, P, P, I, P, S, P], I),
            "hsq_mlp_workspace_bytes": ([I, I, I, I, I, I], S),
            "hsq_w4a4_lowrank_mlp": ([P, I, I, I, I, P, P, P, P, P, I, P, I, P, P, P, P, P, I, P, P, I, P,
                                      P, S, P], I),
            "hsq_hessian_workspace_bytes": ([I, I], S),
            "hsq_hessian_accumulate": ([P, I, I, P, P, I, P, S, P], I),
            "hsq_deflate_workspace_bytes": ([I, I], S),
            "hsq_deflate_hessian": ([P, I, P, I, P, P, P, P, S, P], I),
            "hsq_closed_form_l2_workspace_bytes": ([I, I, I], S),
            "hsq_closed_form_l2": ([P, P, I, I, I, I, P, P, P, P, P, S, P], I),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def header_functions():
    """Names of the functions include/hsq.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(hsq_[a-z0-9_]+)\s*\(", text)))


# --------------------------------------------------------------- marshalling
def _torch():
    import torch

    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_tensor(t, name, dtypes, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if dtypes and t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return t


def _half_types():
    torch = _torch()
    return (torch.bfloat16, torch.float16, torch.int16, torch.uint16)


def _check(status: int, what: str):
    if status != OK:
        raise HsqError(status, what)


# ------------------------------------------------------------------ the API
def layout_version() -> int:
    return int(_load().hsq_layout_version())


def packed_weight_bytes(K: int, N: int) -> int:
    return int(_load().hsq_packed_weight_bytes(K, N))


def workspace_bytes(M: int, K: int, N: int, r: int, batch: int = 1, group: int = 64) -> int:
    lib = _load()
    if group == 64:
        return int(lib.hsq_workspace_bytes(M, K, N, r, batch))
    return int(lib.hsq_workspace_bytes_g(M, K, N, r, batch, group))


def pack_weights(codes, packed=None, status=None):
    """codes: (K, N) int8 device tensor -> (packed uint8 blob, device status int32)."""
    torch = _torch()
    lib = _load()
    _dev_tensor(codes, "codes", (torch.int8,))
    K, N = codes.shape
    nbytes = lib.hsq_packed_weight_bytes(K, N)
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=codes.device)
    if status is None:
        status = torch.empty(4, dtype=torch.int32, device=codes.device)
    _dev_tensor(packed, "packed", (torch.uint8,), (nbytes,))
    _check(lib.hsq_pack_weights(_ptr(codes), K, N, _ptr(packed), _ptr(status), _stream()),
           "hsq_pack_weights")
    return packed, status


def unpack_weights(packed, K: int, N: int):
    torch = _torch()
    lib = _load()
    _dev_tensor(packed, "packed", (torch.uint8,))
    codes = torch.empty((K, N), dtype=torch.int8, device=packed.device)
    _check(lib.hsq_unpack_weights(_ptr(packed), K, N, _ptr(codes), _stream()), "hsq_unpack_weights")
    return codes


def quantize_act(X, lam, L1=None):
    """X (M, K) bf16, lam (K,) fp16, L1 (K, r) bf16 or None ->
    (qx (M, K/2) uint8, sx (M, K/64) int16 fp16 bits, U (M, r) fp32)."""
    torch = _torch()
    lib = _load()
    _dev_tensor(X, "X", _half_types())
    M, K = X.shape
    _dev_tensor(lam, "lambda", _half_types(), (K,))
    r = 0 if L1 is None else int(L1.shape[1])
    if L1 is not None:
        _dev_tensor(L1, "L1", _half_types(), (K, r))
    dev = X.device
    qx = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    sx = torch.empty((M, max(K // 64, 1)), dtype=torch.int16, device=dev)
    U = torch.empty((M, max(r, 1)), dtype=torch.float32, device=dev)
    _check(lib.hsq_quantize_act(_ptr(X), M, K, _ptr(lam), _ptr(L1), r, _ptr(qx), _ptr(sx),
                                _ptr(U) if r else None, _stream()), "hsq_quantize_act")
    return qx, sx, U[:, :r]


_ACT_QUANT = {"sym": 0, "asym": 1}


def w4a4_lowrank_linear(X, lam, packed_w, sw, L1=None, L2=None, bias=None, *, N: int,
                        batch: int = 1, y_dtype: str = "bf16", out=None, workspace=None,
                        kernel: str = "auto", group: int = 64, act_quant: str = "sym"):
    """The fused layer.  Shapes: X (M, K); lam (K,); packed_w (batch * blob,);
    sw (batch, K/group, N); L1 (batch, K, r); L2 (batch, r, N); bias (batch, N).
    Returns Y (batch, M, N) as bf16 or fp32.  Symmetric group-64 activations
    call hsq_w4a4_lowrank_linear_ex, other widths hsq_w4a4_lowrank_linear_g,
    asymmetric activations (act_quant="asym") hsq_w4a4_lowrank_linear_aq."""
    torch = _torch()
    lib = _load()
    _dev_tensor(X, "X", _half_types())
    M, K = X.shape
    G = K // group
    _dev_tensor(lam, "lambda", _half_types(), (K,))
    _dev_tensor(packed_w, "packed_w", (torch.uint8,), (batch * lib.hsq_packed_weight_bytes(K, N),))
    _dev_tensor(sw, "sw", _half_types(), (batch, G, N))
    r = 0 if L1 is None else int(L1.shape[-1])
    if r:
        _dev_tensor(L1, "L1", _half_types(), (batch, K, r))
        _dev_tensor(L2, "L2", _half_types(), (batch, r, N))
    if bias is not None:
        _dev_tensor(bias, "bias", _half_types(), (batch, N))
    ydt = {"bf16": (BF16, torch.bfloat16), "f32": (F32, torch.float32)}[y_dtype]
    if out is None:
        out = torch.empty((batch, M, N), dtype=ydt[1], device=X.device)
    _dev_tensor(out, "out", (ydt[1],), (batch, M, N))
    need = workspace_bytes(M, K, N, r, batch, group)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    _dev_tensor(workspace, "workspace", (torch.uint8,))
    args = (_ptr(lam), _ptr(packed_w), _ptr(sw), _ptr(L1) if r else None, _ptr(L2) if r else None,
            r, _ptr(bias), _ptr(out), ydt[0], _ptr(workspace), workspace.numel(), _KERNELS[kernel],
            _stream())
    if act_quant != "sym":
        _check(lib.hsq_w4a4_lowrank_linear_aq(_ptr(X), M, K, N, batch, group, _ACT_QUANT[act_quant], *args),
               "hsq_w4a4_lowrank_linear_aq")
    elif group == 64:
        _check(lib.hsq_w4a4_lowrank_linear_ex(_ptr(X), M, K, N, batch, *args), "hsq_w4a4_lowrank_linear")
    else:
        _check(lib.hsq_w4a4_lowrank_linear_g(_ptr(X), M, K, N, batch, group, *args),
               "hsq_w4a4_lowrank_linear_g")
    return out


def w4a4_lowrank_linear_noalloc(X, lam, packed_w, sw, L1=None, L2=None, bias=None, *, N: int,
                                batch: int = 1, y_dtype: str = "bf16", out=None):
    """The fused layer (group 64, symmetric activations) with its workspace
    in the library's static per-device scratch (hsq_w4a4_lowrank_linear_noalloc):
    no workspace argument and no allocation inside the call.  ``out`` must
    be given by callers that cannot allocate (this wrapper allocates it
    otherwise).  Calls that overlap in time on one GPU race on the scratch."""
    torch = _torch()
    lib = _load()
    _dev_tensor(X, "X", _half_types())
    M, K = X.shape
    _dev_tensor(lam, "lambda", _half_types(), (K,))
    _dev_tensor(packed_w, "packed_w", (torch.uint8,), (batch * lib.hsq_packed_weight_bytes(K, N),))
    _dev_tensor(sw, "sw", _half_types(), (batch, K // 64, N))
    r = 0 if L1 is None else int(L1.shape[-1])
    if r:
        _dev_tensor(L1, "L1", _half_types(), (batch, K, r))
        _dev_tensor(L2, "L2", _half_types(), (batch, r, N))
    if bias is not None:
        _dev_tensor(bias, "bias", _half_types(), (batch, N))
    ydt = {"bf16": (BF16, torch.bfloat16), "f32": (F32, torch.float32)}[y_dtype]
    if out is None:
        out = torch.empty((batch, M, N), dtype=ydt[1], device=X.device)
    _dev_tensor(out, "out", (ydt[1],), (batch, M, N))
    _check(lib.hsq_w4a4_lowrank_linear_noalloc(_ptr(X), M, K, N, batch, _ptr(lam), _ptr(packed_w), _ptr(sw),
                                               _ptr(L1) if r else None, _ptr(L2) if r else None, r, _ptr(bias),
                                               _ptr(out), ydt[0], _stream()),
           "hsq_w4a4_lowrank_linear_noalloc")
    return out


def quantize_stage(X, lam, L1, *, N: int, batch: int, workspace, group: int = 64,
                   act_quant: str = "sym"):
    """First stage of the layer: quantize X and form U into ``workspace``."""
    lib = _load()
    M, K = X.shape
    r = 0 if L1 is None else int(L1.shape[-1])
    _check(lib.hsq_w4a4_quantize_stage_aq(_ptr(X), M, K, N, batch, group, _ACT_QUANT[act_quant],
                                          _ptr(lam), _ptr(L1) if r else None, r, _ptr(workspace),
                                          workspace.numel(), _stream()),
           "hsq_w4a4_quantize_stage_aq")


def contract_stage(M: int, K: int, packed_w, sw, L2, bias, out, *, N: int, batch: int, r: int,
                   workspace, kernel: str = "auto", group: int = 64):
    """Second stage: contraction + epilogue from the workspace into ``out``."""
    torch = _torch()
    lib = _load()
    ydt = BF16 if out.dtype == torch.bfloat16 else F32
    _check(lib.hsq_w4a4_contract_stage_g(M, K, N, batch, group, _ptr(packed_w), _ptr(sw),
                                         _ptr(L2) if r else None, r, _ptr(bias), _ptr(out), ydt,
                                         _ptr(workspace), workspace.numel(), _KERNELS[kernel],
                                         _stream()),
           "hsq_w4a4_contract_stage_g")


def w4a4_group_partials(X, lam, packed_w, N: int, m0: int, mc: int, n0: int, nc: int,
                        workspace=None, kernel: str = "auto", group: int = 64, act_quant: str = "sym"):
    """int32 P (mc, nc, K/group) of the window, from the production kernels."""
    torch = _torch()
    lib = _load()
    _dev_tensor(X, "X", _half_types())
    M, K = X.shape
    _dev_tensor(lam, "lambda", _half_types(), (K,))
    _dev_tensor(packed_w, "packed_w", (torch.uint8,))
    P = torch.empty((mc, nc, K // group), dtype=torch.int32, device=X.device)
    need = workspace_bytes(M, K, N, 0, 1, group)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    args = (_ptr(lam), _ptr(packed_w), m0, mc, n0, nc, _ptr(P), _ptr(workspace), workspace.numel(),
            _KERNELS[kernel], _stream())
    if act_quant != "sym":
        _check(lib.hsq_w4a4_group_partials_aq(_ptr(X), M, K, N, group, _ACT_QUANT[act_quant], *args),
               "hsq_w4a4_group_partials_aq")
    elif group == 64:
        _check(lib.hsq_w4a4_group_partials(_ptr(X), M, K, N, *args), "hsq_w4a4_group_partials")
    else:
        _check(lib.hsq_w4a4_group_partials_g(_ptr(X), M, K, N, group, *args),
               "hsq_w4a4_group_partials_g")
    return P


class Layer:
    """A packed W4A4 + rank-r layer resident on the device: holds the packed
    residual blobs, the scales, the low-rank factors, the bias and a reusable
    workspace, and runs the fused call on the current stream."""

    def __init__(self, lam, qw, sw, L1=None, L2=None, bias=None, max_tokens: int = 0,
                 group: int = 64):
        torch = _torch()
        self.batch, self.K, self.N = qw.shape
        self.group = group
        self.r = 0 if L1 is None else int(L1.shape[-1])
        blobs = [pack_weights(qw[b].contiguous())[0] for b in range(self.batch)]
        self.packed = torch.cat(blobs) if self.batch > 1 else blobs[0]
        self.lam, self.sw, self.L1, self.L2, self.bias = lam, sw, L1, L2, bias
        self.workspace = None
        if max_tokens:
            self.workspace = torch.empty(
                workspace_bytes(max_tokens, self.K, self.N, self.r, self.batch, group),
                dtype=torch.uint8, device=qw.device)

    def __call__(self, X, y_dtype: str = "bf16", out=None, kernel: str = "auto"):
        ws = self.workspace
        need = workspace_bytes(X.shape[0], self.K, self.N, self.r, self.batch, self.group)
        if ws is None or ws.numel() < need:
            ws = None
        return w4a4_lowrank_linear(X, self.lam, self.packed, self.sw, self.L1, self.L2, self.bias,
                                   N=self.N, batch=self.batch, y_dtype=y_dtype, out=out,
                                   workspace=ws, kernel=kernel, group=self.group)


# ------------------------------------------------------------- MX-fp4 variant
def mx_pack_weights(R):
    """R (K, N) fp32 device tensor -> packed MX-fp4 blob (uint8)."""
    torch = _torch()
    lib = _load()
    _dev_tensor(R, "R", (torch.float32,))
    K, N = R.shape
    packed = torch.empty(lib.hsq_mx_packed_weight_bytes(K, N), dtype=torch.uint8, device=R.device)
    _check(lib.hsq_mx_pack_weights(_ptr(R), K, N, _ptr(packed), _stream()), "hsq_mx_pack_weights")
    return packed


def mx_lowrank_linear(X, lam, packed, L1=None, L2=None, bias=None, *, N: int, y_dtype: str = "bf16",
                      out=None, workspace=None):
    """The MX-fp4 layer: X (M, K) bf16, lam (K,), packed (from mx_pack_weights),
    L1 (K, r), L2 (r, N), bias (N,) -> Y (M, N)."""
    torch = _torch()
    lib = _load()
    _dev_tensor(X, "X", _half_types())
    M, K = X.shape
    _dev_tensor(lam, "lambda", _half_types(), (K,))
    _dev_tensor(packed, "packed", (torch.uint8,), (lib.hsq_mx_packed_weight_bytes(K, N),))
    r = 0 if L1 is None else int(L1.shape[-1])
    if r:
        _dev_tensor(L1, "L1", _half_types(), (K, r))
        _dev_tensor(L2, "L2", _half_types(), (r, N))
    if bias is not None:
        _dev_tensor(bias, "bias", _half_types(), (N,))
    ydt = {"bf16": (BF16, torch.bfloat16), "f32": (F32, torch.float32)}[y_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=ydt[1], device=X.device)
    _dev_tensor(out, "out", (ydt[1],), (M, N))
    if workspace is None:
        workspace = torch.empty(lib.hsq_mx_workspace_bytes(M, K, r), dtype=torch.uint8, device=X.device)
    _check(lib.hsq_mx_lowrank_linear(_ptr(X), M, K, N, _ptr(lam), _ptr(packed), _ptr(L1) if r else None,
                                     _ptr(L2) if r else None, r, _ptr(bias), _ptr(out), ydt[0],
                                     _ptr(workspace), workspace.numel(), _stream()),
           "hsq_mx_lowrank_linear")
    return out


# ------------------------------------------------------------- fused chain
def mlp_workspace_bytes(M: int, K: int, H: int, N: int, r_up: int, r_down: int) -> int:
    return int(_load().hsq_mlp_workspace_bytes(M, K, H, N, r_up, r_down))


def w4a4_lowrank_mlp(X, up, down, *, H: int, N: int, act: str = "gelu_tanh", y_dtype: str = "bf16",
                     out=None, hidden_out=None, workspace=None):
    """Y = down(act(up(X))) with the down layer's quantized input formed in the
    up layer's epilogue.  ``up`` / ``down`` are dicts with lam, packed, sw,
    L1, L2, bias (shapes as for one projection of w4a4_lowrank_linear; L1,
    L2 may be None for rank 0).  hidden_out: optional (M, H) fp32 tensor that
    receives the up layer's output before the activation."""
    torch = _torch()
    lib = _load()
    _dev_tensor(X, "X", _half_types())
    M, K = X.shape
    r1 = 0 if up.get("L1") is None else int(up["L1"].shape[-1])
    r2 = 0 if down.get("L1") is None else int(down["L1"].shape[-1])
    for name, d, kk, nn, r in (("up", up, K, H, r1), ("down", down, H, N, r2)):
        _dev_tensor(d["lam"], f"{name}.lam", _half_types(), (kk,))
        _dev_tensor(d["packed"], f"{name}.packed", (torch.uint8,), (lib.hsq_packed_weight_bytes(kk, nn),))
        _dev_tensor(d["sw"], f"{name}.sw", _half_types(), (kk // 64, nn))
        if r:
            _dev_tensor(d["L1"], f"{name}.L1", _half_types(), (kk, r))
            _dev_tensor(d["L2"], f"{name}.L2", _half_types(), (r, nn))
        if d.get("bias") is not None:
            _dev_tensor(d["bias"], f"{name}.bias", _half_types(), (nn,))
    ydt = {"bf16": (BF16, torch.bfloat16), "f32": (F32, torch.float32)}[y_dtype]
    if out is None:
        out = torch.empty((M, N), dtype=ydt[1], device=X.device)
    _dev_tensor(out, "out", (ydt[1],), (M, N))
    if hidden_out is not None:
        _dev_tensor(hidden_out, "hidden_out", (torch.float32,), (M, H))
    if workspace is None:
        workspace = torch.empty(mlp_workspace_bytes(M, K, H, N, r1, r2), dtype=torch.uint8, device=X.device)
    _dev_tensor(workspace, "workspace", (torch.uint8,))

    def layer_args(d, r):
        return (_ptr(d["lam"]), _ptr(d["packed"]), _ptr(d["sw"]), _ptr(d["L1"]) if r else None,
                _ptr(d["L2"]) if r else None, r, _ptr(d.get("bias")))

    _check(lib.hsq_w4a4_lowrank_mlp(_ptr(X), M, K, H, N, *layer_args(up, r1), _ACTS[act],
                                    *layer_args(down, r2), _ptr(out), ydt[0], _ptr(hidden_out),
                                    _ptr(workspace), workspace.numel(), _stream()),
           "hsq_w4a4_lowrank_mlp")
    return out


# ------------------------------------------------------------- calibration
def _workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def hessian_accumulate(X, lam, H=None, accumulate: bool = False, workspace=None):
    """H = Xh^T Xh (or H += it): X (M, K) bf16, lam (K,) fp16 -> H (K, K) fp32."""
    torch = _torch()
    lib = _load()
    _dev_tensor(X, "X", _half_types())
    M, K = X.shape
    _dev_tensor(lam, "lambda", _half_types(), (K,))
    if H is None:
        H = torch.empty((K, K), dtype=torch.float32, device=X.device)
    _dev_tensor(H, "H", (torch.float32,), (K, K))
    need = int(lib.hsq_hessian_workspace_bytes(M, K))
    if workspace is None:
        workspace = _workspace(need, X.device)
    _check(lib.hsq_hessian_accumulate(_ptr(X), M, K, _ptr(lam), _ptr(H), int(bool(accumulate)),
                                      _ptr(workspace), workspace.numel(), _stream()),
           "hsq_hessian_accumulate")
    return H


def deflate_hessian(H, L1, Hperp=None, workspace=None):
    """Deflation of H (K, K) fp32 by span(L1), L1 (K, r) bf16 ->
    (Hperp (K, K) fp32, HL1 (K, r) fp32, Cinv (r, r) fp64).  Pass Hperp=H
    to deflate in place."""
    torch = _torch()
    lib = _load()
    K = H.shape[0]
    _dev_tensor(H, "H", (torch.float32,), (K, K))
    r = int(L1.shape[1])
    _dev_tensor(L1, "L1", _half_types(), (K, r))
    if Hperp is None:
        Hperp = torch.empty_like(H)
    _dev_tensor(Hperp, "Hperp", (torch.float32,), (K, K))
    HL1 = torch.empty((K, r), dtype=torch.float32, device=H.device)
    Cinv = torch.empty((r, r), dtype=torch.float64, device=H.device)
    if workspace is None:
        workspace = _workspace(lib.hsq_deflate_workspace_bytes(K, r), H.device)
    _check(lib.hsq_deflate_hessian(_ptr(H), K, _ptr(L1), r, _ptr(Hperp), _ptr(HL1), _ptr(Cinv),
                                   _ptr(workspace), workspace.numel(), _stream()),
           "hsq_deflate_hessian")
    return Hperp, HL1, Cinv


def closed_form_l2(HL1, Cinv, W, packed_w, sw, group: int = 64, out=None, workspace=None):
    """L2* (r, N) fp32 from HL1 (K, r), Cinv (r, r) fp64, W (K, N) bf16 and the
    packed residual (codes + sw (K/group, N) fp16) of the same projection."""
    torch = _torch()
    lib = _load()
    K, r = HL1.shape
    _dev_tensor(HL1, "HL1", (torch.float32,), (K, r))
    _dev_tensor(Cinv, "Cinv", (torch.float64,), (r, r))
    _dev_tensor(W, "W", _half_types())
    N = int(W.shape[1])
    _dev_tensor(W, "W", _half_types(), (K, N))
    _dev_tensor(packed_w, "packed_w", (torch.uint8,), (lib.hsq_packed_weight_bytes(K, N),))
    _dev_tensor(sw, "sw", _half_types(), (K // group, N))
    if out is None:
        out = torch.empty((r, N), dtype=torch.float32, device=W.device)
    _dev_tensor(out, "L2", (torch.float32,), (r, N))
    if workspace is None:
        workspace = _workspace(lib.hsq_closed_form_l2_workspace_bytes(K, N, r), W.device)
    _check(lib.hsq_closed_form_l2(_ptr(HL1), _ptr(Cinv), K, N, r, group, _ptr(W), _ptr(packed_w),
                                  _ptr(sw), _ptr(out), _ptr(workspace), workspace.numel(), _stream()),
           "hsq_closed_form_l2")
    return out

