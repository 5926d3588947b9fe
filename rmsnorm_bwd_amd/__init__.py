"""Python binding of the MI355X RMSNorm library (``librmsnorm_mi355x.so``).

Argument marshalling only: every function here checks shapes, dtypes,
devices and contiguity of torch tensors, passes raw device pointers and the
current HIP stream to the C entry point of the same name, and turns a
non-zero status into an exception. All arithmetic runs in the library's HIP
kernels; there is no fallback. If the library is not built, importing works
but every call raises.

Pages cited, by title:
  [I769] FlyDSL issue #769, "[Feature] Add rmsnorm backward (+ forward saves
         rstd) to enable training / downstream (quack) integration" - also its
         PR sequence and status updates for the LayerNorm entry points
         (forward saving mean and rstd, backward with dbias, weight and bias
         length checks)
  [P800] FlyDSL PR #800, "[rmsnorm] Add fused-add / residual backward
         (PR 2/3, #769)" - its review-fix commit asks for the shape and
         contiguity checks, its fused-add commit for one dtype across operands.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librmsnorm_mi355x.so")

F32, F16, BF16 = 0, 1, 2
DGAMMA_AUTO, DGAMMA_DETERMINISTIC, DGAMMA_ATOMIC, CHECK_DEVICE = 0, 1, 2, 4
MAX_N = 16384
_DTYPE_CODE = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}

_lib = None


class RmsnError(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, fn, status, text):
        super().__init__(f"{fn}: status {status} ({text})")
        self.status = status


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "(hipcc, gfx950). There is no fallback path.")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, F, I, U, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                               ctypes.c_uint, ctypes.c_size_t)
        L.rmsnorm_fwd_rstd.argtypes = [P, P, P, P, I64, I64, F, I, P]
        L.fused_add_rmsnorm_fwd_rstd.argtypes = [P, P, P, P, P, P, I64, I64, F, I, P]
        L.rmsnorm_bwd_workspace_bytes.argtypes = [I64, I64, I, U]
        L.rmsnorm_bwd_workspace_bytes.restype = SZ
        L.rmsnorm_bwd.argtypes = [P, P, P, P, P, P, P, P, SZ, I64, I64, I, U, P]
        L.fused_add_rmsnorm_bwd.argtypes = [P, P, P, P, P, P, P, P, P, SZ, I64, I64, I, U, P]
        L.layernorm_fwd_stats.argtypes = [P, P, P, P, P, P, I64, I64, F, I, P]
        L.layernorm_bwd_workspace_bytes.argtypes = [I64, I64, I, U]
        L.layernorm_bwd_workspace_bytes.restype = SZ
        L.layernorm_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, SZ, I64, I64, I, U, P]
        L.rmsn_status_string.argtypes = [I]
        L.rmsn_status_string.restype = ctypes.c_char_p
        for fn in ("rmsnorm_fwd_rstd", "fused_add_rmsnorm_fwd_rstd", "rmsnorm_bwd",
                   "fused_add_rmsnorm_bwd", "layernorm_fwd_stats", "layernorm_bwd"):
            getattr(L, fn).restype = I
        _lib = L
    return _lib


def status_string(status):
    return lib().rmsn_status_string(int(status)).decode()


def _raise_on(fn, status):
    if status != 0:
        raise RmsnError(fn, status, status_string(status))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on_device(device, fn, *args):
    """Call fn with `device` current (the library launches on the current
    device, as the pages' device guard requires), switching only if needed."""
    if device.index == torch.cuda.current_device():
        return fn(*args)
    with torch.cuda.device(device):
        return fn(*args)


def _rows(x, gamma, name):
    """(M, N) view of x with the pages' guards: last dim == len(gamma), contiguous."""
    if gamma.dim() != 1:
        raise ValueError(f"{name}: gamma must be 1-D")
    if x.shape[-1] != gamma.shape[0]:
        raise ValueError(f"{name}: x.shape[-1]={x.shape[-1]} != len(gamma)={gamma.shape[0]}")
    if not x.is_contiguous() or not gamma.is_contiguous():
        raise ValueError(f"{name}: tensors must be contiguous (row-major)")
    return x.reshape(-1, x.shape[-1])


def _same(name, ref, *ts):
    for t in ts:
        if t is None:
            continue
        if t.dtype != ref.dtype:
            raise TypeError(f"{name}: dtype mismatch {t.dtype} vs {ref.dtype}")
        if t.device != ref.device:
            raise ValueError(f"{name}: tensors on different devices")
        if not t.is_contiguous():
            raise ValueError(f"{name}: tensors must be contiguous (row-major)")


def _code(t, name):
    if t.dtype not in _DTYPE_CODE:
        raise TypeError(f"{name}: unsupported dtype {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: tensors must be on a GPU")
    return _DTYPE_CODE[t.dtype]


def rmsnorm_fwd_rstd(x, gamma, eps, y=None, rstd=None):
    """Forward that saves rstd ([I769] Scope/tasks item 2). Returns (y, rstd)."""
    dt = _code(x, "rmsnorm_fwd_rstd")
    x2 = _rows(x, gamma, "rmsnorm_fwd_rstd")
    M, N = x2.shape
    y = torch.empty_like(x) if y is None else y
    rstd = torch.empty(M, dtype=torch.float32, device=x.device) if rstd is None else rstd
    _same("rmsnorm_fwd_rstd", x, gamma, y)
    _check_rstd(rstd, M, x.device)
    st = _on_device(x.device, lambda: lib().rmsnorm_fwd_rstd(
        _p(x2), _p(gamma), _p(y), _p(rstd), M, N, float(eps), dt, _stream(x.device)))
    _raise_on("rmsnorm_fwd_rstd", st)
    return y, rstd


def fused_add_rmsnorm_fwd_rstd(x, residual, gamma, eps, out=None, residual_out=None, rstd=None):
    """Fused-add forward ([P800] fused-add commit). Returns (out, residual_out, rstd)."""
    dt = _code(x, "fused_add_rmsnorm_fwd_rstd")
    x2 = _rows(x, gamma, "fused_add_rmsnorm_fwd_rstd")
    if residual.shape != x.shape:
        raise ValueError("fused_add_rmsnorm_fwd_rstd: residual must have x's shape")
    M, N = x2.shape
    out = torch.empty_like(x) if out is None else out
    residual_out = torch.empty_like(x) if residual_out is None else residual_out
    rstd = torch.empty(M, dtype=torch.float32, device=x.device) if rstd is None else rstd
    _same("fused_add_rmsnorm_fwd_rstd", x, residual, gamma, out, residual_out)
    _check_rstd(rstd, M, x.device)
    st = _on_device(x.device, lambda: lib().fused_add_rmsnorm_fwd_rstd(
        _p(x2), _p(residual), _p(gamma), _p(out), _p(residual_out), _p(rstd), M, N, float(eps),
        dt, _stream(x.device)))
    _raise_on("fused_add_rmsnorm_fwd_rstd", st)
    return out, residual_out, rstd


def rmsnorm_bwd_workspace_bytes(M, N, dtype, flags=DGAMMA_AUTO):
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().rmsnorm_bwd_workspace_bytes(int(M), int(N), code, int(flags)))


# One workspace per (device, stream), reused by calls that pass none: calls on
# one stream run in order, so they never share it concurrently, and a call
# then allocates nothing.
_workspaces = {}


def _cached_workspace(device, need):
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _check_rstd(rstd, M, device):
    if rstd.dtype != torch.float32 or rstd.numel() != M or not rstd.is_contiguous() \
            or rstd.device != device:
        raise ValueError("rstd must be a contiguous float32 tensor of M elements on x's device")


def _bwd(fn, x, gamma, dy, dres, rstd, dx, dgamma_f32, dgamma, workspace, flags):
    dt = _code(x, fn)
    x2 = _rows(x, gamma, fn)
    M, N = x2.shape
    if dy.shape != x.shape or (dres is not None and dres.shape != x.shape):
        raise ValueError(f"{fn}: dy/dresidual_out must have x's shape")
    dx = torch.empty_like(x) if dx is None else dx
    dgamma_f32 = torch.empty(N, dtype=torch.float32, device=x.device) if dgamma_f32 is None \
        else dgamma_f32
    _same(fn, x, gamma, dy, dres, dx, dgamma)
    _check_rstd(rstd, M, x.device)
    if dgamma_f32.dtype != torch.float32 or dgamma_f32.numel() != N:
        raise ValueError(f"{fn}: dgamma_f32 must be float32 of N elements")
    if dgamma is not None and dgamma.numel() != N:
        raise ValueError(f"{fn}: dgamma must have N elements")
    need = rmsnorm_bwd_workspace_bytes(M, N, dt, flags)
    if workspace is None:
        workspace = _cached_workspace(x.device, need)
    if fn == "rmsnorm_bwd":
        st = _on_device(x.device, lambda: lib().rmsnorm_bwd(
            _p(x2), _p(gamma), _p(dy), _p(rstd), _p(dx), _p(dgamma_f32), _p(dgamma),
            _p(workspace), workspace.numel(), M, N, dt, int(flags), _stream(x.device)))
    else:
        st = _on_device(x.device, lambda: lib().fused_add_rmsnorm_bwd(
            _p(x2), _p(gamma), _p(dy), _p(dres), _p(rstd), _p(dx), _p(dgamma_f32), _p(dgamma),
            _p(workspace), workspace.numel(), M, N, dt, int(flags), _stream(x.device)))
    _raise_on(fn, st)
    return dx, dgamma_f32, dgamma


def rmsnorm_bwd(x, gamma, dy, rstd, dx=None, dgamma_f32=None, dgamma=None, workspace=None,
                flags=DGAMMA_AUTO):
    """Backward ([I769] Implementation plan, Math). Returns (dx, dgamma_f32, dgamma)."""
    return _bwd("rmsnorm_bwd", x, gamma, dy, None, rstd, dx, dgamma_f32, dgamma, workspace, flags)


def fused_add_rmsnorm_bwd(added, gamma, dy, dresidual_out, rstd, dx=None, dgamma_f32=None,
                          dgamma=None, workspace=None, flags=DGAMMA_AUTO):
    """Fused-add backward ([P800] fused-add commit). Returns (dx, dgamma_f32, dgamma);
    dx is also the gradient of the residual."""
    return _bwd("fused_add_rmsnorm_bwd", added, gamma, dy, dresidual_out, rstd, dx, dgamma_f32,
                dgamma, workspace, flags)


def layernorm_fwd_stats(x, gamma, beta, eps, y=None, mean=None, rstd=None):
    """LayerNorm forward that saves mean and rstd. beta may be None (zeros).
    Returns (y, mean, rstd)."""
    fn = "layernorm_fwd_stats"
    dt = _code(x, fn)
    x2 = _rows(x, gamma, fn)
    M, N = x2.shape
    if beta is not None and (beta.dim() != 1 or beta.numel() != N):
        raise ValueError(f"{fn}: beta must have N={N} elements")
    y = torch.empty_like(x) if y is None else y
    mean = torch.empty(M, dtype=torch.float32, device=x.device) if mean is None else mean
    rstd = torch.empty(M, dtype=torch.float32, device=x.device) if rstd is None else rstd
    _same(fn, x, gamma, beta, y)
    _check_rstd(mean, M, x.device)
    _check_rstd(rstd, M, x.device)
    st = _on_device(x.device, lambda: lib().layernorm_fwd_stats(
        _p(x2), _p(gamma), _p(beta), _p(y), _p(mean), _p(rstd), M, N, float(eps), dt, _stream(x.device)))
    _raise_on(fn, st)
    return y, mean, rstd


def layernorm_bwd_workspace_bytes(M, N, dtype, flags=DGAMMA_AUTO):
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().layernorm_bwd_workspace_bytes(int(M), int(N), code, int(flags)))


def layernorm_bwd(x, gamma, dy, mean, rstd, dx=None, dgamma_f32=None, dbeta_f32=None, dgamma=None,
                  dbeta=None, workspace=None, flags=DGAMMA_AUTO):
    """LayerNorm backward. Returns (dx, dgamma_f32, dbeta_f32, dgamma, dbeta)."""
    fn = "layernorm_bwd"
    dt = _code(x, fn)
    x2 = _rows(x, gamma, fn)
    M, N = x2.shape
    if dy.shape != x.shape:
        raise ValueError(f"{fn}: dy must have x's shape")
    dx = torch.empty_like(x) if dx is None else dx
    f32 = dict(dtype=torch.float32, device=x.device)
    dgamma_f32 = torch.empty(N, **f32) if dgamma_f32 is None else dgamma_f32
    dbeta_f32 = torch.empty(N, **f32) if dbeta_f32 is None else dbeta_f32
    _same(fn, x, gamma, dy, dx, dgamma, dbeta)
    _check_rstd(mean, M, x.device)
    _check_rstd(rstd, M, x.device)
    for name, t in (("dgamma_f32", dgamma_f32), ("dbeta_f32", dbeta_f32)):
        if t.dtype != torch.float32 or t.numel() != N:
            raise ValueError(f"{fn}: {name} must be float32 of N elements")
    for name, t in (("dgamma", dgamma), ("dbeta", dbeta)):
        if t is not None and t.numel() != N:
            raise ValueError(f"{fn}: {name} must have N elements")
    need = layernorm_bwd_workspace_bytes(M, N, dt, flags)
    if workspace is None:
        workspace = _cached_workspace(x.device, need)
    st = _on_device(x.device, lambda: lib().layernorm_bwd(
        _p(x2), _p(gamma), _p(dy), _p(mean), _p(rstd), _p(dx), _p(dgamma_f32), _p(dbeta_f32), _p(dgamma),
        _p(dbeta), _p(workspace), workspace.numel(), M, N, dt, int(flags), _stream(x.device)))
    _raise_on(fn, st)
    return dx, dgamma_f32, dbeta_f32, dgamma, dbeta


from .autograd import (FusedAddRMSNormFunction, LayerNormFunction, RMSNormFunction,  # noqa: E402,F401
                       fused_add_rmsnorm, layer_norm, rmsnorm)
