"""CPU oracle for RMSNorm forward (saving rstd), backward, and the fused-add
(prenorm residual) variants, and for LayerNorm (forward saving mean and rstd,
backward with dbias): a ctypes wrapper over ``oracle/oracle.c``.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The GPU library and
its Python binding never import it, and it imports nothing from them.

All tensors here are torch CPU tensors (plumbing only); every step of the
arithmetic runs in the C code, in fp64, single-threaded.

Pages cited, by title:
  [I769] FlyDSL issue #769, "[Feature] Add rmsnorm backward (+ forward saves
         rstd) to enable training / downstream (quack) integration"
  [P800] FlyDSL PR #800, "[rmsnorm] Add fused-add / residual backward
         (PR 2/3, #769)"
"""
import ctypes
import os

import torch

from . import build as _build

_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_lib = None


def lib():
    """Load ``liboracle.so``, compiling it with gcc first if it is not built."""
    global _lib
    if _lib is None:
        # ORACLE_LIB lets the mutation test load a deliberately broken copy
        path = os.environ.get("ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        P, I64, D, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int
        L.orc_decode.argtypes = [P, I64, I, P]
        L.orc_encode.argtypes = [P, I64, I, P]
        L.orc_encode_bits.argtypes = [P, I64, I, P]
        L.orc_rmsnorm_fwd.argtypes = [P, P, I, I64, I64, D, P, P]
        L.orc_fused_add_rmsnorm_fwd.argtypes = [P, P, P, I, I64, I64, D, P, P, P]
        L.orc_rmsnorm_bwd.argtypes = [P, P, P, P, I, I64, I64, P, P]
        L.orc_fused_add_rmsnorm_bwd.argtypes = [P, P, P, P, P, I, I64, I64, P, P]
        L.orc_layernorm_fwd.argtypes = [P, P, P, I, I64, I64, D, P, P, P]
        L.orc_layernorm_bwd.argtypes = [P, P, P, P, P, I, I64, I64, P, P, P]
        L.orc_elem_bytes.argtypes = [I]
        for name in ("orc_decode", "orc_encode", "orc_encode_bits", "orc_rmsnorm_fwd",
                     "orc_fused_add_rmsnorm_fwd", "orc_rmsnorm_bwd",
                     "orc_fused_add_rmsnorm_bwd", "orc_layernorm_fwd", "orc_layernorm_bwd",
                     "orc_elem_bytes"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _code(t):
    if t.dtype not in _DTYPES:
        raise TypeError(f"oracle: unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _ptr(t):
    if t is None:
        return None
    if t.device.type != "cpu" or not t.is_contiguous():
        raise ValueError("oracle: tensors must be contiguous CPU tensors")
    return ctypes.c_void_p(t.data_ptr())


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle: {what} rejected its arguments (rc={rc})")


def _shape(x, gamma):
    if x.dim() != 2 or gamma.dim() != 1 or x.shape[1] != gamma.shape[0]:
        raise ValueError("oracle: x must be (M, N) and gamma (N,)")
    if x.dtype != gamma.dtype:
        raise TypeError("oracle: x and gamma must share one dtype")
    return x.shape[0], x.shape[1]


def decode(t):
    """Exact widening of a float32/float16/bfloat16 tensor to float64."""
    t = t.contiguous()
    out = torch.empty(t.shape, dtype=torch.float64)
    _check(lib().orc_decode(_ptr(t), t.numel(), _code(t), _ptr(out)), "decode")
    return out


def encode(v, dtype):
    """Round a float64 tensor to ``dtype`` once, to nearest, ties to even."""
    v = v.to(torch.float64).contiguous()
    out = torch.empty(v.shape, dtype=dtype)
    _check(lib().orc_encode(_ptr(v), v.numel(), _DTYPES[dtype], _ptr(out)), "encode")
    return out


def encode_bits(v, dtype):
    """Bit patterns (as int64) of the generic encoder's rounding of ``v``."""
    v = v.to(torch.float64).contiguous()
    out = torch.empty(v.shape, dtype=torch.int32)
    _check(lib().orc_encode_bits(_ptr(v), v.numel(), _DTYPES[dtype], _ptr(out)),
           "encode_bits")
    return out.to(torch.int64) & 0xFFFFFFFF


def rmsnorm_fwd(x, gamma, eps, want_y=True):
    """Forward that saves rstd: returns (rstd float32 (M,), y float64 (M, N) or None).

    [I769] Implementation plan (the forward's rrms) and [P800] PR-1 commit
    (the saved rstd).
    """
    M, N = _shape(x, gamma)
    rstd = torch.empty(M, dtype=torch.float32)
    y = torch.empty((M, N), dtype=torch.float64) if want_y else None
    _check(lib().orc_rmsnorm_fwd(_ptr(x), _ptr(gamma), _code(x), M, N, float(eps),
                                 _ptr(rstd), _ptr(y)), "rmsnorm_fwd")
    return rstd, y


def fused_add_rmsnorm_fwd(x, residual, gamma, eps, want_out=True):
    """Fused-add forward: returns (added in x.dtype, rstd float32, out float64 or None).

    [P800] fused-add commit: added = x + residual is residual_out, and its
    per-row rstd is saved.
    """
    M, N = _shape(x, gamma)
    if residual.shape != x.shape or residual.dtype != x.dtype:
        raise ValueError("oracle: residual must match x")
    added = torch.empty((M, N), dtype=x.dtype)
    rstd = torch.empty(M, dtype=torch.float32)
    out = torch.empty((M, N), dtype=torch.float64) if want_out else None
    _check(lib().orc_fused_add_rmsnorm_fwd(_ptr(x), _ptr(residual), _ptr(gamma), _code(x),
                                           M, N, float(eps), _ptr(added), _ptr(rstd),
                                           _ptr(out)), "fused_add_rmsnorm_fwd")
    return added, rstd, out


def rmsnorm_bwd(x, gamma, dy, rstd, want_dx=True, want_dgamma=True):
    """Backward: returns (dx float64 (M, N) or None, dgamma float64 (N,) or None).

    [I769] Implementation plan, Math.
    """
    M, N = _shape(x, gamma)
    if dy.shape != x.shape or dy.dtype != x.dtype or rstd.shape != (M,) \
            or rstd.dtype != torch.float32:
        raise ValueError("oracle: dy must match x, rstd must be float32 (M,)")
    dx = torch.empty((M, N), dtype=torch.float64) if want_dx else None
    dg = torch.empty(N, dtype=torch.float64) if want_dgamma else None
    _check(lib().orc_rmsnorm_bwd(_ptr(x), _ptr(gamma), _ptr(dy), _ptr(rstd), _code(x),
                                 M, N, _ptr(dx), _ptr(dg)), "rmsnorm_bwd")
    return dx, dg


def fused_add_rmsnorm_bwd(added, gamma, dy, dresidual_out, rstd, want_dx=True,
                          want_dgamma=True):
    """Fused-add backward: returns (dx == dresidual float64 or None, dgamma float64 or None).

    [P800] fused-add commit: the plain backward over added, plus
    dresidual_out (None means zeros).
    """
    M, N = _shape(added, gamma)
    if dy.shape != added.shape or dy.dtype != added.dtype or rstd.shape != (M,) \
            or rstd.dtype != torch.float32:
        raise ValueError("oracle: dy must match added, rstd must be float32 (M,)")
    if dresidual_out is not None and (dresidual_out.shape != added.shape
                                      or dresidual_out.dtype != added.dtype):
        raise ValueError("oracle: dresidual_out must match added")
    dx = torch.empty((M, N), dtype=torch.float64) if want_dx else None
    dg = torch.empty(N, dtype=torch.float64) if want_dgamma else None
    _check(lib().orc_fused_add_rmsnorm_bwd(_ptr(added), _ptr(gamma), _ptr(dy),
                                           _ptr(dresidual_out), _ptr(rstd), _code(added),
                                           M, N, _ptr(dx), _ptr(dg)), "fused_add_rmsnorm_bwd")
    return dx, dg


def layernorm_fwd(x, gamma, beta, eps, want_y=True):
    """LayerNorm forward that saves its statistics: returns (mean float32
    (M,), rstd float32 (M,), y float64 (M, N) or None). beta may be None.

    [I769] PR sequence and status updates: the forward saves mean and rstd.
    """
    M, N = _shape(x, gamma)
    if beta is not None and (beta.shape != gamma.shape or beta.dtype != gamma.dtype):
        raise ValueError("oracle: beta must match gamma")
    mean = torch.empty(M, dtype=torch.float32)
    rstd = torch.empty(M, dtype=torch.float32)
    y = torch.empty((M, N), dtype=torch.float64) if want_y else None
    _check(lib().orc_layernorm_fwd(_ptr(x), _ptr(gamma), _ptr(beta), _code(x), M, N,
                                   float(eps), _ptr(mean), _ptr(rstd), _ptr(y)), "layernorm_fwd")
    return mean, rstd, y


def layernorm_bwd(x, gamma, dy, mean, rstd, want_dx=True, want_dgamma=True, want_dbeta=True):
    """LayerNorm backward: returns (dx float64 (M, N), dgamma float64 (N,),
    dbeta float64 (N,)), each None when not wanted.

    [I769] PR sequence: the RMSNorm approach plus mean handling and dbias.
    """
    M, N = _shape(x, gamma)
    for t in (mean, rstd):
        if t.shape != (M,) or t.dtype != torch.float32:
            raise ValueError("oracle: mean and rstd must be float32 (M,)")
    if dy.shape != x.shape or dy.dtype != x.dtype:
        raise ValueError("oracle: dy must match x")
    dx = torch.empty((M, N), dtype=torch.float64) if want_dx else None
    dg = torch.empty(N, dtype=torch.float64) if want_dgamma else None
    db = torch.empty(N, dtype=torch.float64) if want_dbeta else None
    _check(lib().orc_layernorm_bwd(_ptr(x), _ptr(gamma), _ptr(dy), _ptr(mean), _ptr(rstd),
                                   _code(x), M, N, _ptr(dx), _ptr(dg), _ptr(db)), "layernorm_bwd")
    return dx, dg, db
