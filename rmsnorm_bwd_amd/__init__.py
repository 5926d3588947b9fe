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
import threading
from collections import OrderedDict

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librmsnorm_mi355x.so")

F32, F16, BF16 = 0, 1, 2
DGAMMA_AUTO, DGAMMA_DETERMINISTIC, DGAMMA_ATOMIC, DGAMMA_ONE_BLOCK, CHECK_DEVICE = 0, 1, 2, 3, 4
MAX_N = 32768
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
        L.rmsnorm_bwd_no_alloc.argtypes = [P, P, P, P, P, P, P, I64, I64, I, U, P]
        L.layernorm_fwd_stats.argtypes = [P, P, P, P, P, P, I64, I64, F, I, P]
        L.layernorm_bwd_workspace_bytes.argtypes = [I64, I64, I, U]
        L.layernorm_bwd_workspace_bytes.restype = SZ
        L.layernorm_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, P, SZ, I64, I64, I, U, P]
        L.rmsnorm_fwd_rstd_strided.argtypes = [P, I64, P, P, I64, P, I64, I64, F, I, P]
        L.fused_add_rmsnorm_fwd_rstd_strided.argtypes = [P, I64, P, I64, P, P, I64, P, I64, P, I64, I64,
                                                         F, I, P]
        L.rmsnorm_bwd_strided.argtypes = [P, I64, P, P, I64, P, P, I64, P, P, P, SZ, I64, I64, I, U, P]
        L.fused_add_rmsnorm_bwd_strided.argtypes = [P, I64, P, P, I64, P, I64, P, P, I64, P, P, P, SZ,
                                                    I64, I64, I, U, P]
        L.layernorm_fwd_stats_strided.argtypes = [P, I64, P, P, P, I64, P, P, I64, I64, F, I, P]
        L.layernorm_bwd_strided.argtypes = [P, I64, P, P, I64, P, P, P, I64, P, P, P, P, P, SZ, I64,
                                            I64, I, U, P]
        L.rmsn_status_string.argtypes = [I]
        L.rmsn_status_string.restype = ctypes.c_char_p
        for fn in ("rmsnorm_fwd_rstd", "fused_add_rmsnorm_fwd_rstd", "rmsnorm_bwd",
                   "fused_add_rmsnorm_bwd", "rmsnorm_bwd_no_alloc", "layernorm_fwd_stats", "layernorm_bwd",
                   "rmsnorm_fwd_rstd_strided", "fused_add_rmsnorm_fwd_rstd_strided",
                   "rmsnorm_bwd_strided", "fused_add_rmsnorm_bwd_strided",
                   "layernorm_fwd_stats_strided", "layernorm_bwd_strided"):
            getattr(L, fn).restype = I
        _lib = L
    return _lib


def status_string(status):
    return lib().rmsn_status_string(int(status)).decode()


def _raise_on(fn, status):
    if status != 0:
        raise RmsnError(fn, status, status_string(status))


def _p(t):
    # an int (or None for NULL): ctypes converts it through the declared
    # c_void_p argument type
    return None if t is None else t.data_ptr()


# torch's raw accessors of the current stream and device when it has them:
# the same values as torch.cuda.current_stream(d).cuda_stream and
# torch.cuda.current_device(), without building Python objects on every call
_raw_stream_fn = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_raw_device_fn = getattr(torch._C, "_cuda_getDevice", None)


def _raw_stream(device):
    """The current HIP stream of `device`, as an integer handle."""
    if _raw_stream_fn is not None:
        return _raw_stream_fn(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _cur_dev():
    if _raw_device_fn is not None and torch.cuda.is_initialized():
        return _raw_device_fn()
    return torch.cuda.current_device()


def _stream(device):
    return _raw_stream(device)


def _on_device(device, fn, *args):
    """Call fn with `device` current (the library launches on the current
    device, as the pages' device guard requires), switching only if needed."""
    if device.index == _cur_dev():
        return fn(*args)
    with torch.cuda.device(device):
        return fn(*args)


def _vec(t, N, name, what):
    """Check a 1-D per-column tensor (gamma, beta, their gradients)."""
    if t.dim() != 1 or t.numel() != N or not t.is_contiguous():
        raise ValueError(f"{name}: {what} must be a contiguous 1-D tensor of N={N} elements")


def _view(t, N, name, what):
    """(M, ld) of a row tensor: its last dimension is the row (N elements at
    unit stride) and its leading dimensions must collapse into one row index
    with a single stride ld (a contiguous tensor, or a slice or column block
    of wider rows). Anything else is refused; the caller can copy it."""
    if t.dim() == 0 or t.shape[-1] != N:
        raise ValueError(f"{name}: {what} must have rows of N={N} elements")
    if t.is_contiguous():
        return t.numel() // N, N
    if N > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name}: {what} must have unit stride along its rows")
    lead = [(sz, st) for sz, st in zip(t.shape[:-1], t.stride()[:-1]) if sz != 1]
    M = 1
    for sz, _ in lead:
        M *= sz
    if not lead:
        return M, N
    for (sz, st), (sz2, st2) in zip(lead[:-1], lead[1:]):
        if st != st2 * sz2:
            raise ValueError(f"{name}: {what}'s leading dimensions do not form one row stride")
    ld = lead[-1][1]
    if ld < N:
        raise ValueError(f"{name}: {what}'s rows overlap (row stride {ld} < N={N})")
    return M, ld


def _rows(x, gamma, name):
    """(M, N, ldx) of x with the pages' guards: last dim == len(gamma), one dtype."""
    if gamma.dim() != 1:
        raise ValueError(f"{name}: gamma must be 1-D")
    if x.shape[-1] != gamma.shape[0]:
        raise ValueError(f"{name}: x.shape[-1]={x.shape[-1]} != len(gamma)={gamma.shape[0]}")
    N = gamma.shape[0]
    _vec(gamma, N, name, "gamma")
    M, ld = _view(x, N, name, "x")
    return M, N, ld


def _didx(device):
    """A device's index as Tensor.get_device() gives it (-1 off the GPU)."""
    return -1 if device.index is None or device.type != "cuda" else device.index


def _same(name, ref, *ts):
    dtype, dev = ref.dtype, ref.get_device()  # device index (-1 on the host)
    for t in ts:
        if t is None:
            continue
        if t.dtype != dtype:
            raise TypeError(f"{name}: dtype mismatch {t.dtype} vs {dtype}")
        if t.get_device() != dev:
            raise ValueError(f"{name}: tensors on different devices")


def _ld(t, shape, N, name, what):
    """Row stride of a row tensor that must have x's shape (None: N)."""
    if t is None:
        return N
    if t.is_contiguous() and t.shape == shape:
        return N
    if t.shape != shape:
        raise ValueError(f"{name}: {what} must have x's shape")
    return _view(t, N, name, what)[1]


def _code(t, name):
    if t.dtype not in _DTYPE_CODE:
        raise TypeError(f"{name}: unsupported dtype {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: tensors must be on a GPU")
    return _DTYPE_CODE[t.dtype]


def rmsnorm_fwd_rstd(x, gamma, eps, y=None, rstd=None):
    """Forward that saves rstd ([I769] Scope/tasks item 2). Returns (y, rstd).
    Row tensors may be views with one row stride (the *_strided entry point)."""
    fn = "rmsnorm_fwd_rstd"
    dt = _code(x, fn)
    M, N, ldx = _rows(x, gamma, fn)
    y = torch.empty(x.shape, dtype=x.dtype, device=x.device) if y is None else y
    rstd = torch.empty(M, dtype=torch.float32, device=x.device) if rstd is None else rstd
    _same(fn, x, gamma, y)
    ldy = _ld(y, x.shape, N, fn, "y")
    _check_rstd(rstd, M, x.device)
    if ldx == N and ldy == N:
        call = lambda: lib().rmsnorm_fwd_rstd(  # noqa: E731
            _p(x), _p(gamma), _p(y), _p(rstd), M, N, float(eps), dt, _stream(x.device))
    else:
        call = lambda: lib().rmsnorm_fwd_rstd_strided(  # noqa: E731
            _p(x), ldx, _p(gamma), _p(y), ldy, _p(rstd), M, N, float(eps), dt, _stream(x.device))
    _raise_on(fn, _on_device(x.device, call))
    return y, rstd


def fused_add_rmsnorm_fwd_rstd(x, residual, gamma, eps, out=None, residual_out=None, rstd=None):
    """Fused-add forward ([P800] fused-add commit). Returns (out, residual_out, rstd)."""
    fn = "fused_add_rmsnorm_fwd_rstd"
    dt = _code(x, fn)
    M, N, ldx = _rows(x, gamma, fn)
    out = torch.empty(x.shape, dtype=x.dtype, device=x.device) if out is None else out
    residual_out = torch.empty(x.shape, dtype=x.dtype, device=x.device) if residual_out is None \
        else residual_out
    rstd = torch.empty(M, dtype=torch.float32, device=x.device) if rstd is None else rstd
    _same(fn, x, residual, gamma, out, residual_out)
    ldr = _ld(residual, x.shape, N, fn, "residual")
    ldo = _ld(out, x.shape, N, fn, "out")
    ldro = _ld(residual_out, x.shape, N, fn, "residual_out")
    _check_rstd(rstd, M, x.device)
    if ldx == ldr == ldo == ldro == N:
        call = lambda: lib().fused_add_rmsnorm_fwd_rstd(  # noqa: E731
            _p(x), _p(residual), _p(gamma), _p(out), _p(residual_out), _p(rstd), M, N, float(eps), dt,
            _stream(x.device))
    else:
        call = lambda: lib().fused_add_rmsnorm_fwd_rstd_strided(  # noqa: E731
            _p(x), ldx, _p(residual), ldr, _p(gamma), _p(out), ldo, _p(residual_out), ldro, _p(rstd),
            M, N, float(eps), dt, _stream(x.device))
    _raise_on(fn, _on_device(x.device, call))
    return out, residual_out, rstd


_ws_bytes = {}
_WS_BYTES_MAX = 4096  # remembered answers; forgotten all at once past this many


def _ws_query(entry, M, N, dtype, flags):
    """The library's workspace answer, remembered per arguments (it depends
    on nothing else)."""
    code = _DTYPE_CODE[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    key = (entry, M, N, code, flags)
    b = _ws_bytes.get(key)
    if b is None:
        b = int(getattr(lib(), entry)(int(M), int(N), code, int(flags)))
        if len(_ws_bytes) >= _WS_BYTES_MAX:
            _ws_bytes.clear()
        _ws_bytes[key] = b
    return b


def rmsnorm_bwd_workspace_bytes(M, N, dtype, flags=DGAMMA_AUTO):
    return _ws_query("rmsnorm_bwd_workspace_bytes", M, N, dtype, flags)


# One workspace per (device, stream), reused by calls that pass none: calls on
# one stream run in order, so they never share it concurrently, and a call
# then allocates nothing. At most _WS_STREAMS streams keep one, the least
# recently used giving its up first (a program that creates streams per step
# would otherwise keep a workspace for every stream it ever used). Dropping
# one is safe while eager work that uses it is still queued: torch's caching
# allocator hands a freed block only to later allocations on the stream that
# allocated it, which run after that work.
#
# A call made while its stream is being captured into a HIP graph never uses
# this cache: the graph bakes the workspace's address into its kernels and
# replays them long after the call returns, when a cached buffer may have been
# replaced and its memory handed to someone else. Such a call gets a buffer of
# its own from the graph's private memory pool instead, which torch keeps for
# as long as the graph exists and reuses only for later work of the same
# capture, in stream order.
_workspaces = OrderedDict()
_WS_STREAMS = 16


_workspaces_lock = threading.Lock()  # torch runs backward passes on per-device threads
_capturing = torch.cuda.is_current_stream_capturing


def _is_capturing(device):
    """Whether the current stream of `device` is being captured into a graph."""
    if device.type != "cuda":
        return False
    if device.index == _cur_dev():
        return _capturing()
    with torch.cuda.device(device):
        return _capturing()


def _cached_workspace(device, need, stream):
    if _is_capturing(device):
        return torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    key = (device.index, stream)
    with _workspaces_lock:
        ws = _workspaces.get(key)
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
            _workspaces[key] = ws
        _workspaces.move_to_end(key)
        while len(_workspaces) > _WS_STREAMS:
            _workspaces.popitem(last=False)
        return ws


def _f32_vec(t, N, device, fn, name):
    """A float32 per-column output (dgamma_f32, dbeta_f32) on x's device."""
    if t.dtype != torch.float32:
        raise ValueError(f"{fn}: {name} must be float32")
    if t.get_device() != _didx(device):
        raise ValueError(f"{fn}: {name} must be on x's device")
    _vec(t, N, fn, name)


def _workspace(workspace, need, device, fn, stream):
    """(pointer, bytes) of the caller's workspace, or of the cached one."""
    if workspace is None:
        workspace = _cached_workspace(device, need, stream)
    elif workspace.get_device() != _didx(device) or not workspace.is_contiguous():
        raise ValueError(f"{fn}: workspace must be a contiguous tensor on x's device")
    return _p(workspace), workspace.numel() * workspace.element_size()


def _check_rstd(rstd, M, device):
    if rstd.dtype != torch.float32 or rstd.numel() != M or not rstd.is_contiguous() \
            or rstd.get_device() != _didx(device):
        raise ValueError("rstd must be a contiguous float32 tensor of M elements on x's device")


class BoundCall:
    """One backward call checked and marshalled once, for repeated launches
    over fixed buffers (a training step's static tensors, a timing loop).
    Calling it enqueues the same entry point with the same pointers on the
    device's stream that is current at that moment (so the call can also be
    captured into a HIP graph) and returns the output tensors. It keeps the
    tensors it was bound to alive; their storage must not be replaced (in-place
    writes to their values are what a loop does). Calls of one bound object on
    different streams must not overlap: they share its workspace."""

    __slots__ = ("_name", "_fn", "_args", "_dev", "outputs", "_keep")

    def __init__(self, name, fn, args, dev, outputs, keep):
        self._name, self._fn, self._args, self._dev = name, fn, args, dev
        self.outputs, self._keep = outputs, keep

    def __call__(self):
        _raise_on(self._name, _on_device(self._dev, self._fn, *self._args, _raw_stream(self._dev)))
        return self.outputs


def _bound_workspace(workspace, need, dev, fn):
    """The workspace a bound call owns: the caller's (checked for size now),
    or a new one of the size the library asks for."""
    if workspace is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if workspace.numel() * workspace.element_size() < need:
        raise RmsnError(fn, 5, "workspace missing or too small")
    return workspace


def _bwd(fn, x, gamma, dy, dres, rstd, dx, dgamma_f32, dgamma, workspace, flags, bind=False):
    dt = _code(x, fn)
    M, N, ldx = _rows(x, gamma, fn)
    dev, shape = x.device, x.shape
    dx = torch.empty(shape, dtype=x.dtype, device=dev) if dx is None else dx
    dgamma_f32 = torch.empty(N, dtype=torch.float32, device=dev) if dgamma_f32 is None \
        else dgamma_f32
    _same(fn, x, gamma, dy, dres, dx, dgamma)
    lddy = _ld(dy, shape, N, fn, "dy")
    ldr = _ld(dres, shape, N, fn, "dresidual_out")
    lddx = _ld(dx, shape, N, fn, "dx")
    _check_rstd(rstd, M, dev)
    _f32_vec(dgamma_f32, N, dev, fn, "dgamma_f32")
    if dgamma is not None:
        _vec(dgamma, N, fn, "dgamma")
    need = rmsnorm_bwd_workspace_bytes(M, N, dt, flags)
    st_ = None if bind else _stream(dev)
    if bind:
        workspace = _bound_workspace(workspace, need, dev, fn)
    ws, wsb = _workspace(workspace, need, dev, fn, st_)
    strided = not (ldx == lddy == ldr == lddx == N)
    if fn == "rmsnorm_bwd" and not strided:
        entry, args = "rmsnorm_bwd", (_p(x), _p(gamma), _p(dy), _p(rstd), _p(dx), _p(dgamma_f32),
                                      _p(dgamma), ws, wsb, M, N, dt, int(flags))
    elif fn == "rmsnorm_bwd":
        entry, args = "rmsnorm_bwd_strided", (_p(x), ldx, _p(gamma), _p(dy), lddy, _p(rstd), _p(dx), lddx,
                                              _p(dgamma_f32), _p(dgamma), ws, wsb, M, N, dt, int(flags))
    elif not strided:
        entry, args = "fused_add_rmsnorm_bwd", (_p(x), _p(gamma), _p(dy), _p(dres), _p(rstd), _p(dx),
                                                _p(dgamma_f32), _p(dgamma), ws, wsb, M, N, dt, int(flags))
    else:
        entry, args = "fused_add_rmsnorm_bwd_strided", (
            _p(x), ldx, _p(gamma), _p(dy), lddy, _p(dres), ldr, _p(rstd), _p(dx), lddx, _p(dgamma_f32),
            _p(dgamma), ws, wsb, M, N, dt, int(flags))
    f = getattr(lib(), entry)
    if bind:
        return BoundCall(fn, f, args, dev, (dx, dgamma_f32, dgamma),
                         (x, gamma, dy, dres, rstd, dx, dgamma_f32, dgamma, workspace))
    _raise_on(fn, _on_device(dev, f, *args, st_))
    return dx, dgamma_f32, dgamma


def rmsnorm_bwd(x, gamma, dy, rstd, dx=None, dgamma_f32=None, dgamma=None, workspace=None,
                flags=DGAMMA_AUTO):
    """Backward ([I769] Implementation plan, Math). Returns (dx, dgamma_f32, dgamma)."""
    return _bwd("rmsnorm_bwd", x, gamma, dy, None, rstd, dx, dgamma_f32, dgamma, workspace, flags)


def rmsnorm_bwd_no_alloc(x, gamma, dy, rstd, dx, dgamma_f32, dgamma=None, flags=DGAMMA_AUTO):
    """rmsnorm_bwd over caller-given outputs with the library's static scratch
    as its workspace (no device allocation by the library or by this
    binding). Calls that overlap on one GPU share that scratch and race.
    Contiguous rows only. Returns (dx, dgamma_f32, dgamma)."""
    fn = "rmsnorm_bwd_no_alloc"
    dt = _code(x, fn)
    M, N, ldx = _rows(x, gamma, fn)
    _same(fn, x, gamma, dy, dx, dgamma)
    if ldx != N or _ld(dy, x.shape, N, fn, "dy") != N or _ld(dx, x.shape, N, fn, "dx") != N:
        raise ValueError(f"{fn}: row tensors must be contiguous")
    _check_rstd(rstd, M, x.device)
    _f32_vec(dgamma_f32, N, x.device, fn, "dgamma_f32")
    if dgamma is not None:
        _vec(dgamma, N, fn, "dgamma")
    call = lambda: lib().rmsnorm_bwd_no_alloc(  # noqa: E731
        _p(x), _p(gamma), _p(dy), _p(rstd), _p(dx), _p(dgamma_f32), _p(dgamma), M, N, dt, int(flags),
        _stream(x.device))
    _raise_on(fn, _on_device(x.device, call))
    return dx, dgamma_f32, dgamma


def fused_add_rmsnorm_bwd(added, gamma, dy, dresidual_out, rstd, dx=None, dgamma_f32=None,
                          dgamma=None, workspace=None, flags=DGAMMA_AUTO):
    """Fused-add backward ([P800] fused-add commit). Returns (dx, dgamma_f32, dgamma);
    dx is also the gradient of the residual."""
    return _bwd("fused_add_rmsnorm_bwd", added, gamma, dy, dresidual_out, rstd, dx, dgamma_f32,
                dgamma, workspace, flags)


def bind_rmsnorm_bwd(x, gamma, dy, rstd, dx=None, dgamma_f32=None, dgamma=None, workspace=None,
                     flags=DGAMMA_AUTO):
    """rmsnorm_bwd's checks and marshalling done once: returns a BoundCall
    whose call enqueues the backward and returns (dx, dgamma_f32, dgamma)."""
    return _bwd("rmsnorm_bwd", x, gamma, dy, None, rstd, dx, dgamma_f32, dgamma, workspace, flags,
                bind=True)


def bind_fused_add_rmsnorm_bwd(added, gamma, dy, dresidual_out, rstd, dx=None, dgamma_f32=None,
                               dgamma=None, workspace=None, flags=DGAMMA_AUTO):
    """fused_add_rmsnorm_bwd bound once (see bind_rmsnorm_bwd)."""
    return _bwd("fused_add_rmsnorm_bwd", added, gamma, dy, dresidual_out, rstd, dx, dgamma_f32, dgamma,
                workspace, flags, bind=True)


def layernorm_fwd_stats(x, gamma, beta, eps, y=None, mean=None, rstd=None):
    """LayerNorm forward that saves mean and rstd. beta may be None (zeros).
    Returns (y, mean, rstd)."""
    fn = "layernorm_fwd_stats"
    dt = _code(x, fn)
    M, N, ldx = _rows(x, gamma, fn)
    if beta is not None:
        _vec(beta, N, fn, "beta")
    y = torch.empty(x.shape, dtype=x.dtype, device=x.device) if y is None else y
    mean = torch.empty(M, dtype=torch.float32, device=x.device) if mean is None else mean
    rstd = torch.empty(M, dtype=torch.float32, device=x.device) if rstd is None else rstd
    _same(fn, x, gamma, beta, y)
    ldy = _ld(y, x.shape, N, fn, "y")
    _check_rstd(mean, M, x.device)
    _check_rstd(rstd, M, x.device)
    if ldx == ldy == N:
        call = lambda: lib().layernorm_fwd_stats(  # noqa: E731
            _p(x), _p(gamma), _p(beta), _p(y), _p(mean), _p(rstd), M, N, float(eps), dt, _stream(x.device))
    else:
        call = lambda: lib().layernorm_fwd_stats_strided(  # noqa: E731
            _p(x), ldx, _p(gamma), _p(beta), _p(y), ldy, _p(mean), _p(rstd), M, N, float(eps), dt,
            _stream(x.device))
    _raise_on(fn, _on_device(x.device, call))
    return y, mean, rstd


def layernorm_bwd_workspace_bytes(M, N, dtype, flags=DGAMMA_AUTO):
    return _ws_query("layernorm_bwd_workspace_bytes", M, N, dtype, flags)


def _ln_bwd(x, gamma, dy, mean, rstd, dx, dgamma_f32, dbeta_f32, dgamma, dbeta, workspace, flags, bind):
    fn = "layernorm_bwd"
    dt = _code(x, fn)
    M, N, ldx = _rows(x, gamma, fn)
    dev = x.device
    dx = torch.empty(x.shape, dtype=x.dtype, device=dev) if dx is None else dx
    f32 = dict(dtype=torch.float32, device=dev)
    dgamma_f32 = torch.empty(N, **f32) if dgamma_f32 is None else dgamma_f32
    dbeta_f32 = torch.empty(N, **f32) if dbeta_f32 is None else dbeta_f32
    _same(fn, x, gamma, dy, dx, dgamma, dbeta)
    lddy = _ld(dy, x.shape, N, fn, "dy")
    lddx = _ld(dx, x.shape, N, fn, "dx")
    _check_rstd(mean, M, dev)
    _check_rstd(rstd, M, dev)
    for name, t in (("dgamma_f32", dgamma_f32), ("dbeta_f32", dbeta_f32)):
        _f32_vec(t, N, dev, fn, name)
    for name, t in (("dgamma", dgamma), ("dbeta", dbeta)):
        if t is not None:
            _vec(t, N, fn, name)
    need = layernorm_bwd_workspace_bytes(M, N, dt, flags)
    st_ = None if bind else _stream(dev)
    if bind:
        workspace = _bound_workspace(workspace, need, dev, fn)
    ws, wsb = _workspace(workspace, need, dev, fn, st_)
    if ldx == lddy == lddx == N:
        entry, args = "layernorm_bwd", (_p(x), _p(gamma), _p(dy), _p(mean), _p(rstd), _p(dx), _p(dgamma_f32),
                                        _p(dbeta_f32), _p(dgamma), _p(dbeta), ws, wsb, M, N, dt, int(flags))
    else:
        entry, args = "layernorm_bwd_strided", (
            _p(x), ldx, _p(gamma), _p(dy), lddy, _p(mean), _p(rstd), _p(dx), lddx, _p(dgamma_f32),
            _p(dbeta_f32), _p(dgamma), _p(dbeta), ws, wsb, M, N, dt, int(flags))
    f = getattr(lib(), entry)
    outs = (dx, dgamma_f32, dbeta_f32, dgamma, dbeta)
    if bind:
        return BoundCall(fn, f, args, dev, outs, (x, gamma, dy, mean, rstd, *outs, workspace))
    _raise_on(fn, _on_device(dev, f, *args, st_))
    return outs


def layernorm_bwd(x, gamma, dy, mean, rstd, dx=None, dgamma_f32=None, dbeta_f32=None, dgamma=None,
                  dbeta=None, workspace=None, flags=DGAMMA_AUTO):
    """LayerNorm backward. Returns (dx, dgamma_f32, dbeta_f32, dgamma, dbeta)."""
    return _ln_bwd(x, gamma, dy, mean, rstd, dx, dgamma_f32, dbeta_f32, dgamma, dbeta, workspace, flags,
                   bind=False)


def bind_layernorm_bwd(x, gamma, dy, mean, rstd, dx=None, dgamma_f32=None, dbeta_f32=None, dgamma=None,
                       dbeta=None, workspace=None, flags=DGAMMA_AUTO):
    """layernorm_bwd bound once (see bind_rmsnorm_bwd); a call returns
    (dx, dgamma_f32, dbeta_f32, dgamma, dbeta)."""
    return _ln_bwd(x, gamma, dy, mean, rstd, dx, dgamma_f32, dbeta_f32, dgamma, dbeta, workspace, flags,
                   bind=True)


from .autograd import (FusedAddRMSNormFunction, LayerNormFunction, RMSNormFunction,  # noqa: E402,F401
                       fused_add_rmsnorm, layer_norm, rmsnorm)
