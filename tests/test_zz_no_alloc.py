"""rmsnorm_bwd_no_alloc, the backward entry point that allocates nothing,
against rmsnorm_bwd (the entry point it mirrors) through the C ABI.

The no-alloc call runs the same kernels with the library's static scratch as
its workspace, so for the same arguments its outputs must equal rmsnorm_bwd's
bit for bit (the default mode sums dgamma in a fixed order). Two calls in a
row, the second on a smaller problem, check that nothing carried in the
shared scratch from one call leaks into the next. A call that needs more
scratch than the static array holds is refused before anything is enqueued,
and the atomic mode, which needs only the scratch's header, runs at any N.

Math: FlyDSL issue #769 ("[Feature] Add rmsnorm backward (+ forward saves
rstd) ..."), Implementation plan: Math.
"""
import ctypes

import pytest
import torch

import oracle
import rmsnorm_bwd_amd as R
import workloads
from parity_util import DEV, assert_close, rel, tol_dgamma

pytestmark = pytest.mark.gpu

SCRATCH = 10  # RMSN_ERR_SCRATCH
P = ctypes.c_void_p


def _ptr(t):
    return None if t is None else P(t.data_ptr())


def no_alloc(x, g, dy, rstd, dx, dg32, dgt, M, N, dt, flags=R.DGAMMA_AUTO):
    """One call of the C entry point on torch's current stream."""
    stream = torch.cuda.current_stream().cuda_stream
    return R.lib().rmsnorm_bwd_no_alloc(_ptr(x), _ptr(g), _ptr(dy), _ptr(rstd), _ptr(dx), _ptr(dg32),
                                        _ptr(dgt), M, N, dt, flags, P(stream))


def _inputs(M, N, dtype, seed):
    w = workloads.custom("plain", M, N, dtype, 1e-6, seed=seed, dy_sigma=1e-2)
    d = workloads.make_inputs(w)
    r, _ = oracle.rmsnorm_fwd(d["x"], d["gamma"], w.eps, want_y=False)
    return w, d, r


def test_no_alloc_matches_rmsnorm_bwd_on_two_calls_in_a_row():
    code = {"bf16": R.BF16, "f32": R.F32, "f16": R.F16}
    # the 4096 x 4096 bf16 workload, then a smaller call that uses less of the
    # scratch and fewer workgroups; last, long rows whose partials fill the
    # scratch exactly (64 workgroups of 32768 columns)
    for M, N, dtype, seed in ((4096, 4096, "bf16", 1), (512, 2048, "bf16", 2), (300, 3000, "f32", 3),
                              (64, 32768, "bf16", 5)):
        print("case no_alloc", M, N, dtype, flush=True)
        w, d, r = _inputs(M, N, dtype, seed)
        T = w.torch_dtype
        x, g, dy, rstd = (t.to(DEV) for t in (d["x"], d["gamma"], d["dy"], r))
        ref_dx, ref_dg32, ref_dgt = R.rmsnorm_bwd(x, g, dy, rstd, dgamma=torch.empty(N, dtype=T, device=DEV))
        dx = torch.full_like(x, float("nan"))
        dg32 = torch.full((N,), float("nan"), device=DEV)
        dgt = torch.full((N,), float("nan"), dtype=T, device=DEV)
        st = no_alloc(x, g, dy, rstd, dx, dg32, dgt, M, N, code[dtype])
        torch.cuda.synchronize()
        assert st == 0, R.status_string(st)
        assert torch.equal(dx, ref_dx), "dx differs from rmsnorm_bwd"
        assert torch.equal(dg32, ref_dg32), "dgamma_f32 differs from rmsnorm_bwd"
        assert torch.equal(dgt, ref_dgt), "dgamma differs from rmsnorm_bwd"
        dx_ref, dg_ref = oracle.rmsnorm_bwd(d["x"], d["gamma"], d["dy"], r)
        assert_close("dx", dx, dx_ref, T)
        assert rel(dg32, dg_ref) <= tol_dgamma(M)


def test_no_alloc_refuses_more_scratch_than_it_holds_and_runs_atomic_mode():
    print("case no_alloc 256 x 16384 bf16", flush=True)
    M, N = 256, 16384
    assert R.rmsnorm_bwd_workspace_bytes(M, N, R.BF16) > 256 + 256 * 8192 * 4
    w, d, r = _inputs(M, N, "bf16", 4)
    x, g, dy, rstd = (t.to(DEV) for t in (d["x"], d["gamma"], d["dy"], r))
    dx = torch.full_like(x, 7.0)
    dg32 = torch.full((N,), 7.0, device=DEV)
    assert no_alloc(x, g, dy, rstd, dx, dg32, None, M, N, R.BF16) == SCRATCH
    torch.cuda.synchronize()
    assert bool((dx == 7.0).all()) and bool((dg32 == 7.0).all()), "a refused call wrote its outputs"
    st = no_alloc(x, g, dy, rstd, dx, dg32, None, M, N, R.BF16, flags=R.DGAMMA_ATOMIC)
    torch.cuda.synchronize()
    assert st == 0, R.status_string(st)
    ref_dx, ref_dg32, _ = R.rmsnorm_bwd(x, g, dy, rstd, flags=R.DGAMMA_ATOMIC)
    torch.cuda.synchronize()
    assert torch.equal(dx, ref_dx)
    assert rel(dg32, ref_dg32.cpu().double()) <= 1e-6
    dx_ref, dg_ref = oracle.rmsnorm_bwd(d["x"], d["gamma"], d["dy"], r)
    assert_close("dx", dx, dx_ref, torch.bfloat16)
    assert rel(dg32, dg_ref) <= tol_dgamma(M)
