"""Host-side checks of the C ABI library; no GPU needed and no kernel launched.

- the built library loads and exports every function include/*.h declares;
- argument validation returns the documented status before any HIP call
  (each case below breaks exactly one rule, and where a missed check could
  reach a launch, a second, later-checked rule is broken too, so no case can
  ever enqueue work on the fake addresses it passes);
- the workspace query is pure host arithmetic with the documented bounds.
"""
import ctypes
import glob
import os
import re

import pytest
import torch

import rmsnorm_bwd_amd as R

# These cases hand the library fake device addresses that validation must
# refuse. They only run where no GPU is visible, so that a validation gap can
# never turn into a launch on those addresses.
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake-address validation cases run on GPU-less hosts only")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL, SHAPE, DTYPE, EPS, WORKSPACE, FLAGS, DEVICE, HIP, ALIGN, SCRATCH = range(11)
A = 0x10000          # a 256-byte-aligned fake device address
P = ctypes.c_void_p


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = re.sub(r"^\s*#[^\n]*", "", text, flags=re.M)  # preprocessor lines
        for m in re.finditer(r"\b([A-Za-z_]\w*)\s*\(([^;{}]*)\)\s*;", text):
            names.append(m.group(1))
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"rmsnorm_fwd_rstd", "rmsnorm_bwd", "fused_add_rmsnorm_fwd_rstd",
            "fused_add_rmsnorm_bwd", "rmsnorm_bwd_workspace_bytes",
            "rmsn_status_string"} <= set(names)
    lib = ctypes.CDLL(R.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_status_strings():
    for s in range(11):
        assert R.status_string(s) and R.status_string(s) != "unknown status"
    assert R.status_string(99) == "unknown status"


def bwd(**kw):
    a = dict(x=A, gamma=A, dy=A, rstd=A, dx=A, dg32=A, dg=None, ws=A, wsb=0,
             M=4, N=64, dtype=R.BF16, flags=0)
    a.update(kw)
    return R.lib().rmsnorm_bwd(P(a["x"]), P(a["gamma"]), P(a["dy"]), P(a["rstd"]), P(a["dx"]),
                               P(a["dg32"]), P(a["dg"]), P(a["ws"]), a["wsb"], a["M"], a["N"],
                               a["dtype"], a["flags"], None)


def fused_bwd(**kw):
    a = dict(x=A, gamma=A, dy=A, dres=None, rstd=A, dx=A, dg32=A, dg=None, ws=A, wsb=0,
             M=4, N=64, dtype=R.BF16, flags=0)
    a.update(kw)
    return R.lib().fused_add_rmsnorm_bwd(P(a["x"]), P(a["gamma"]), P(a["dy"]), P(a["dres"]),
                                         P(a["rstd"]), P(a["dx"]), P(a["dg32"]), P(a["dg"]),
                                         P(a["ws"]), a["wsb"], a["M"], a["N"], a["dtype"],
                                         a["flags"], None)


def ln_bwd(**kw):
    a = dict(x=A, gamma=A, dy=A, mean=A, rstd=A, dx=A, dg32=A, db32=A, dg=None, db=None, ws=A,
             wsb=0, M=4, N=64, dtype=R.BF16, flags=0)
    a.update(kw)
    return R.lib().layernorm_bwd(P(a["x"]), P(a["gamma"]), P(a["dy"]), P(a["mean"]), P(a["rstd"]),
                                 P(a["dx"]), P(a["dg32"]), P(a["db32"]), P(a["dg"]), P(a["db"]),
                                 P(a["ws"]), a["wsb"], a["M"], a["N"], a["dtype"], a["flags"], None)


def fwd(**kw):
    a = dict(x=A, gamma=A, y=A, rstd=A, M=0, N=64, eps=1e-5, dtype=R.BF16)
    a.update(kw)
    return R.lib().rmsnorm_fwd_rstd(P(a["x"]), P(a["gamma"]), P(a["y"]), P(a["rstd"]), a["M"],
                                    a["N"], a["eps"], a["dtype"], None)


def fused_fwd(**kw):
    a = dict(x=A, res=A, gamma=A, out=A, res_out=A, rstd=A, M=0, N=64, eps=1e-5, dtype=R.BF16)
    if "y" in kw:
        kw["out"] = kw.pop("y")
    a.update(kw)
    return R.lib().fused_add_rmsnorm_fwd_rstd(P(a["x"]), P(a["res"]), P(a["gamma"]), P(a["out"]),
                                              P(a["res_out"]), P(a["rstd"]), a["M"], a["N"],
                                              a["eps"], a["dtype"], None)


# Every backward case leaves wsb = 0 (too small), and WORKSPACE is checked
# last: a validation gap would surface as WORKSPACE, never as a launch.
BWD_CASES = [
    ("bad dtype", dict(dtype=3), DTYPE),
    ("negative dtype", dict(dtype=-1), DTYPE),
    ("N = 0", dict(N=0), SHAPE),
    ("N too large", dict(N=R.MAX_N + 1), SHAPE),
    ("M < 0", dict(M=-1), SHAPE),
    ("M too large", dict(M=1 << 31), SHAPE),
    ("unknown flag", dict(flags=8), FLAGS),
    ("unknown high flag", dict(flags=16), FLAGS),
    ("gamma NULL", dict(gamma=None), NULL),
    ("dgamma_f32 NULL", dict(dg32=None), NULL),
    ("workspace NULL", dict(ws=None), NULL),
    ("x NULL", dict(x=None), NULL),
    ("dy NULL", dict(dy=None), NULL),
    ("rstd NULL", dict(rstd=None), NULL),
    ("dx NULL", dict(dx=None), NULL),
    ("x misaligned", dict(x=A + 1), ALIGN),
    ("f32 dx misaligned", dict(dx=A + 2, dtype=R.F32), ALIGN),
    ("rstd misaligned", dict(rstd=A + 2), ALIGN),
    ("dgamma misaligned", dict(dg=A + 1), ALIGN),
    ("workspace not 256-aligned", dict(ws=A + 16), ALIGN),
    ("workspace too small", dict(wsb=0), WORKSPACE),
]


@pytest.mark.parametrize("name,kw,want", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bwd_validation(name, kw, want):
    assert bwd(**kw) == want
    assert fused_bwd(**kw) == want
    assert ln_bwd(**kw) == want


def test_layernorm_bwd_validation_of_its_own_operands():
    assert ln_bwd(mean=None) == NULL
    assert ln_bwd(db32=None) == NULL
    assert ln_bwd(mean=A + 2) == ALIGN
    assert ln_bwd(db32=A + 2) == ALIGN
    assert ln_bwd(db=A + 1) == ALIGN
    # no rows: the mean may be absent; still refused for the workspace size
    assert ln_bwd(M=0, mean=None) == WORKSPACE
    for M, N, dt in ((4096, 4096, R.BF16), (512, 3000, R.F32)):
        need = R.layernorm_bwd_workspace_bytes(M, N, dt)
        assert ln_bwd(M=M, N=N, dtype=dt, wsb=need - 1) == WORKSPACE


def test_small_short_row_problems_run_in_one_block():
    """The default mode's measured rule: rows of at most 1024 elements and at
    most 8192 elements in all, or at most two rows of up to 8192 elements,
    run in one block that writes dgamma itself (no partials); anything
    larger uses per-block partials. The explicit modes ignore the rule."""
    q = R.rmsnorm_bwd_workspace_bytes
    for M, N in ((32, 256), (8, 1024), (1, 4096), (1, 16384), (64, 128), (2, 4096), (2, 8192)):
        assert q(M, N, R.BF16) == 256, (M, N)
        assert q(M, N, R.BF16, R.DGAMMA_ONE_BLOCK) == 256, (M, N)
        assert q(M, N, R.BF16, R.DGAMMA_DETERMINISTIC) > 256, (M, N)
    for M, N in ((33, 256), (9, 1024), (3, 4096), (5, 2048), (2, 16384), (2, 8200)):
        assert q(M, N, R.BF16) > 256, (M, N)
        assert q(M, N, R.BF16, R.DGAMMA_ONE_BLOCK) == 256, (M, N)


def test_layernorm_workspace_holds_two_partial_arrays():
    q, ql = R.rmsnorm_bwd_workspace_bytes, R.layernorm_bwd_workspace_bytes
    assert ql(4096, 4096, R.BF16) == 256 + 2 * 256 * 4096 * 4
    assert ql(4096, 4096, R.BF16, R.DGAMMA_ATOMIC) == 256
    assert ql(1, 4096, R.BF16) == 256
    for M in (1, 7, 5000):
        for N in (1, 255, 4096, 16384, 32768):
            assert ql(M, N, R.F32) - 256 == 2 * (q(M, N, R.F32) - 256)
    assert ql(4, 0, R.BF16) == 0 and ql(4, 64, 9) == 0


def test_bwd_workspace_one_byte_short():
    # everything valid except the size: one byte below the query is refused
    for M, N, dt in ((4096, 4096, R.BF16), (512, 3000, R.F32), (8, 256, R.F32)):
        need = R.rmsnorm_bwd_workspace_bytes(M, N, dt)
        assert bwd(M=M, N=N, dtype=dt, wsb=need - 1) == WORKSPACE


def test_fused_bwd_dres_misaligned():
    assert fused_bwd(dres=A + 1) == ALIGN


# Forward cases use M = 0 where they can (nothing is launched for no rows);
# the M > 0 cases also misalign y, which is checked after the NULL checks.
FWD_CASES = [
    ("bad dtype", dict(dtype=5), DTYPE),
    ("N = 0", dict(N=0), SHAPE),
    ("N too large", dict(N=R.MAX_N + 1), SHAPE),
    ("M < 0", dict(M=-3), SHAPE),
    ("eps NaN", dict(eps=float("nan")), EPS),
    ("eps negative", dict(eps=-1e-6), EPS),
    ("eps infinite", dict(eps=float("inf")), EPS),
    ("gamma NULL", dict(gamma=None), NULL),
    ("gamma misaligned", dict(gamma=A + 1), ALIGN),
    ("x NULL", dict(M=2, x=None, y=A + 1), NULL),
    ("y NULL", dict(M=2, y=None, x=A + 1), NULL),
    ("rstd NULL", dict(M=2, rstd=None, y=A + 1), NULL),
]


@pytest.mark.parametrize("name,kw,want", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_fwd_validation(name, kw, want):
    assert fwd(**kw) == want
    assert fused_fwd(**kw) == want


def test_fused_fwd_needs_residual():
    assert fused_fwd(M=2, res=None, out=A + 1) == NULL
    assert fused_fwd(M=2, res_out=None, out=A + 1) == NULL


def ln_fwd(**kw):
    a = dict(x=A, gamma=A, beta=None, y=A, mean=A, rstd=A, M=0, N=64, eps=1e-5, dtype=R.BF16)
    a.update(kw)
    return R.lib().layernorm_fwd_stats(P(a["x"]), P(a["gamma"]), P(a["beta"]), P(a["y"]),
                                       P(a["mean"]), P(a["rstd"]), a["M"], a["N"], a["eps"],
                                       a["dtype"], None)


@pytest.mark.parametrize("name,kw,want", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_layernorm_fwd_validation(name, kw, want):
    assert ln_fwd(**kw) == want


def test_layernorm_fwd_own_operands():
    assert ln_fwd(M=2, mean=None, y=A + 1) == NULL
    assert ln_fwd(beta=A + 1) == ALIGN
    assert ln_fwd(mean=A + 2) == ALIGN
    assert ln_fwd(M=0) == OK


def test_fwd_with_no_rows_is_ok_without_a_launch():
    assert fwd(M=0) == OK
    assert fused_fwd(M=0) == OK


def test_workspace_query():
    q = R.rmsnorm_bwd_workspace_bytes
    assert q(4, 0, R.BF16) == 0 and q(4, 64, 9) == 0 and q(-1, 64, R.BF16) == 0
    assert q(4, 64, R.BF16, flags=8) == 0
    # a single block writes dgamma itself: header only (the one-block mode at
    # any size)
    assert q(4096, 4096, R.BF16, R.DGAMMA_ONE_BLOCK) == 256
    # the deterministic mode always uses partials, a single block's included
    assert q(1, 4096, R.BF16, R.DGAMMA_DETERMINISTIC) == 256 + 4096 * 4
    assert q(1, 4096, R.BF16) == 256
    assert q(0, 4096, R.BF16) == 256
    # many rows: one fp32 partial row per block (at most 256 blocks), in the
    # deterministic and the default mode; the atomic mode needs none
    assert q(4096, 4096, R.BF16) == 256 + 256 * 4096 * 4
    assert q(4096, 4096, R.BF16, R.DGAMMA_DETERMINISTIC) == 256 + 256 * 4096 * 4
    assert q(4096, 4096, R.BF16, R.DGAMMA_ATOMIC) == 256
    for M in (1, 7, 100, 5000, 1 << 20):
        for N in (1, 3, 255, 3000, 4096, 16384, 16385, 20000, 32768):
            for dt in (R.F32, R.F16, R.BF16):
                v = q(M, N, dt)
                assert 256 <= v <= 256 + 256 * (-(-N // 16) * 16) * 4


# --------------------------------------------------------------------------
# Strided twins: row strides are validated like shapes
# --------------------------------------------------------------------------

MAX_LD = 1 << 24


def bwd_strided(ldx=64, lddy=64, lddx=64, **kw):
    a = dict(x=A, gamma=A, dy=A, rstd=A, dx=A, dg32=A, dg=None, ws=A, wsb=0, M=4, N=64,
             dtype=R.BF16, flags=0)
    a.update(kw)
    return R.lib().rmsnorm_bwd_strided(P(a["x"]), ldx, P(a["gamma"]), P(a["dy"]), lddy,
                                       P(a["rstd"]), P(a["dx"]), lddx, P(a["dg32"]), P(a["dg"]),
                                       P(a["ws"]), a["wsb"], a["M"], a["N"], a["dtype"],
                                       a["flags"], None)


def fused_bwd_strided(ldx=64, lddy=64, ldres=64, lddx=64, dres=A):
    return R.lib().fused_add_rmsnorm_bwd_strided(P(A), ldx, P(A), P(A), lddy, P(dres), ldres,
                                                 P(A), P(A), lddx, P(A), None, P(A), 0, 4, 64,
                                                 R.BF16, 0, None)


def ln_bwd_strided(ldx=64, lddy=64, lddx=64):
    return R.lib().layernorm_bwd_strided(P(A), ldx, P(A), P(A), lddy, P(A), P(A), P(A), lddx,
                                         P(A), P(A), None, None, P(A), 0, 4, 64, R.BF16, 0, None)


@pytest.mark.parametrize("which", ["ldx", "lddy", "lddx"])
@pytest.mark.parametrize("ld,want", [(63, SHAPE), (0, SHAPE), (-64, SHAPE), (MAX_LD + 1, SHAPE),
                                     (64, WORKSPACE), (1000, WORKSPACE), (MAX_LD, WORKSPACE)])
def test_backward_row_strides(which, ld, want):
    # a valid stride is accepted and the call then stops at the (too small)
    # workspace, before any launch
    assert bwd_strided(**{which: ld}) == want
    assert ln_bwd_strided(**{which: ld}) == want
    assert fused_bwd_strided(**{which: ld}) == want


def test_fused_backward_dresidual_stride():
    assert fused_bwd_strided(ldres=10) == SHAPE
    # a NULL dresidual_out (zeros) has no stride to check
    assert fused_bwd_strided(ldres=10, dres=None) == WORKSPACE


def test_strides_do_not_matter_without_rows():
    assert bwd_strided(M=0, ldx=1, lddy=1, lddx=1) == WORKSPACE
    assert R.lib().rmsnorm_fwd_rstd_strided(P(A), 1, P(A), P(A), 1, P(A), 0, 64, 1e-5, R.BF16,
                                            None) == OK


def test_forward_row_strides():
    fs = R.lib().rmsnorm_fwd_rstd_strided
    assert fs(P(A), 63, P(A), P(A + 2), 64, P(A), 2, 64, 1e-5, R.BF16, None) == SHAPE
    assert fs(P(A), 64, P(A), P(A + 2), MAX_LD + 1, P(A), 2, 64, 1e-5, R.BF16, None) == SHAPE
    # valid strides: stops at the misaligned y, before any launch
    assert fs(P(A), 100, P(A), P(A + 1), 64, P(A), 2, 64, 1e-5, R.BF16, None) == ALIGN
    ff = R.lib().fused_add_rmsnorm_fwd_rstd_strided
    for bad in range(4):
        ld = [64, 64, 64, 64]
        ld[bad] = 10
        assert ff(P(A), ld[0], P(A), ld[1], P(A), P(A + 1), ld[2], P(A), ld[3], P(A), 2, 64, 1e-5,
                  R.BF16, None) == SHAPE
    fl = R.lib().layernorm_fwd_stats_strided
    assert fl(P(A), 10, P(A), None, P(A + 1), 64, P(A), P(A), 2, 64, 1e-5, R.BF16, None) == SHAPE
    assert fl(P(A), 64, P(A), None, P(A + 1), 64, P(A), P(A), 2, 64, 1e-5, R.BF16, None) == ALIGN


def no_alloc(**kw):
    a = dict(x=A, gamma=A, dy=A, rstd=A, dx=A, dg32=A, dg=None, M=256, N=16384, dtype=R.BF16, flags=0)
    a.update(kw)
    return R.lib().rmsnorm_bwd_no_alloc(P(a["x"]), P(a["gamma"]), P(a["dy"]), P(a["rstd"]), P(a["dx"]),
                                        P(a["dg32"]), P(a["dg"]), a["M"], a["N"], a["dtype"], a["flags"],
                                        None)


def test_no_alloc_refuses_before_any_hip_call():
    """The entry point without a workspace: a call needing more than its
    static scratch is refused with its own status, and arguments the
    backward rejects keep their statuses, all before any HIP call (every
    case is refused, so nothing can reach a launch on the fake addresses)."""
    limit = 256 + 256 * 8192 * 4
    assert R.rmsnorm_bwd_workspace_bytes(256, 16384, R.BF16) > limit
    assert R.rmsnorm_bwd_workspace_bytes(32768, 8192, R.BF16) <= limit
    assert no_alloc() == SCRATCH
    assert no_alloc(flags=R.DGAMMA_DETERMINISTIC) == SCRATCH
    assert no_alloc(dtype=3) == DTYPE
    assert no_alloc(N=0) == SHAPE
    assert no_alloc(N=R.MAX_N + 1) == SHAPE
    assert no_alloc(M=-1) == SHAPE
    assert no_alloc(flags=8) == FLAGS
    assert no_alloc(flags=16) == FLAGS
