"""GPU parity on tensors of more than 4 GiB, where the byte offsets of rows
pass 2^32.

Inputs: m0 distinct seeded rows (the named workloads' distributions),
repeated down the tensor on the GPU until one tensor passes 4.25 GiB. A row's
outputs (y, rstd, residual_out, dx; LayerNorm's mean) depend on that row and
the weights alone, and the library forms every row the same way, so each
repetition must equal the first bit for bit; the first m0 rows are held to
the oracle at the usual tolerances (y and dx normwise and one ulp per
element, rstd 1e-5 per element, residual_out bit-exact). The weight gradients
sum over all M rows: reps times the oracle's sum over the m0 rows, held to
1e-4 * sqrt(M) normwise and, column by column, to the fp32 summation bound.

Math: FlyDSL issue #769 ("[Feature] Add rmsnorm backward (+ forward saves
rstd) ..."), Implementation plan: Math, and PR sequence (the LayerNorm
follow-up); FlyDSL PR #800 ("[rmsnorm] Add fused-add / residual backward
(PR 2/3, #769)"), fused-add commit.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_bwd_amd as R
import workloads
from parity_util import DEV, F64, assert_close, assert_sum_bound, rel, tol_dgamma

pytestmark = pytest.mark.gpu

T = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
BIG = int(4.25 * 2 ** 30)  # bytes one row tensor passes

CASES = [  # (op, N, dtype, distinct rows)
    ("plain", 8192, "bf16", 257),
    ("plain", 4096, "f32", 257),
    ("fused", 8192, "bf16", 257),
    ("layernorm", 8192, "bf16", 257),
    ("plain", 32768, "bf16", 31),    # long rows, 16-byte chunks
    ("fused", 32768, "bf16", 31),
    ("plain", 20001, "f16", 29),     # long rows, single elements
    ("plain", 24576, "bf16", 37),    # long rows, the next row loaded during the current one
    ("plain", 20000, "f32", 29),     # long rows, gamma held in registers
    ("layernorm", 24576, "bf16", 37),  # long rows, one read
]


def _reps(m0, N, dt):
    return -(-BIG // (m0 * N * T[dt].itemsize))


def _tile(t, reps):
    return t.to(DEV).repeat(reps, *([1] * (t.dim() - 1))).contiguous()


def _repeats_first(name, t, m0, reps):
    """Every block of m0 rows of t equals the first, bit for bit."""
    v = t.view(reps, m0, *t.shape[1:])
    assert torch.equal(v, v[:1].expand_as(v)), f"{name}: some repetition differs from the first"


def _check_rstd(rstd, r_ref, m0, reps):
    er = ((rstd[:m0].cpu().double() - r_ref.double()).abs() / r_ref.double().abs()).max().item()
    assert er <= 1e-5, f"rstd: error {er:.3g}"
    _repeats_first("rstd", rstd, m0, reps)


def _check_grad(name, got, ref_small, abs_small, reps, M):
    ref = ref_small * reps
    e = rel(got, ref)
    assert e <= tol_dgamma(M), f"{name}: error {e:.3g} > {tol_dgamma(M):.3g}"
    assert_sum_bound(name, got, ref, abs_small * reps, M)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _plain(N, dt, m0):
    reps = _reps(m0, N, dt)
    M = m0 * reps
    td = T[dt]
    w = workloads.custom("plain", m0, N, dt, 1e-6, seed=4242)
    d = workloads.make_inputs(w)
    x, g, dy = d["x"], d["gamma"], d["dy"]
    r_ref, y_ref = oracle.rmsnorm_fwd(x, g, 1e-6)
    dx_ref, dg_ref = oracle.rmsnorm_bwd(x, g, dy, r_ref)
    gg = g.to(DEV)
    xg = _tile(x, reps)
    print(f"  plain M={M} N={N} {dt}: {xg.numel() * td.itemsize / 2 ** 30:.2f} GiB a tensor", flush=True)
    y, rstd = R.rmsnorm_fwd_rstd(xg, gg, 1e-6)
    torch.cuda.synchronize()
    _check_rstd(rstd, r_ref, m0, reps)
    assert_close("y", y[:m0], y_ref, td)
    _repeats_first("y", y, m0, reps)
    del y, rstd
    _free()
    dyg = _tile(dy, reps)
    dx, dg32, dgt = R.rmsnorm_bwd(xg, gg, dyg, _tile(r_ref, reps), dgamma=torch.empty(N, dtype=td, device=DEV))
    torch.cuda.synchronize()
    assert_close("dx", dx[:m0], dx_ref, td)
    _repeats_first("dx", dx, m0, reps)
    abs_small = (dy.to(F64) * x.to(F64) * r_ref.to(F64)[:, None]).abs().sum(0)
    _check_grad("dgamma", dg32, dg_ref, abs_small, reps, M)
    assert torch.equal(dgt.cpu(), dg32.cpu().to(td))


def _fused(N, dt, m0):
    reps = _reps(m0, N, dt)
    M = m0 * reps
    td = T[dt]
    w = workloads.custom("fused", m0, N, dt, 1e-6, seed=4243)
    d = workloads.make_inputs(w)
    x, res, g, dy, dres = d["x"], d["residual"], d["gamma"], d["dy"], d["dresidual_out"]
    a_ref, r_ref, o_ref = oracle.fused_add_rmsnorm_fwd(x, res, g, 1e-6)
    dx_ref, dg_ref = oracle.fused_add_rmsnorm_bwd(a_ref, g, dy, dres, r_ref)
    gg = g.to(DEV)
    xg, resg = _tile(x, reps), _tile(res, reps)
    print(f"  fused M={M} N={N} {dt}: {xg.numel() * td.itemsize / 2 ** 30:.2f} GiB a tensor", flush=True)
    out, res_out, rstd = R.fused_add_rmsnorm_fwd_rstd(xg, resg, gg, 1e-6)
    torch.cuda.synchronize()
    _check_rstd(rstd, r_ref, m0, reps)
    assert torch.equal(res_out[:m0].cpu(), a_ref), "residual_out not bit-exact"
    _repeats_first("residual_out", res_out, m0, reps)
    assert_close("out", out[:m0], o_ref, td)
    _repeats_first("out", out, m0, reps)
    del xg, resg, out, res_out, rstd
    _free()
    ag, dyg, dresg = _tile(a_ref, reps), _tile(dy, reps), _tile(dres, reps)
    dx, dg32, dgt = R.fused_add_rmsnorm_bwd(ag, gg, dyg, dresg, _tile(r_ref, reps),
                                            dgamma=torch.empty(N, dtype=td, device=DEV))
    torch.cuda.synchronize()
    assert_close("dx", dx[:m0], dx_ref, td)
    _repeats_first("dx", dx, m0, reps)
    abs_small = (dy.to(F64) * a_ref.to(F64) * r_ref.to(F64)[:, None]).abs().sum(0)
    _check_grad("dgamma", dg32, dg_ref, abs_small, reps, M)
    assert torch.equal(dgt.cpu(), dg32.cpu().to(td))


def _layernorm(N, dt, m0):
    reps = _reps(m0, N, dt)
    M = m0 * reps
    td = T[dt]
    gen = np.random.Generator(np.random.PCG64(4244))
    x = workloads.normal(gen, (m0, N), 0.5, 1.0, td).reshape(m0, N)
    g = workloads.normal(gen, (N,), 1.0, 0.1, td)
    b = workloads.normal(gen, (N,), 0.0, 0.1, td)
    dy = workloads.normal(gen, (m0, N), 0.0, 1e-2, td).reshape(m0, N)
    mean_ref, rstd_ref, y_ref = oracle.layernorm_fwd(x, g, b, 1e-6)
    dx_ref, dg_ref, db_ref = oracle.layernorm_bwd(x, g, dy, mean_ref, rstd_ref)
    gg, bg = g.to(DEV), b.to(DEV)
    xg = _tile(x, reps)
    print(f"  layernorm M={M} N={N} {dt}: {xg.numel() * td.itemsize / 2 ** 30:.2f} GiB a tensor", flush=True)
    y, mean, rstd = R.layernorm_fwd_stats(xg, gg, bg, 1e-6)
    torch.cuda.synchronize()
    _check_rstd(rstd, rstd_ref, m0, reps)
    scale = x.double().abs().amax(dim=1)
    em = ((mean[:m0].cpu().double() - mean_ref.double()).abs() / scale).max().item()
    assert em <= 1e-6, f"mean: error {em:.3g}"
    _repeats_first("mean", mean, m0, reps)
    assert_close("y", y[:m0], y_ref, td)
    _repeats_first("y", y, m0, reps)
    del y, mean, rstd
    _free()
    dyg = _tile(dy, reps)
    dx, dg32, db32, dgt, dbt = R.layernorm_bwd(xg, gg, dyg, _tile(mean_ref, reps), _tile(rstd_ref, reps),
                                               dgamma=torch.empty(N, dtype=td, device=DEV),
                                               dbeta=torch.empty(N, dtype=td, device=DEV))
    torch.cuda.synchronize()
    assert_close("dx", dx[:m0], dx_ref, td)
    _repeats_first("dx", dx, m0, reps)
    xc = x.to(F64) - mean_ref.to(F64)[:, None]
    _check_grad("dgamma", dg32, dg_ref, (dy.to(F64) * xc * rstd_ref.to(F64)[:, None]).abs().sum(0), reps, M)
    _check_grad("dbeta", db32, db_ref, dy.to(F64).abs().sum(0), reps, M)
    assert torch.equal(dgt.cpu(), dg32.cpu().to(td))
    assert torch.equal(dbt.cpu(), db32.cpu().to(td))


RUN = {"plain": _plain, "fused": _fused, "layernorm": _layernorm}


@pytest.mark.parametrize("op,N,dt,m0", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}" for c in CASES])
def test_tensors_past_4GiB(op, N, dt, m0):
    print("case big", op, N, dt, m0, flush=True)
    assert m0 * _reps(m0, N, dt) * N * T[dt].itemsize > 2 ** 32
    try:
        RUN[op](N, dt, m0)
    finally:
        _free()

