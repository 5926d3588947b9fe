"""Pins of the CPU oracle's LayerNorm to things other than itself.

The LayerNorm forward (saving mean and rstd) and backward (dx, dgamma,
dbeta) are held against hand-derived worked examples (tests/golden),
float64 torch layer_norm autograd on the CPU, central finite differences of
the oracle's own forward, the shift invariance of the normalisation (each
row's dx sums to zero), the exact bias gradient, and the RMSNorm backward,
which it must equal on rows whose mean is zero and whose sum of dy * gamma
is zero. tests/test_oracle_mutants.py checks that these catch planted
mistakes.

Math being pinned: FlyDSL issue #769 ("[Feature] Add rmsnorm backward (+
forward saves rstd) ..."), PR sequence and status updates (the LayerNorm
follow-up: the RMSNorm approach plus mean handling and a bias gradient, the
forward saving mean and rstd), read as the textbook layer norm.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
F64 = torch.float64


def t64(a):
    return torch.tensor(a, dtype=F64)


def rel(a, b):
    a, b = torch.as_tensor(a, dtype=F64), torch.as_tensor(b, dtype=F64)
    den = b.abs().max().item()
    return (a - b).abs().max().item() / (den if den > 0 else 1.0)


def grid_values(gen, shape, scale_bits=6, lim=256):
    """float32 values k * 2^-scale_bits, |k| <= lim: sums of them are exact in
    fp64 and a small power-of-two perturbation stays exact in float32."""
    k = gen.integers(-lim, lim + 1, size=shape)
    return torch.tensor(k * 2.0 ** -scale_bits, dtype=torch.float32)


def _golden_cases():
    with open(os.path.join(HERE, "golden", "ln_closed_forms.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_golden_worked_examples(case, dtype):
    T = lambda k: torch.tensor(case[k], dtype=F64).to(dtype)
    beta = T("beta") if case["beta"] is not None else None
    x, gamma = T("x"), T("gamma")
    mean, rstd, y = oracle.layernorm_fwd(x, gamma, beta, case["eps"])
    dx, dg, db = oracle.layernorm_bwd(x, gamma, T("dy"), mean, rstd)
    assert torch.equal(mean.to(F64), t64(case["mean"]))
    assert torch.equal(rstd.to(F64), t64(case["rstd"]))
    assert torch.equal(y, t64(case["y"]))
    assert torch.equal(dx, t64(case["dx"]))
    assert torch.equal(dg, t64(case["dgamma"]))
    assert torch.equal(db, t64(case["dbeta"]))


def _inputs(seed, M, N, dtype, with_beta=True):
    gen = np.random.Generator(np.random.PCG64(seed))
    x = torch.tensor(gen.normal(0.5, 1.0, (M, N)), dtype=torch.float32).to(dtype)
    g = torch.tensor(gen.normal(1.0, 0.1, N), dtype=torch.float32).to(dtype)
    b = torch.tensor(gen.normal(0.0, 0.1, N), dtype=torch.float32).to(dtype) if with_beta else None
    dy = torch.tensor(gen.normal(0.0, 1.0, (M, N)), dtype=torch.float32).to(dtype)
    return x, g, b, dy


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("M,N", [(4, 7), (3, 256), (2, 3000)])
@pytest.mark.parametrize("eps", [1e-5, 1e-2])
def test_against_torch_layer_norm_autograd(dtype, M, N, eps):
    """float64 torch layer_norm on the exactly widened inputs. The oracle's
    backward reads the statistics as saved in fp32, so the gradients agree to
    fp32 rounding of mean and rstd, not to fp64."""
    x, g, b, dy = _inputs(7, M, N, dtype)
    mean, rstd, y = oracle.layernorm_fwd(x, g, b, eps)
    dx, dg, db = oracle.layernorm_bwd(x, g, dy, mean, rstd)
    x64 = x.to(F64).requires_grad_()
    g64 = g.to(F64).requires_grad_()
    b64 = b.to(F64).requires_grad_()
    y64 = F.layer_norm(x64, (N,), g64, b64, eps)
    y64.backward(dy.to(F64))
    var, mu = torch.var_mean(x.to(F64), dim=1, unbiased=False)
    assert rel(y, y64.detach()) <= 1e-12
    assert rel(mean.to(F64), mu) <= 1e-6
    assert rel(rstd.to(F64), 1.0 / torch.sqrt(var + eps)) <= 1e-6
    assert rel(dx, x64.grad) <= 1e-5
    assert rel(dg, g64.grad) <= 1e-5
    assert rel(db, b64.grad) <= 1e-12


@pytest.mark.parametrize("M,N", [(1, 3), (2, 8), (3, 33)])
@pytest.mark.parametrize("eps", [0.0, 1e-2])
def test_bwd_matches_finite_differences(M, N, eps):
    """dL/dx, dL/dgamma and dL/dbeta of L = sum(y * dy), from central
    differences of the oracle's forward with exact float32 perturbations."""
    gen = np.random.Generator(np.random.PCG64(100 + M * N))
    x = grid_values(gen, (M, N))
    g = grid_values(gen, N, lim=64) + 1.0
    b = grid_values(gen, N, lim=32)
    dy = grid_values(gen, (M, N), lim=64)
    mean, rstd, _ = oracle.layernorm_fwd(x, g, b, eps)
    dx, dg, db = oracle.layernorm_bwd(x, g, dy, mean, rstd)
    h = 2.0 ** -12

    def loss(xx, gg, bb):
        _, _, y = oracle.layernorm_fwd(xx, gg, bb, eps)
        return (y * dy.to(F64)).sum().item()

    def fd(t, idx):
        tp, tm = t.clone(), t.clone()
        tp[idx] += h
        tm[idx] -= h
        return tp, tm

    num_dx = torch.zeros(M, N, dtype=F64)
    for i in range(M):
        for j in range(N):
            xp, xm = fd(x, (i, j))
            num_dx[i, j] = (loss(xp, g, b) - loss(xm, g, b)) / (2 * h)
    num_dg = torch.zeros(N, dtype=F64)
    num_db = torch.zeros(N, dtype=F64)
    for j in range(N):
        gp, gm = fd(g, j)
        num_dg[j] = (loss(x, gp, b) - loss(x, gm, b)) / (2 * h)
        bp, bm = fd(b, j)
        num_db[j] = (loss(x, g, bp) - loss(x, g, bm)) / (2 * h)
    scale = max(num_dx.abs().max().item(), 1.0)
    assert (dx - num_dx).abs().max().item() <= 1e-4 * scale
    assert rel(dg, num_dg) <= 1e-5
    assert rel(db, num_db) <= 1e-9


def test_rows_of_dx_sum_to_zero():
    """Adding a constant to a row leaves its LayerNorm unchanged, so each row
    of dx sums to zero, for any eps. The backward reads the mean as saved in
    fp32, so the rows are chosen with a mean that fp32 holds exactly (grid
    values over a power-of-two N); dy and gamma are arbitrary."""
    gen = np.random.Generator(np.random.PCG64(11))
    M, N = 6, 512
    x = grid_values(gen, (M, N))
    _, g, b, dy = _inputs(11, M, N, torch.float32)
    for eps in (0.0, 1e-5, 0.5):
        mean, rstd, _ = oracle.layernorm_fwd(x, g, b, eps)
        assert torch.equal(mean.to(F64), x.to(F64).mean(dim=1))
        dx, _, _ = oracle.layernorm_bwd(x, g, dy, mean, rstd)
        assert dx.sum(dim=1).abs().max().item() <= 1e-13 * dx.abs().max().item() * N


def test_dbeta_is_the_column_sum_of_dy():
    gen = np.random.Generator(np.random.PCG64(5))
    dy = grid_values(gen, (9, 40))
    x, g, b, _ = _inputs(5, 9, 40, torch.float32)
    mean, rstd, _ = oracle.layernorm_fwd(x, g, b, 1e-5)
    _, _, db = oracle.layernorm_bwd(x, g, dy, mean, rstd)
    assert torch.equal(db, dy.to(F64).sum(dim=0))


def test_beta_shifts_the_output_only():
    x, g, b, dy = _inputs(13, 5, 64, torch.float32)
    m1, r1, y1 = oracle.layernorm_fwd(x, g, b, 1e-5)
    m0, r0, y0 = oracle.layernorm_fwd(x, g, None, 1e-5)
    assert torch.equal(m1, m0) and torch.equal(r1, r0)
    assert rel(y1 - y0, b.to(F64).expand(5, 64)) <= 1e-15


def test_zero_mean_rows_reduce_to_rmsnorm():
    """On a row whose mean is exactly zero, LayerNorm's statistics are
    RMSNorm's; with sum(dy * gamma) = 0 as well, c2 = 0 and the two backwards
    coincide bit for bit. Without that condition dx differs by c2 * rstd."""
    gen = np.random.Generator(np.random.PCG64(21))
    M, N = 4, 64
    half = grid_values(gen, (M, N // 2))
    x = torch.cat([half, -half.flip(1)], dim=1)        # exact zero mean
    g = torch.ones(N, dtype=torch.float32)
    dyh = grid_values(gen, (M, N // 2), lim=64)
    dy = torch.cat([dyh, -dyh], dim=1)                   # sum(dy * gamma) = 0
    for eps in (0.0, 1e-3):
        mean, rstd, _ = oracle.layernorm_fwd(x, g, None, eps)
        assert torch.equal(mean, torch.zeros(M))
        r_rms, _ = oracle.rmsnorm_fwd(x, g, eps, want_y=False)
        assert torch.equal(rstd, r_rms)
        dx, dg, _ = oracle.layernorm_bwd(x, g, dy, mean, rstd)
        dx_r, dg_r = oracle.rmsnorm_bwd(x, g, dy, r_rms)
        assert torch.equal(dx, dx_r) and torch.equal(dg, dg_r)
    # general dy: dx_ln = dx_rms - c2 * rstd with c2 = mean(dy * gamma)
    dy2 = grid_values(gen, (M, N), lim=64)
    mean, rstd, _ = oracle.layernorm_fwd(x, g, None, 1e-3)
    dx, _, _ = oracle.layernorm_bwd(x, g, dy2, mean, rstd)
    dx_r, _ = oracle.rmsnorm_bwd(x, g, dy2, rstd)
    c2 = dy2.to(F64).mean(dim=1, keepdim=True)
    assert rel(dx, dx_r - c2 * rstd.to(F64)[:, None]) <= 1e-12


def test_zero_upstream_gradient_gives_zero():
    x, g, b, dy = _inputs(3, 3, 100, torch.bfloat16)
    mean, rstd, _ = oracle.layernorm_fwd(x, g, b, 1e-5)
    dx, dg, db = oracle.layernorm_bwd(x, g, torch.zeros_like(dy), mean, rstd)
    assert not dx.any() and not dg.any() and not db.any()


def test_empty_batch_and_argument_errors():
    g = torch.ones(8)
    mean, rstd, y = oracle.layernorm_fwd(torch.zeros(0, 8), g, None, 1e-5)
    assert mean.numel() == 0 and y.numel() == 0
    dx, dg, db = oracle.layernorm_bwd(torch.zeros(0, 8), g, torch.zeros(0, 8), mean, rstd)
    assert not dg.any() and not db.any()
    with pytest.raises(ValueError):
        oracle.layernorm_fwd(torch.zeros(2, 8), g, torch.ones(7), 1e-5)
    with pytest.raises(ValueError):
        oracle.layernorm_fwd(torch.zeros(2, 8), g, None, -1.0)
