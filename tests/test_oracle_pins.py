"""Pins of the CPU oracle to things other than itself.

Each test holds the oracle against something the mathematics or a library
fixes: hand-derived worked examples (tests/golden), central finite differences
of the oracle's own forward, an explicit Jacobian, float64 torch.autograd on
the CPU, closed forms, invariants, and torch/numpy conversions. Together they
are meant to catch a dropped term, a wrong sign, a wrong index or a swapped
operand anywhere in the oracle (tests/test_oracle_mutants.py checks that).

Math being pinned: FlyDSL issue #769 ("[Feature] Add rmsnorm backward (+
forward saves rstd) ..."), Implementation plan: Math; fused-add behaviour:
FlyDSL PR #800 ("[rmsnorm] Add fused-add / residual backward (PR 2/3, #769)"),
fused-add commit.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
F64 = torch.float64


def t64(a):
    return torch.tensor(a, dtype=F64)


def rel(a, b):
    """Normwise infinity-relative error of a against b."""
    a, b = torch.as_tensor(a, dtype=F64), torch.as_tensor(b, dtype=F64)
    den = b.abs().max().item()
    return (a - b).abs().max().item() / (den if den > 0 else 1.0)


def grid_values(gen, shape, scale_bits=6, lim=256):
    """float32 values k * 2^-scale_bits, |k| <= lim: few significant bits, so a
    small power-of-two perturbation stays exact in float32."""
    k = gen.integers(-lim, lim + 1, size=shape)
    return torch.tensor(k * 2.0 ** -scale_bits, dtype=torch.float32)


# --------------------------------------------------------------------------
# Worked examples (tests/golden/closed_forms.json)
# --------------------------------------------------------------------------

def _golden_cases():
    with open(os.path.join(HERE, "golden", "closed_forms.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_golden_worked_examples(case, dtype):
    # Every value in the fixtures is exact in bf16/f16, so all dtypes must
    # reproduce them bit for bit.
    T = lambda k: torch.tensor(case[k], dtype=F64).to(dtype)
    gamma, dy = T("gamma"), T("dy")
    if case["op"] == "plain":
        x = T("x")
        rstd, y = oracle.rmsnorm_fwd(x, gamma, case["eps"])
        dx, dg = oracle.rmsnorm_bwd(x, gamma, dy, rstd)
    else:
        added, rstd, y = oracle.fused_add_rmsnorm_fwd(T("x"), T("residual"), gamma, case["eps"])
        assert torch.equal(added, T("added"))
        dx, dg = oracle.fused_add_rmsnorm_bwd(added, gamma, dy, T("dresidual_out"), rstd)
    assert torch.equal(rstd.to(F64), t64(case["rstd"]))
    assert torch.equal(y, t64(case["y"]))
    assert torch.equal(dx, t64(case["dx"]))
    assert torch.equal(dg, t64(case["dgamma"]))


# --------------------------------------------------------------------------
# Central finite differences of the oracle's own forward
# --------------------------------------------------------------------------

def _loss_plain(x, gamma, dy, eps):
    _, y = oracle.rmsnorm_fwd(x, gamma, eps)
    return float((y * dy.to(F64)).sum())


FD_SHAPES = [(1, 2), (2, 3), (3, 5), (2, 8), (1, 17), (2, 64)]


@pytest.mark.parametrize("M,N", FD_SHAPES)
@pytest.mark.parametrize("eps", [0.0, 1e-5, 1e-2])
def test_plain_bwd_matches_finite_differences(M, N, eps):
    gen = np.random.Generator(np.random.PCG64(100 * M + N))
    x = grid_values(gen, (M, N))
    gamma = torch.tensor(gen.uniform(0.5, 1.5, N), dtype=torch.float32)
    dy = torch.tensor(gen.standard_normal((M, N)), dtype=torch.float32)
    # keep every row away from zero (y = x * rstd is not differentiable there)
    x[:, 0] = 1.0
    rstd, _ = oracle.rmsnorm_fwd(x, gamma, eps)
    dx, dg = oracle.rmsnorm_bwd(x, gamma, dy, rstd)
    h = 2.0 ** -17
    fd = torch.zeros(M, N, dtype=F64)
    for i in range(M):
        for j in range(N):
            xp, xm = x.clone(), x.clone()
            xp[i, j] += h
            xm[i, j] -= h
            fd[i, j] = (_loss_plain(xp, gamma, dy, eps) - _loss_plain(xm, gamma, dy, eps)) / (2 * h)
    # the oracle's backward uses the float32-rounded rstd, the finite difference
    # the exact one: agreement is bounded by float32 rounding (~6e-8 relative)
    assert rel(dx, fd) < 1e-6
    # dweight: the loss is linear in gamma, so the difference quotient is exact
    fdg = torch.zeros(N, dtype=F64)
    for j in range(N):
        gp, gm = gamma.clone(), gamma.clone()
        gp[j] += 2.0 ** -10
        gm[j] -= 2.0 ** -10
        fdg[j] = (_loss_plain(x, gp, dy, eps) - _loss_plain(x, gm, dy, eps)) / 2.0 ** -9
    assert rel(dg, fdg) < 1e-6


def test_single_column_closed_form_vs_fd():
    # N = 1: dx = gamma * dy * eps * r^3, tiny next to r * gamma * dy; use an
    # absolute bound scaled by |r * gamma * dy|.
    x = torch.tensor([[0.75], [-1.25], [2.0]], dtype=torch.float32)
    gamma = torch.tensor([1.25], dtype=torch.float32)
    dy = torch.tensor([[1.0], [-0.5], [2.0]], dtype=torch.float32)
    eps = 1e-2
    rstd, _ = oracle.rmsnorm_fwd(x, gamma, eps)
    dx, _ = oracle.rmsnorm_bwd(x, gamma, dy, rstd)
    x64 = x.to(F64)
    r_exact = 1.0 / torch.sqrt(x64 ** 2 + eps)
    closed = 1.25 * dy.to(F64) * eps * r_exact ** 3
    scale = (r_exact * 1.25 * dy.to(F64)).abs().max().item()
    assert (dx - closed).abs().max().item() < 1e-6 * scale


@pytest.mark.parametrize("M,N", [(1, 3), (2, 8), (2, 33)])
@pytest.mark.parametrize("with_dres", [False, True])
def test_fused_bwd_matches_finite_differences_in_x_and_residual(M, N, with_dres):
    gen = np.random.Generator(np.random.PCG64(7 * M + N))
    x = grid_values(gen, (M, N))
    res = grid_values(gen, (M, N))
    x[:, 0] = 2.0
    res[:, 0] = 1.0
    gamma = torch.tensor(gen.uniform(0.5, 1.5, N), dtype=torch.float32)
    dy = torch.tensor(gen.standard_normal((M, N)), dtype=torch.float32)
    dres = torch.tensor(gen.standard_normal((M, N)), dtype=torch.float32) if with_dres else None
    eps = 1e-5

    def loss(xx, rr):
        added, _, out = oracle.fused_add_rmsnorm_fwd(xx, rr, gamma, eps)
        L = float((out * dy.to(F64)).sum())
        if dres is not None:
            L += float((added.to(F64) * dres.to(F64)).sum())
        return L

    added, rstd, _ = oracle.fused_add_rmsnorm_fwd(x, res, gamma, eps)
    dx, _ = oracle.fused_add_rmsnorm_bwd(added, gamma, dy, dres, rstd)
    h = 2.0 ** -17
    for which in ("x", "residual"):
        fd = torch.zeros(M, N, dtype=F64)
        for i in range(M):
            for j in range(N):
                a, b = (x.clone(), res.clone()), (x.clone(), res.clone())
                k = 0 if which == "x" else 1
                a[k][i, j] += h
                b[k][i, j] -= h
                fd[i, j] = (loss(*a) - loss(*b)) / (2 * h)
        assert rel(dx, fd) < 1e-6, which


# --------------------------------------------------------------------------
# Explicit Jacobian (a formula independent of the c1 form)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 5, 16, 64])
def test_plain_bwd_matches_explicit_jacobian(N):
    gen = np.random.Generator(np.random.PCG64(N))
    M = 3
    x = torch.tensor(gen.standard_normal((M, N)), dtype=torch.float32)
    gamma = torch.tensor(gen.normal(1.0, 0.1, N), dtype=torch.float32)
    dy = torch.tensor(gen.standard_normal((M, N)), dtype=torch.float32)
    eps = 1e-5
    rstd, _ = oracle.rmsnorm_fwd(x, gamma, eps)
    dx, dg = oracle.rmsnorm_bwd(x, gamma, dy, rstd)
    X, G, DY = x.double().numpy(), gamma.double().numpy(), dy.double().numpy()
    for i in range(M):
        r = float(rstd[i])  # the same stored rstd the oracle reads
        # y_j = gamma_j x_j r(x);  d r / d x_k = -r^3 x_k / N
        J = np.diag(G * r) - np.outer(G * X[i], X[i]) * (r ** 3 / N)  # J[j, k] = dy_j/dx_k
        ref = J.T @ DY[i]
        scale = max(np.abs(ref).max(), np.abs(G * DY[i] * r).max())
        assert np.abs(dx[i].numpy() - ref).max() <= 1e-12 * scale
    # dgamma_j = sum_i d(sum dy*y)/d gamma_j = sum_i dy_ij x_ij r_i
    R = rstd.double().numpy()[:, None]
    assert np.abs(dg.numpy() - (DY * X * R).sum(0)).max() < 1e-12 * np.abs(DY * X * R).sum(0).max()


# --------------------------------------------------------------------------
# float64 torch.autograd on the CPU
# --------------------------------------------------------------------------

def _torch_rmsnorm(x64, g64, eps):
    return x64 * torch.rsqrt((x64 * x64).mean(-1, keepdim=True) + eps) * g64


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("M,N", [(4, 7), (3, 256), (2, 3000)])
@pytest.mark.parametrize("eps", [1e-5, 1e-6, 1e-2])
def test_plain_against_torch_autograd(dtype, M, N, eps):
    w = workloads.custom("plain", M, N, {torch.float32: "f32", torch.float16: "f16",
                                          torch.bfloat16: "bf16"}[dtype], eps, seed=M * N)
    d = workloads.make_inputs(w)
    x, gamma, dy = d["x"], d["gamma"], d["dy"]
    rstd, y = oracle.rmsnorm_fwd(x, gamma, eps)
    dx, dg = oracle.rmsnorm_bwd(x, gamma, dy, rstd)
    x64 = x.to(F64).requires_grad_(True)
    g64 = gamma.to(F64).requires_grad_(True)
    y_ref = _torch_rmsnorm(x64, g64, eps)
    (y_ref * dy.to(F64)).sum().backward()
    assert rel(y, y_ref.detach()) < 1e-14
    r_ref = torch.rsqrt((x.to(F64) ** 2).mean(-1) + eps)
    assert rel(rstd.to(F64), r_ref) < 1e-7          # fp32 storage of rstd
    assert rel(dx, x64.grad) < 1e-6                 # bounded by that storage
    assert rel(dg, g64.grad) < 1e-6


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("with_dres", [False, True])
def test_fused_against_torch_autograd(dtype, with_dres):
    M, N, eps = 5, 130, 1e-6
    w = workloads.custom("fused", M, N, "f32" if dtype == torch.float32 else "bf16", eps, seed=3)
    d = workloads.make_inputs(w)
    dres = d["dresidual_out"] if with_dres else None
    added, rstd, out = oracle.fused_add_rmsnorm_fwd(d["x"], d["residual"], d["gamma"], eps)
    # torch's float32 addition rounded once to the dtype is the same stored sum
    assert torch.equal(added, (d["x"].float() + d["residual"].float()).to(dtype))
    dx, dg = oracle.fused_add_rmsnorm_bwd(added, d["gamma"], d["dy"], dres, rstd)
    a64 = added.to(F64).requires_grad_(True)
    g64 = d["gamma"].to(F64).requires_grad_(True)
    o = _torch_rmsnorm(a64, g64, eps)
    L = (o * d["dy"].to(F64)).sum()
    if dres is not None:
        L = L + (a64 * dres.to(F64)).sum()
    L.backward()
    assert rel(out, o.detach()) < 1e-14
    assert rel(dx, a64.grad) < 1e-6
    assert rel(dg, g64.grad) < 1e-6


# --------------------------------------------------------------------------
# Closed forms and invariants
# --------------------------------------------------------------------------

def test_zero_upstream_gradient_gives_zero():
    d = workloads.make_inputs(workloads.custom("plain", 6, 40, "f32", 1e-5))
    rstd, _ = oracle.rmsnorm_fwd(d["x"], d["gamma"], 1e-5)
    dx, dg = oracle.rmsnorm_bwd(d["x"], d["gamma"], torch.zeros_like(d["dy"]), rstd)
    assert torch.count_nonzero(dx) == 0 and torch.count_nonzero(dg) == 0


def test_single_row_dgamma_is_dy_times_x_hat():
    d = workloads.make_inputs(workloads.custom("plain", 1, 77, "bf16", 1e-6))
    rstd, _ = oracle.rmsnorm_fwd(d["x"], d["gamma"], 1e-6)
    _, dg = oracle.rmsnorm_bwd(d["x"], d["gamma"], d["dy"], rstd)
    assert torch.equal(dg, d["dy"][0].to(F64) * (d["x"][0].to(F64) * float(rstd[0])))


@pytest.mark.parametrize("eps", [0.0, 1e-5, 1e-2])
def test_orthogonality_identity(eps):
    # sum_j x_hat_j dx_j = N c1 eps r^3 with r the exact rstd; the oracle reads
    # the float32 one, so the identity holds to float32 rounding of r.
    gen = np.random.Generator(np.random.PCG64(5))
    M, N = 6, 96
    x = torch.tensor(gen.normal(0, 0.1, (M, N)), dtype=torch.float32)  # eps*r^2 is O(1) at 1e-2
    gamma = torch.tensor(gen.normal(1, 0.1, N), dtype=torch.float32)
    dy = torch.tensor(gen.standard_normal((M, N)), dtype=torch.float32)
    rstd, _ = oracle.rmsnorm_fwd(x, gamma, eps)
    dx, _ = oracle.rmsnorm_bwd(x, gamma, dy, rstd)
    x64, g64, dy64 = x.to(F64), gamma.to(F64), dy.to(F64)
    r = torch.rsqrt((x64 ** 2).mean(-1) + eps)
    x_hat = x64 * r[:, None]
    c1 = (x_hat * dy64 * g64).mean(-1)
    lhs = (x_hat * dx).sum(-1)
    rhs = N * c1 * eps * r ** 3
    scale = (N * c1.abs() * r)
    assert ((lhs - rhs).abs() <= 1e-6 * scale).all()


def test_orthogonality_exact_rows():
    # rows with mean(x^2) + eps a power of four: r is exact and the identity is exact
    case = next(c for c in _golden_cases() if c["name"] == "row_with_eps")
    x = torch.tensor(case["x"], dtype=torch.float32)
    gamma = torch.tensor(case["gamma"], dtype=torch.float32)
    gen = np.random.Generator(np.random.PCG64(9))
    dy = torch.tensor(gen.integers(-8, 9, size=(1, 4)) / 8.0, dtype=torch.float32)
    rstd, _ = oracle.rmsnorm_fwd(x, gamma, 3.0)
    dx, _ = oracle.rmsnorm_bwd(x, gamma, dy, rstd)
    r = float(rstd[0])
    x_hat = x.to(F64) * r
    c1 = float((x_hat * dy.to(F64) * gamma.to(F64)).mean())
    assert float((x_hat * dx).sum()) == pytest.approx(4 * c1 * 3.0 * r ** 3, rel=1e-15, abs=1e-15)


def test_scale_invariance_at_eps0_is_exact():
    d = workloads.make_inputs(workloads.custom("plain", 4, 300, "f32", 0.0))
    x, gamma, dy = d["x"], d["gamma"], d["dy"]
    r1, _ = oracle.rmsnorm_fwd(x, gamma, 0.0)
    r2, _ = oracle.rmsnorm_fwd(2 * x, gamma, 0.0)
    assert torch.equal(r2, r1 / 2)
    dx1, dg1 = oracle.rmsnorm_bwd(x, gamma, dy, r1)
    dx2, dg2 = oracle.rmsnorm_bwd(2 * x, gamma, dy, r2)
    assert torch.equal(dx2, dx1 / 2)
    assert torch.equal(dg2, dg1)


def test_linearity_in_dy_and_gamma_dy_product():
    d = workloads.make_inputs(workloads.custom("plain", 5, 64, "f32", 1e-5))
    x, gamma, dy = d["x"], d["gamma"], d["dy"]
    rstd, _ = oracle.rmsnorm_fwd(x, gamma, 1e-5)
    dx, dg = oracle.rmsnorm_bwd(x, gamma, dy, rstd)
    dx2, dg2 = oracle.rmsnorm_bwd(x, gamma, 2 * dy, rstd)
    assert torch.equal(dx2, 2 * dx) and torch.equal(dg2, 2 * dg)
    # two upstream gradients whose float32 sum is exact
    gen = np.random.Generator(np.random.PCG64(21))
    dy, dyb = grid_values(gen, (5, 64)), grid_values(gen, (5, 64))
    dx, dg = oracle.rmsnorm_bwd(x, gamma, dy, rstd)
    dxb, dgb = oracle.rmsnorm_bwd(x, gamma, dyb, rstd)
    dxs, dgs = oracle.rmsnorm_bwd(x, gamma, dy + dyb, rstd)
    assert rel(dxs, dx + dxb) < 1e-12 and rel(dgs, dg + dgb) < 1e-12
    # dx depends on gamma and dy only through their product; dgamma not on gamma
    dx4, dg4 = oracle.rmsnorm_bwd(x, 2 * gamma, dy / 2, rstd)
    assert torch.equal(dx4, dx) and torch.equal(dg4, dg / 2)
    _, dg5 = oracle.rmsnorm_bwd(x, 2 * gamma, dy, rstd)
    assert torch.equal(dg5, dg)


def test_dgamma_is_additive_over_row_splits():
    d = workloads.make_inputs(workloads.custom("plain", 9, 50, "bf16", 1e-6))
    rstd, _ = oracle.rmsnorm_fwd(d["x"], d["gamma"], 1e-6)
    _, dg = oracle.rmsnorm_bwd(d["x"], d["gamma"], d["dy"], rstd)
    _, a = oracle.rmsnorm_bwd(d["x"][:4].contiguous(), d["gamma"], d["dy"][:4].contiguous(), rstd[:4].contiguous())
    _, b = oracle.rmsnorm_bwd(d["x"][4:].contiguous(), d["gamma"], d["dy"][4:].contiguous(), rstd[4:].contiguous())
    assert rel(dg, a + b) < 1e-14


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_fused_equals_plain_on_added_plus_dresidual(dtype):
    name = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[dtype]
    d = workloads.make_inputs(workloads.custom("fused", 7, 200, name, 1e-6))
    added, rstd, out = oracle.fused_add_rmsnorm_fwd(d["x"], d["residual"], d["gamma"], 1e-6)
    r2, y2 = oracle.rmsnorm_fwd(added, d["gamma"], 1e-6)
    assert torch.equal(rstd, r2) and torch.equal(out, y2)
    dxp, dgp = oracle.rmsnorm_bwd(added, d["gamma"], d["dy"], rstd)
    dxf, dgf = oracle.fused_add_rmsnorm_bwd(added, d["gamma"], d["dy"], d["dresidual_out"], rstd)
    dx0, dg0 = oracle.fused_add_rmsnorm_bwd(added, d["gamma"], d["dy"], None, rstd)
    assert torch.equal(dx0, dxp) and torch.equal(dg0, dgp) and torch.equal(dgf, dgp)
    assert torch.equal(dxf, dxp + d["dresidual_out"].to(F64))


def test_half_inputs_equal_their_exact_float32_widening():
    # the dtype only changes how inputs are read: a bf16/f16 tensor gives the
    # same fp64 results as its exact float32 widening
    for name, dt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        d = workloads.make_inputs(workloads.custom("plain", 3, 90, name, 1e-5))
        rh, yh = oracle.rmsnorm_fwd(d["x"], d["gamma"], 1e-5)
        rf, yf = oracle.rmsnorm_fwd(d["x"].float(), d["gamma"].float(), 1e-5)
        assert torch.equal(rh, rf) and torch.equal(yh, yf)
        dxh, dgh = oracle.rmsnorm_bwd(d["x"], d["gamma"], d["dy"], rh)
        dxf, dgf = oracle.rmsnorm_bwd(d["x"].float(), d["gamma"].float(), d["dy"].float(), rf)
        assert torch.equal(dxh, dxf) and torch.equal(dgh, dgf)


def test_eps_is_honoured():
    # eps enters the forward: each of 1e-5, 1e-6, 1e-2 gives rstd = (ms + eps)^-1/2
    d = workloads.make_inputs(workloads.custom("plain", 3, 64, "f32", 0.0))
    x = d["x"] * 0.01
    ms = (x.to(F64) ** 2).mean(-1)
    seen = set()
    for eps in (1e-5, 1e-6, 1e-2):
        rstd, _ = oracle.rmsnorm_fwd(x, d["gamma"], eps)
        assert rel(rstd.to(F64), torch.rsqrt(ms + eps)) < 1e-7
        seen.add(tuple(rstd.tolist()))
    assert len(seen) == 3


def test_empty_batch_and_argument_errors():
    gamma = torch.ones(8)
    x = torch.empty(0, 8)
    rstd, y = oracle.rmsnorm_fwd(x, gamma, 1e-5)
    assert rstd.numel() == 0
    dx, dg = oracle.rmsnorm_bwd(x, gamma, x, rstd)
    assert dx.numel() == 0 and torch.equal(dg, torch.zeros(8, dtype=F64))
    with pytest.raises(ValueError):
        oracle.rmsnorm_fwd(torch.ones(2, 8), gamma, float("nan"))
    with pytest.raises(ValueError):
        oracle.rmsnorm_fwd(torch.ones(2, 8), gamma, -1.0)
    with pytest.raises(ValueError):
        oracle.rmsnorm_fwd(torch.ones(2, 0), torch.ones(0), 1e-5)


# --------------------------------------------------------------------------
# The oracle's own dtype decode / encode against torch and numpy
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_decode_all_half_patterns(dtype):
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    t = bits.view(dtype)
    got, ref = oracle.decode(t), t.to(F64)
    assert torch.equal(torch.isnan(got), torch.isnan(ref))
    ok = ~torch.isnan(ref)
    assert torch.equal(got[ok], ref[ok])
    assert torch.equal(torch.signbit(got[ok]), torch.signbit(ref[ok]))


def _f32_sample():
    hi = torch.arange(0, 1 << 16, dtype=torch.int64)
    lows = [0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2FFF, 0x3000,
            0x3001, 0x7FFF, 0x8000, 0x8001, 0x9000, 0xBFFF, 0xC000, 0xE000, 0xFFFF]
    gen = np.random.Generator(np.random.PCG64(11))
    lows += [int(v) for v in gen.integers(0, 1 << 16, size=6)]
    pats = torch.cat([(hi << 16) | lo for lo in lows])
    return pats.to(torch.int32).view(torch.float32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_encode_matches_torch_rounding(dtype):
    # every exponent and sign, with low halves that hit ties, near-ties and
    # sticky bits at the bf16 and f16 rounding positions
    f = _f32_sample()
    got = oracle.encode(f.to(F64), dtype)
    ref = f.to(dtype)
    gn, rn = torch.isnan(got), torch.isnan(ref)
    assert torch.equal(gn, rn)
    assert torch.equal(got[~gn].view(torch.int16), ref[~rn].view(torch.int16))


def test_generic_encoder_matches_c_float_conversion():
    gen = np.random.Generator(np.random.PCG64(12))
    f = _f32_sample().to(F64).numpy()
    # doubles near float32 ties: x + k * ulp64 for small k around halfway points
    # (values past the float32 range round to infinity on purpose)
    with np.errstate(over="ignore"):
        mid = (np.nextafter(f.astype(np.float32), np.float32(np.inf)).astype(np.float64) + f) / 2
        probes = np.concatenate([f, mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf),
                                 gen.standard_normal(100000) * 10.0 ** gen.integers(-40, 39, 100000)])
        probes = probes[np.isfinite(probes)]
        got = oracle.encode_bits(torch.from_numpy(probes), torch.float32).numpy()
        ref = probes.astype(np.float32).view(np.uint32).astype(np.int64)
    assert np.array_equal(got, ref)


def test_encoder_from_float64_matches_numpy_half():
    # numpy rounds float64 -> float16 directly (one rounding)
    gen = np.random.Generator(np.random.PCG64(13))
    v = np.concatenate([gen.standard_normal(200000) * 10.0 ** gen.integers(-9, 6, 200000),
                        np.array([65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25,
                                  3 * 2.0 ** -26, 2.0 ** -14, -0.0])])
    got = oracle.encode(torch.from_numpy(v), torch.float16).view(torch.int16).numpy()
    with np.errstate(over="ignore"):  # values past the float16 range round to infinity
        ref = v.astype(np.float16).view(np.int16)
    assert np.array_equal(got, ref)
