"""The autograd wrappers on the GPU: rmsnorm(x, weight, eps) and
fused_add_rmsnorm(x, residual, weight, eps, prenorm) against the CPU oracle
(values) and against plain PyTorch autograd in fp64 (how gradients flow:
batched input, both outputs of the prenorm form, one gradient for x and
residual).

FlyDSL issue #769 ("[Feature] Add rmsnorm backward (+ forward saves rstd)
..."), Scope / tasks items 3-4; FlyDSL PR #800 ("[rmsnorm] Add fused-add /
residual backward (PR 2/3, #769)"), PR-1 commit (end-to-end autograd test on
batched input with gradients on x and weight) and fused-add commit.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_bwd_amd as R
import workloads
from parity_util import DEV, assert_close, rel, tol_dgamma

pytestmark = pytest.mark.gpu


def _draw(shape, seed, mu=0.0, sigma=1.0, dtype=torch.bfloat16):
    gen = np.random.Generator(np.random.PCG64(seed))
    return workloads.normal(gen, shape, mu, sigma, dtype).reshape(shape)


def test_rmsnorm_autograd_batched_bf16():
    print("case autograd rmsnorm (4, 6, 640) bf16", flush=True)
    shape, N, eps = (4, 6, 640), 640, 1e-6
    x = _draw(shape, 1)
    w = _draw((N,), 2, 1.0, 0.1)
    g = _draw(shape, 3, 0.0, 1e-2)
    xg = x.to(DEV).requires_grad_()
    wg = w.to(DEV).requires_grad_()
    y = R.rmsnorm(xg, wg, eps)
    assert y.shape == shape and y.dtype == torch.bfloat16
    y.backward(g.to(DEV))
    torch.cuda.synchronize()
    x2 = x.reshape(-1, N)
    r_ref, y_ref = oracle.rmsnorm_fwd(x2, w, eps)
    dx_ref, dg_ref = oracle.rmsnorm_bwd(x2, w, g.reshape(-1, N), r_ref)
    assert_close("y", y.detach().reshape(-1, N), y_ref, torch.bfloat16)
    assert xg.grad.shape == shape
    assert_close("dx", xg.grad.reshape(-1, N), dx_ref, torch.bfloat16)
    assert wg.grad.dtype == torch.bfloat16
    assert_close("dweight", wg.grad, dg_ref, torch.bfloat16)


def test_rmsnorm_autograd_f32_matches_fp64_torch():
    """fp32 gradients against PyTorch autograd of the plain formula in fp64."""
    print("case autograd rmsnorm (37, 300) f32", flush=True)
    M, N, eps = 37, 300, 1e-5
    x = _draw((M, N), 4, dtype=torch.float32)
    w = _draw((N,), 5, 1.0, 0.1, dtype=torch.float32)
    g = _draw((M, N), 6, dtype=torch.float32)
    xg = x.to(DEV).requires_grad_()
    wg = w.to(DEV).requires_grad_()
    R.rmsnorm(xg, wg, eps).backward(g.to(DEV))
    torch.cuda.synchronize()
    x64 = x.double().requires_grad_()
    w64 = w.double().requires_grad_()
    y64 = x64 * torch.rsqrt((x64 * x64).mean(-1, keepdim=True) + eps) * w64
    y64.backward(g.double())
    assert rel(xg.grad, x64.grad) <= 1e-5
    assert rel(wg.grad, w64.grad) <= tol_dgamma(M)


@pytest.mark.parametrize("prenorm", [True, False])
def test_fused_add_autograd(prenorm):
    print("case autograd fused_add_rmsnorm prenorm", prenorm, flush=True)
    shape, N, eps = (8, 3, 1024), 1024, 1e-6
    x = _draw(shape, 7)
    res = _draw(shape, 8)
    w = _draw((N,), 9, 1.0, 0.1)
    g1 = _draw(shape, 10, 0.0, 1e-2)
    g2 = _draw(shape, 11, 0.0, 1e-2)
    xg = x.to(DEV).requires_grad_()
    rg = res.to(DEV).requires_grad_()
    wg = w.to(DEV).requires_grad_()
    got = R.fused_add_rmsnorm(xg, rg, wg, eps, prenorm=prenorm)
    if prenorm:
        out, res_out = got
        torch.autograd.backward([out, res_out], [g1.to(DEV), g2.to(DEV)])
    else:
        out = got
        out.backward(g1.to(DEV))
    torch.cuda.synchronize()
    x2, r2 = x.reshape(-1, N), res.reshape(-1, N)
    added, r_ref, out_ref = oracle.fused_add_rmsnorm_fwd(x2, r2, w, eps)
    dres = g2.reshape(-1, N) if prenorm else None
    dx_ref, dg_ref = oracle.fused_add_rmsnorm_bwd(added, w, g1.reshape(-1, N), dres, r_ref)
    assert_close("out", out.detach().reshape(-1, N), out_ref, torch.bfloat16)
    if prenorm:
        assert torch.equal(res_out.detach().reshape(-1, N).cpu(), added)
    assert torch.equal(xg.grad, rg.grad), "x and residual must get one gradient"
    assert_close("dx", xg.grad.reshape(-1, N), dx_ref, torch.bfloat16)
    assert_close("dweight", wg.grad, dg_ref, torch.bfloat16)


def test_rmsnorm_autograd_of_a_sum_takes_an_expanded_gradient():
    """loss = y.sum(): autograd hands the backward a stride-0 (expanded)
    gradient of ones, which the wrapper must copy before the library reads it."""
    print("case autograd rmsnorm sum() (5, 768) bf16", flush=True)
    M, N, eps = 5, 768, 1e-6
    x = _draw((M, N), 12)
    w = _draw((N,), 13, 1.0, 0.1)
    xg = x.to(DEV).requires_grad_()
    wg = w.to(DEV).requires_grad_()
    R.rmsnorm(xg, wg, eps).sum().backward()
    torch.cuda.synchronize()
    ones = torch.ones(M, N, dtype=torch.bfloat16)
    r_ref, _ = oracle.rmsnorm_fwd(x, w, eps)
    dx_ref, dg_ref = oracle.rmsnorm_bwd(x, w, ones, r_ref)
    assert_close("dx", xg.grad, dx_ref, torch.bfloat16)
    assert_close("dweight", wg.grad, dg_ref, torch.bfloat16)


def test_fused_add_autograd_with_only_residual_out_in_the_loss():
    """Only residual_out feeds the loss, so the gradient of out arrives as
    None (zeros): dx must equal the incoming residual gradient exactly, and
    dweight must be zero."""
    print("case autograd fused_add_rmsnorm residual_out only (6, 512) bf16", flush=True)
    M, N, eps = 6, 512, 1e-6
    x, res = _draw((M, N), 14), _draw((M, N), 15)
    w = _draw((N,), 16, 1.0, 0.1)
    g2 = _draw((M, N), 17, 0.0, 1e-2)
    xg, rg, wg = (t.to(DEV).requires_grad_() for t in (x, res, w))
    _, res_out = R.fused_add_rmsnorm(xg, rg, wg, eps, prenorm=True)
    res_out.backward(g2.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(xg.grad.cpu(), g2)
    assert torch.equal(rg.grad.cpu(), g2)
    assert torch.count_nonzero(wg.grad).item() == 0


def test_autograd_long_rows():
    """rmsnorm and fused_add_rmsnorm through autograd on rows longer than
    16384 elements (the two-pass kernels), against the oracle."""
    print("case autograd long rows (2, 3, 20000) bf16", flush=True)
    shape, N, eps = (2, 3, 20000), 20000, 1e-6
    x, res = _draw(shape, 21), _draw(shape, 22)
    w = _draw((N,), 23, 1.0, 0.1)
    g, gr = _draw(shape, 24, 0.0, 1e-2), _draw(shape, 25, 0.0, 1e-2)
    xg, wg = x.to(DEV).requires_grad_(), w.to(DEV).requires_grad_()
    R.rmsnorm(xg, wg, eps).backward(g.to(DEV))
    xf, rf, wf = x.to(DEV).requires_grad_(), res.to(DEV).requires_grad_(), w.to(DEV).requires_grad_()
    out, res_out = R.fused_add_rmsnorm(xf, rf, wf, eps)
    torch.autograd.backward((out, res_out), (g.to(DEV), gr.to(DEV)))
    torch.cuda.synchronize()
    x2, r2 = x.reshape(-1, N), res.reshape(-1, N)
    rs, _ = oracle.rmsnorm_fwd(x2, w, eps)
    dx_ref, dg_ref = oracle.rmsnorm_bwd(x2, w, g.reshape(-1, N), rs)
    assert_close("dx", xg.grad.reshape(-1, N), dx_ref, torch.bfloat16)
    assert_close("dweight", wg.grad, dg_ref, torch.bfloat16)
    a_ref, ra, _ = oracle.fused_add_rmsnorm_fwd(x2, r2, w, eps)
    dxf_ref, dgf_ref = oracle.fused_add_rmsnorm_bwd(a_ref, w, g.reshape(-1, N), gr.reshape(-1, N), ra)
    assert torch.equal(xf.grad, rf.grad)
    assert_close("fused dx", xf.grad.reshape(-1, N), dxf_ref, torch.bfloat16)
    assert_close("fused dweight", wf.grad, dgf_ref, torch.bfloat16)
