"""HIP-graph capture and replay of the C ABI entry points.

A forward (saving the statistics) and a backward of each operation are
captured once into a torch CUDAGraph over static buffers. Each of several
replays then runs on new inputs, which are copied eagerly into those buffers
between replays, with a synchronisation after each replay. Every replay must
equal, bit for bit, an eager call on the same inputs: the graph launches the
same kernels, and the deterministic weight-gradient sum repeats exactly. On
one replay the results are also held to the CPU oracle. The library clears
what must start at zero with kernels, not memset nodes, so each replay
starts clean.

Math: FlyDSL issue #769 ("[Feature] Add rmsnorm backward (+ forward saves
rstd) ..."), Implementation plan: Math; FlyDSL PR #800 ("[rmsnorm] Add
fused-add / residual backward (PR 2/3, #769)"), fused-add commit.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_bwd_amd as R
import workloads
from parity_util import DEV, assert_close, rel, tol_dgamma

pytestmark = pytest.mark.gpu

REPLAYS = 3


def draw(seed, M, N, dt, mu=0.0, sigma=1.0):
    gen = np.random.Generator(np.random.PCG64(seed))
    return workloads.normal(gen, (M, N), mu, sigma, dt).reshape(M, N)


def capture(fn):
    """Capture fn() into a graph after warming it up on a side stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("M,N", [(512, 2048), (300, 4096), (1, 4096), (8, 1024), (600, 24576), (300, 32768)])
def test_rmsnorm_forward_and_backward_replay(M, N):
    print("case graph rmsnorm", M, N, flush=True)
    dt, eps = torch.bfloat16, 1e-6
    g = workloads.normal(np.random.Generator(np.random.PCG64(1)), (N,), 1.0, 0.1, dt).to(DEV)
    x, dy = torch.empty(M, N, dtype=dt, device=DEV), torch.empty(M, N, dtype=dt, device=DEV)
    y, rstd = torch.empty_like(x), torch.empty(M, device=DEV)
    dx, dg32, dgt = torch.empty_like(x), torch.empty(N, device=DEV), torch.empty(N, dtype=dt, device=DEV)
    ws = torch.zeros(R.rmsnorm_bwd_workspace_bytes(M, N, dt), dtype=torch.uint8, device=DEV)

    def step():
        R.rmsnorm_fwd_rstd(x, g, eps, y=y, rstd=rstd)
        R.rmsnorm_bwd(x, g, dy, rstd, dx=dx, dgamma_f32=dg32, dgamma=dgt, workspace=ws)

    x.copy_(draw(2, M, N, dt).to(DEV))
    dy.copy_(draw(3, M, N, dt, 0.0, 1e-2).to(DEV))
    graph = capture(step)
    for i in range(REPLAYS):
        xc, dyc = draw(10 + i, M, N, dt), draw(20 + i, M, N, dt, 0.0, 1e-2)
        x.copy_(xc.to(DEV))
        dy.copy_(dyc.to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (y, rstd, dx, dg32, dgt)]
        step()  # eager, same inputs
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "rstd", "dx", "dgamma_f32", "dgamma"), got, (y, rstd, dx, dg32, dgt)):
            assert torch.equal(a, b), f"replay {i}: {name} differs from the eager call"
        if i == REPLAYS - 1:
            r_ref, y_ref = oracle.rmsnorm_fwd(xc, g.cpu(), eps)
            dx_ref, dg_ref = oracle.rmsnorm_bwd(xc, g.cpu(), dyc, got[1].cpu())
            assert_close("y", got[0], y_ref, dt)
            assert_close("dx", got[2], dx_ref, dt)
            assert rel(got[3], dg_ref) <= tol_dgamma(M)


def test_fused_and_layernorm_backward_replay():
    print("case graph fused + layernorm", flush=True)
    dt, M, N, eps = torch.bfloat16, 256, 8192, 1e-6
    g = workloads.normal(np.random.Generator(np.random.PCG64(4)), (N,), 1.0, 0.1, dt).to(DEV)
    bufs = {k: torch.empty(M, N, dtype=dt, device=DEV) for k in ("a", "dy", "dres", "dx", "dxl")}
    rstd, mean, rstd_l = (torch.empty(M, device=DEV) for _ in range(3))
    yl = torch.empty(M, N, dtype=dt, device=DEV)
    dg, dgl, dbl = (torch.empty(N, device=DEV) for _ in range(3))
    ws = torch.zeros(R.rmsnorm_bwd_workspace_bytes(M, N, dt), dtype=torch.uint8, device=DEV)
    wsl = torch.zeros(R.layernorm_bwd_workspace_bytes(M, N, dt), dtype=torch.uint8, device=DEV)

    def step():
        R.fused_add_rmsnorm_bwd(bufs["a"], g, bufs["dy"], bufs["dres"], rstd, dx=bufs["dx"],
                                dgamma_f32=dg, workspace=ws)
        R.layernorm_fwd_stats(bufs["a"], g, None, eps, y=yl, mean=mean, rstd=rstd_l)
        R.layernorm_bwd(bufs["a"], g, bufs["dy"], mean, rstd_l, dx=bufs["dxl"], dgamma_f32=dgl,
                        dbeta_f32=dbl, workspace=wsl)

    def load(i):
        ins = dict(a=draw(30 + i, M, N, dt, 0.5), dy=draw(40 + i, M, N, dt, 0.0, 1e-2),
                   dres=draw(50 + i, M, N, dt, 0.0, 1e-2))
        for k, v in ins.items():
            bufs[k].copy_(v.to(DEV))
        r, _ = oracle.rmsnorm_fwd(ins["a"], g.cpu(), eps, want_y=False)
        rstd.copy_(r.to(DEV))
        return ins, r

    load(0)
    graph = capture(step)
    outs = (bufs["dx"], dg, yl, mean, rstd_l, bufs["dxl"], dgl, dbl)
    for i in range(REPLAYS):
        ins, r = load(1 + i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        step()
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(zip(got, outs)):
            assert torch.equal(a, b), f"replay {i}: output {j} differs from the eager call"
        if i == REPLAYS - 1:
            dx_ref, dg_ref = oracle.fused_add_rmsnorm_bwd(ins["a"], g.cpu(), ins["dy"], ins["dres"], r)
            assert_close("fused dx", got[0], dx_ref, dt)
            assert rel(got[1], dg_ref) <= tol_dgamma(M)
            m_ref, r_ref, _ = oracle.layernorm_fwd(ins["a"], g.cpu(), None, eps, want_y=False)
            dxl_ref, dgl_ref, dbl_ref = oracle.layernorm_bwd(ins["a"], g.cpu(), ins["dy"], got[3].cpu(),
                                                             got[4].cpu())
            assert_close("layernorm dx", got[5], dxl_ref, dt)
            assert rel(got[6], dgl_ref) <= tol_dgamma(M) and rel(got[7], dbl_ref) <= tol_dgamma(M)


def test_captured_autograd_backward_keeps_its_own_workspace():
    """The autograd backward captured into a graph on a stream whose cached
    workspace an eager call created first; then a larger eager call on that
    stream replaces the cached workspace, and a new tensor of the old size,
    filled with a pattern, takes its memory. Replays of the graph must not
    write into that tensor (a graph keeps the workspace it captured), and
    must still match an eager autograd pass and the oracle."""
    print("case graph: captured autograd backward, then a larger eager call", flush=True)
    dt, eps, N, M, M_big = torch.bfloat16, 1e-6, 4096, 256, 2048
    w = workloads.normal(np.random.Generator(np.random.PCG64(5)), (N,), 1.0, 0.1, dt).to(DEV)
    w.requires_grad_()
    x = draw(60, M, N, dt).to(DEV).requires_grad_()
    dy = draw(61, M, N, dt, 0.0, 1e-2).to(DEV)
    cap = torch.cuda.Stream()

    def step():
        y = R.rmsnorm(x, w, eps)
        return torch.autograd.grad(y, (x, w), dy)

    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()  # eager: creates the cached workspace of stream `cap`
    torch.cuda.synchronize()
    need = R.rmsnorm_bwd_workspace_bytes(M, N, dt)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        gx, gw = step()
    torch.cuda.synchronize()
    xb, dyb = draw(62, M_big, N, dt).to(DEV), draw(63, M_big, N, dt, 0.0, 1e-2).to(DEV)
    with torch.cuda.stream(cap):
        # larger calls replace both caches of stream `cap`: the binding's and
        # the autograd nodes'
        _, rb = R.rmsnorm_fwd_rstd(xb, w.detach(), eps)
        R.rmsnorm_bwd(xb, w.detach(), dyb, rb)
        xbg = xb.clone().requires_grad_()
        torch.autograd.grad(R.rmsnorm(xbg, w, eps), (xbg, w), dyb)
        del xbg
        junk = [torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV) for _ in range(4)]
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        xc, dyc = draw(70 + i, M, N, dt), draw(80 + i, M, N, dt, 0.0, 1e-2)
        with torch.no_grad():
            x.copy_(xc.to(DEV))
        dy.copy_(dyc.to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for j in junk:
            assert bool((j == 0x5A).all()), f"replay {i}: the graph wrote into memory it does not own"
        got = (gx.clone(), gw.clone())
        ex, ew = step()
        torch.cuda.synchronize()
        assert torch.equal(got[0], ex) and torch.equal(got[1], ew), f"replay {i} differs from eager"
        if i == REPLAYS - 1:
            r_ref, _ = oracle.rmsnorm_fwd(xc, w.detach().cpu(), eps, want_y=False)
            dx_ref, dg_ref = oracle.rmsnorm_bwd(xc, w.detach().cpu(), dyc, r_ref)
            assert_close("dx", got[0], dx_ref, dt)
            assert_close("dweight", got[1], dg_ref, dt)
