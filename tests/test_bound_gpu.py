"""Bound backward calls (bind_rmsnorm_bwd, bind_fused_add_rmsnorm_bwd,
bind_layernorm_bwd): checked and marshalled once, then enqueued again on
each call. They must give the same bits as the regular entry points on the
same buffers, follow in-place changes of the inputs, work under HIP-graph
capture (each call looks up the current stream), and refuse a workspace that
is too small when they are bound."""
import numpy as np
import pytest
import torch

import rmsnorm_bwd_amd as R
import workloads
from parity_util import DEV

pytestmark = pytest.mark.gpu
BF = torch.bfloat16


def draw(seed, shape, mu=0.0, sigma=1.0, dt=BF):
    gen = np.random.Generator(np.random.PCG64(seed))
    return workloads.normal(gen, shape, mu, sigma, dt).reshape(shape).to(DEV)


def same(a, b):
    return all(torch.equal(u, v) for u, v in zip(a, b) if u is not None)


@pytest.mark.parametrize("M,N", [(300, 4096), (1, 4096), (40, 256)])
def test_bound_plain_matches_the_regular_call(M, N):
    print("case bound plain", M, N, flush=True)
    x, dy, g = draw(1, (M, N)), draw(2, (M, N), 0.0, 1e-2), draw(3, (N,), 1.0, 0.1)
    _, rstd = R.rmsnorm_fwd_rstd(x, g, 1e-6)
    outs = (torch.empty_like(x), torch.empty(N, device=DEV), torch.empty_like(g))
    run = R.bind_rmsnorm_bwd(x, g, dy, rstd, dx=outs[0], dgamma_f32=outs[1], dgamma=outs[2])
    for seed in (10, 11):
        x.copy_(draw(seed, (M, N)))             # the bound buffers change in place
        _, r2 = R.rmsnorm_fwd_rstd(x, g, 1e-6)
        rstd.copy_(r2)
        got = [t.clone() for t in run()]
        ref = R.rmsnorm_bwd(x, g, dy, rstd, dgamma=torch.empty_like(g))
        torch.cuda.synchronize()
        assert same(got, ref)


def test_bound_fused_and_layernorm_match_the_regular_calls():
    print("case bound fused and layernorm", flush=True)
    M, N = 257, 2048
    a, dy, dres = draw(4, (M, N)), draw(5, (M, N), 0.0, 1e-2), draw(6, (M, N), 0.0, 1e-2)
    g, b = draw(7, (N,), 1.0, 0.1), draw(8, (N,), 0.0, 0.1)
    _, rstd = R.rmsnorm_fwd_rstd(a, g, 1e-6)
    run = R.bind_fused_add_rmsnorm_bwd(a, g, dy, dres, rstd, dgamma=torch.empty_like(g))
    got = [t.clone() for t in run()]
    ref = R.fused_add_rmsnorm_bwd(a, g, dy, dres, rstd, dgamma=torch.empty_like(g))
    _, mean, rstd_l = R.layernorm_fwd_stats(a, g, b, 1e-5)
    run_l = R.bind_layernorm_bwd(a, g, dy, mean, rstd_l, dgamma=torch.empty_like(g),
                                 dbeta=torch.empty_like(g))
    got_l = [t.clone() for t in run_l()]
    ref_l = R.layernorm_bwd(a, g, dy, mean, rstd_l, dgamma=torch.empty_like(g), dbeta=torch.empty_like(g))
    torch.cuda.synchronize()
    assert same(got, ref) and same(got_l, ref_l)


def test_bound_calls_replay_from_a_graph():
    print("case bound graph", flush=True)
    M, N = 512, 4096
    x, dy, g = draw(12, (M, N)), draw(13, (M, N), 0.0, 1e-2), draw(14, (N,), 1.0, 0.1)
    _, rstd = R.rmsnorm_fwd_rstd(x, g, 1e-6)
    run = R.bind_rmsnorm_bwd(x, g, dy, rstd, dgamma=torch.empty_like(g))
    eager = [t.clone() for t in run()]
    torch.cuda.synchronize()
    for t in run.outputs:
        if t is not None:
            t.zero_()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for _ in range(3):
        for t in run.outputs:
            if t is not None:
                t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert same(run.outputs, eager)


def test_bind_refuses_a_small_workspace():
    M, N = 1024, 4096
    x, dy, g = draw(15, (M, N)), draw(16, (M, N)), draw(17, (N,), 1.0, 0.1)
    rstd = torch.ones(M, device=DEV)
    need = R.rmsnorm_bwd_workspace_bytes(M, N, BF)
    with pytest.raises(R.RmsnError):
        R.bind_rmsnorm_bwd(x, g, dy, rstd, workspace=torch.empty(need - 256, dtype=torch.uint8, device=DEV))
