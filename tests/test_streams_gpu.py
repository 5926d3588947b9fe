"""Backward calls on several HIP streams at once.

A call that passes no workspace gets the one the binding keeps for its
(device, stream), so calls running concurrently on different streams never
share partial sums; the kernels keep no other state between calls. Four
streams run the same problems at the same time, over several rounds, and
every result must equal, bit for bit, the one the same call gives alone on
the default stream (the default dgamma sum is deterministic). One problem of
each round is also held to the CPU oracle.

Math: FlyDSL issue #769 ("[Feature] Add rmsnorm backward (+ forward saves
rstd) ..."), Implementation plan: Math, and PR sequence (LayerNorm); FlyDSL
PR #800 ("[rmsnorm] Add fused-add / residual backward (PR 2/3, #769)"),
fused-add commit.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_bwd_amd as R
import workloads
from parity_util import DEV, assert_close, rel, tol_dgamma

pytestmark = pytest.mark.gpu

STREAMS = 4
ROUNDS = 3


def _problem(op, M, N, seed):
    gen = np.random.Generator(np.random.PCG64(seed))
    t = torch.bfloat16
    x = workloads.normal(gen, (M, N), 0.5 if op == "layernorm" else 0.0, 1.0, t).reshape(M, N)
    g = workloads.normal(gen, (N,), 1.0, 0.1, t)
    dy = workloads.normal(gen, (M, N), 0.0, 1e-2, t).reshape(M, N)
    extra = workloads.normal(gen, (M, N), 0.0, 1e-2, t).reshape(M, N)  # dresidual_out
    if op == "layernorm":
        mean, rstd, _ = oracle.layernorm_fwd(x, g, None, 1e-6, want_y=False)
    else:
        mean = None
        rstd, _ = oracle.rmsnorm_fwd(x, g, 1e-6, want_y=False)
    return dict(x=x, g=g, dy=dy, extra=extra, mean=mean, rstd=rstd)


def _run(op, d):
    """One backward call on the current stream; returns its outputs."""
    if op == "plain":
        dx, dg32, _ = R.rmsnorm_bwd(d["x"], d["g"], d["dy"], d["rstd"])
        return dx, dg32
    if op == "fused":
        dx, dg32, _ = R.fused_add_rmsnorm_bwd(d["x"], d["g"], d["dy"], d["extra"], d["rstd"])
        return dx, dg32
    dx, dg32, db32, _, _ = R.layernorm_bwd(d["x"], d["g"], d["dy"], d["mean"], d["rstd"])
    return dx, dg32, db32


def _oracle(op, c):
    if op == "plain":
        return oracle.rmsnorm_bwd(c["x"], c["g"], c["dy"], c["rstd"])
    if op == "fused":
        return oracle.fused_add_rmsnorm_bwd(c["x"], c["g"], c["dy"], c["extra"], c["rstd"])
    return oracle.layernorm_bwd(c["x"], c["g"], c["dy"], c["mean"], c["rstd"])


@pytest.mark.parametrize("op,M,N", [("plain", 2048, 4096), ("fused", 1024, 8192), ("layernorm", 4096, 2048)])
def test_concurrent_streams_match_calls_alone(op, M, N):
    print("case streams", op, M, N, flush=True)
    cpu = [_problem(op, M, N, 100 + i) for i in range(STREAMS)]
    dev = [{k: (v.to(DEV) if v is not None else None) for k, v in c.items()} for c in cpu]
    torch.cuda.synchronize()
    alone = []
    for d in dev:
        alone.append([t.clone() for t in _run(op, d)])
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(STREAMS)]
    for rnd in range(ROUNDS):
        outs = [None] * STREAMS
        for i, s in enumerate(streams):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                outs[i] = _run(op, dev[i])
        torch.cuda.synchronize()
        for i in range(STREAMS):
            for name, a, b in zip(("dx", "dgamma", "dbeta"), outs[i], alone[i]):
                assert torch.equal(a, b), f"round {rnd}, stream {i}: {name} differs from the call alone"
    ref = _oracle(op, cpu[0])
    assert_close("dx", alone[0][0], ref[0], torch.bfloat16)
    assert rel(alone[0][1], ref[1]) <= tol_dgamma(M)
    if op == "layernorm":
        assert rel(alone[0][2], ref[2]) <= tol_dgamma(M)
