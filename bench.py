"""Benchmark: rmsnorm_bwd microseconds per call and achieved HBM bandwidth at
4096 x 4096 bf16, on one MI355X, through the C ABI.

A step is one call of the backward entry point (dx and dgamma, with the dgamma
finalize and the bf16 cast of dgamma inside the call), made through a call
the binding checked and marshalled once for each buffer set. Inputs are seeded
synthetic rows; rstd comes from the library's own forward. By default the
timed calls rotate over enough buffer sets (> 512 MiB) that no call finds its
rows in the 256 MiB memory-side cache: every byte comes from HBM. The line
also carries the hot-cache time (one buffer set, as the pages time it), the
forward's time, the roofline of the dominant kernel and the CPU oracle's time
on the same workload.

python bench.py [--steps K] [--warmup W] [--workload NAME] [--hot] [--gpus 1]
"""
import argparse
import json
import os
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import rmsnorm_bwd_amd as R  # noqa: E402
import workloads  # noqa: E402

HBM_PEAK_GBPS = 8000.0   # MI355X published HBM3E bandwidth
ROTATE_BYTES = 600 << 20  # > 2 x the 256 MiB memory-side cache
OP_NAMES = {"plain": "rmsnorm_bwd", "fused": "fused_add_rmsnorm_bwd", "layernorm": "layernorm_bwd"}


def algorithmic_bytes(w):
    """Bytes the backward must move: read x (or added), dy, [dresidual_out],
    gamma, rstd [and mean]; write dx, dgamma_f32 [and dbeta_f32] and their
    dtype copies."""
    s = w.elem_bytes
    rows = (4 if w.op == "fused" else 3) * w.M * w.N * s
    ngrad = 2 if w.op == "layernorm" else 1
    stats = (8 if w.op == "layernorm" else 4) * w.M
    return rows + w.N * s + stats + ngrad * (4 * w.N + (w.N * s if s != 4 else 0))


def fwd_bytes(w):
    s = w.elem_bytes
    rows = (4 if w.op == "fused" else 2) * w.M * w.N * s
    if w.op == "layernorm":
        return rows + 2 * w.N * s + 8 * w.M
    return rows + w.N * s + 4 * w.M


def make_sets(w, d, nsets):
    """nsets independent device buffer sets holding the same inputs."""
    dev = torch.device("cuda:0")
    g = d["gamma"].to(dev)
    sets = []
    for _ in range(nsets):
        if w.op == "plain":
            x = d["x"].to(dev)
            y, rstd = R.rmsnorm_fwd_rstd(x, g, w.eps)
            s = dict(x=x, dy=d["dy"].to(dev), dres=None, rstd=rstd)
        elif w.op == "layernorm":
            x = d["x"].to(dev)
            beta = d["beta"].to(dev)
            y, mean, rstd = R.layernorm_fwd_stats(x, g, beta, w.eps)
            s = dict(x=x, dy=d["dy"].to(dev), dres=None, rstd=rstd, mean=mean, beta=beta,
                     db32=torch.empty(w.N, dtype=torch.float32, device=dev),
                     db=torch.empty(w.N, dtype=w.torch_dtype, device=dev))
        else:
            x, res = d["x"].to(dev), d["residual"].to(dev)
            out, added, rstd = R.fused_add_rmsnorm_fwd_rstd(x, res, g, w.eps)
            del x, res, out
            s = dict(x=added, dy=d["dy"].to(dev), dres=d["dresidual_out"].to(dev), rstd=rstd)
        s["dx"] = torch.empty_like(s["x"])
        s["dg32"] = torch.empty(w.N, dtype=torch.float32, device=dev)
        s["dg"] = torch.empty(w.N, dtype=w.torch_dtype, device=dev)
        query = R.layernorm_bwd_workspace_bytes if w.op == "layernorm" else R.rmsnorm_bwd_workspace_bytes
        s["ws"] = torch.empty(max(256, query(w.M, w.N, w.torch_dtype)), dtype=torch.uint8, device=dev)
        s["run"] = bind_bwd(w, g, s)
        sets.append(s)
    return g, sets


def bind_bwd(w, g, s):
    """The set's backward call, checked and marshalled once by the binding
    (a BoundCall): each timed call only enqueues the kernels on the current
    stream, as a training loop over fixed buffers would."""
    if w.op == "plain":
        return R.bind_rmsnorm_bwd(s["x"], g, s["dy"], s["rstd"], dx=s["dx"], dgamma_f32=s["dg32"],
                                  dgamma=s["dg"], workspace=s["ws"])
    if w.op == "layernorm":
        return R.bind_layernorm_bwd(s["x"], g, s["dy"], s["mean"], s["rstd"], dx=s["dx"],
                                    dgamma_f32=s["dg32"], dbeta_f32=s["db32"], dgamma=s["dg"],
                                    dbeta=s["db"], workspace=s["ws"])
    return R.bind_fused_add_rmsnorm_bwd(s["x"], g, s["dy"], s["dres"], s["rstd"], dx=s["dx"],
                                        dgamma_f32=s["dg32"], dgamma=s["dg"], workspace=s["ws"])


def call_bwd(w, g, s):
    if "run" in s:
        s["run"]()
        return
    if w.op == "plain":
        R.rmsnorm_bwd(s["x"], g, s["dy"], s["rstd"], dx=s["dx"], dgamma_f32=s["dg32"],
                      dgamma=s["dg"], workspace=s["ws"])
    elif w.op == "layernorm":
        R.layernorm_bwd(s["x"], g, s["dy"], s["mean"], s["rstd"], dx=s["dx"], dgamma_f32=s["dg32"],
                        dbeta_f32=s["db32"], dgamma=s["dg"], dbeta=s["db"], workspace=s["ws"])
    else:
        R.fused_add_rmsnorm_bwd(s["x"], g, s["dy"], s["dres"], s["rstd"], dx=s["dx"],
                                dgamma_f32=s["dg32"], dgamma=s["dg"], workspace=s["ws"])


def time_calls(fn, sets, steps, warmup):
    """Average ms per call over `steps` calls, HIP events on the current stream
    (the stream every call is launched on), synchronised on both sides."""
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(sets[i % len(sets)])
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def time_graph(fn, sets, steps, warmup):
    """Average ms per call of `steps` calls (cycling through the sets, as
    time_calls does) captured in one HIP graph and replayed once, after
    `warmup` eager calls and one untimed replay: the same GPU work without the
    host's launch overhead between kernels, so kernels run back to back."""
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            fn(sets[i % len(sets)])
    graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    graph.replay()
    end.record()
    torch.cuda.synchronize()
    del graph
    return start.elapsed_time(end) / steps


def copy_bandwidth(mib=512, reps=10):
    """Achievable HBM bandwidth on this part: a device-to-device copy of
    `mib` MiB (twice the memory-side cache), read + write bytes per second."""
    n = (mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ms = time_calls(lambda _: dst.copy_(src), [None], reps, 2)
    del src, dst
    return 2 * (mib << 20) / (ms * 1e-3) / 1e9


def _graph_us(fn, calls=20, replays=50):
    """GPU time per call of fn, captured `calls` times in one HIP graph and
    replayed: the host's launch overhead is out of the measurement."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    ms = time_calls(lambda _: graph.replay(), [None], replays, 3)
    return ms * 1e3 / calls


def latency_floor(w_name="plain_1x4096_bf16"):
    """The one-row backward (a single kernel), per call, against a
    one-element torch kernel, both replayed from a HIP graph so that only GPU
    time counts; the graph's dx is checked against an eager call's."""
    w = workloads.WORKLOADS[w_name]
    d = workloads.make_inputs(w)
    g, sets = make_sets(w, d, 1)
    s = sets[0]
    call_bwd(w, g, s)
    torch.cuda.synchronize()
    eager = s["dx"].clone()
    s["dx"].zero_()
    us = _graph_us(lambda: call_bwd(w, g, s))
    torch.cuda.synchronize()
    t = torch.zeros(1, device="cuda:0")
    us_empty = _graph_us(lambda: t.add_(1.0))
    return {"workload": w_name, "us_per_call": round(us, 2), "one_element_kernel_us": round(us_empty, 2),
            "timing": "HIP graph replay", "graph_matches_eager": bool(torch.equal(eager, s["dx"]))}


def mode_sweep(reps=3):
    """The dgamma modes against each other on an (M, N) grid: GPU time per
    call from HIP-graph replay, each mode timed `reps` times in rotating
    order and the median kept (one JSON line per shape). The one-block mode
    (one CU does all the work) is timed up to 512 rows. This is the
    measurement behind the default mode's rule."""
    dev = torch.device("cuda:0")
    modes = (("auto", R.DGAMMA_AUTO), ("deterministic", R.DGAMMA_DETERMINISTIC),
             ("atomic", R.DGAMMA_ATOMIC), ("one_block", R.DGAMMA_ONE_BLOCK))
    for dt in (torch.bfloat16, torch.float32):
        es = 2 if dt == torch.bfloat16 else 4
        for N in (256, 1024, 4096, 8192, 16384):
            for M in (1, 2, 4, 8, 16, 32, 64, 128, 512, 2048, 8192):
                per = 3 * M * N * es
                nsets = max(1, min(8, -(-ROTATE_BYTES // per)))
                g = torch.ones(N, dtype=dt, device=dev)
                sets = []
                for _ in range(nsets):
                    x = torch.randn(M, N, device=dev).to(dt)
                    _, rstd = R.rmsnorm_fwd_rstd(x, g, 1e-6)
                    ws = max(R.rmsnorm_bwd_workspace_bytes(M, N, dt, fl) for _, fl in modes)
                    sets.append((x, torch.randn(M, N, device=dev).to(dt), rstd, torch.empty_like(x),
                                 torch.empty(N, device=dev), torch.empty(N, dtype=dt, device=dev),
                                 torch.empty(max(256, ws), dtype=torch.uint8, device=dev)))
                row = {"dtype": str(dt).split(".")[-1], "M": M, "N": N}
                todo = [(n, fl) for n, fl in modes if n != "one_block" or M <= 512]
                times = {n: [] for n, _ in todo}
                for rep in range(reps):
                    for name, fl in todo[rep % len(todo):] + todo[:rep % len(todo)]:
                        it = iter(range(1 << 30))

                        def call():
                            t = sets[next(it) % nsets]
                            R.rmsnorm_bwd(t[0], g, t[1], t[2], dx=t[3], dgamma_f32=t[4], dgamma=t[5],
                                          workspace=t[6], flags=fl)
                        times[name].append(_graph_us(call, calls=max(nsets, 8), replays=5))
                for name, _ in todo:
                    row[name + "_us"] = round(statistics.median(times[name]), 2)
                print(json.dumps(row), flush=True)
                del sets
                torch.cuda.empty_cache()


def shape_sweep(steps=50, ns=(1024, 2048, 4096, 8192), ms=(1, 128, 512, 1024, 4096, 16384, 32768), dtype="bf16",
                ops=("plain", "fused")):
    """The backward and the forward of plain and fused-add RMSNorm (and, when
    `ops` names it, LayerNorm) over an (M, N) grid in one dtype: GPU time per
    call from one HIP-graph replay of `steps` calls rotating over buffer sets
    of > 512 MiB (as the headline is timed), algorithmic GB/s and its share of
    8 TB/s. One JSON line per shape."""
    dev = torch.device("cuda:0")
    td = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    for op in ops:
        ln = op == "layernorm"
        for N in ns:
            for M in ms:
                w = workloads.custom(op, M, N, dtype, 1e-6, dy_sigma=1e-2)
                per = (4 if op == "fused" else 3) * M * N * td.itemsize
                # a replay touches at most `steps` sets; below 512 MiB in all
                # (short shapes) the calls find their rows in the memory-side
                # cache, as a latency-bound call of that size would in use
                nsets = max(2, min(steps, -(-ROTATE_BYTES // per)))
                g = (1 + 0.1 * torch.randn(N, device=dev)).to(td)
                beta = (0.1 * torch.randn(N, device=dev)).to(td) if ln else None
                sets = []
                for _ in range(nsets):
                    x = torch.randn(M, N, device=dev).to(td)
                    if ln:
                        _, mean, rstd = R.layernorm_fwd_stats(x, g, beta, w.eps)
                    else:
                        mean = None
                        _, rstd = R.rmsnorm_fwd_rstd(x, g, w.eps)
                    t = dict(x=x, dy=(1e-2 * torch.randn(M, N, device=dev)).to(td),
                             dres=(1e-2 * torch.randn(M, N, device=dev)).to(td)
                             if op == "fused" else None,
                             rstd=rstd, mean=mean, dx=torch.empty_like(x), dg32=torch.empty(N, device=dev),
                             dg=torch.empty_like(g))
                    query = R.layernorm_bwd_workspace_bytes if ln else R.rmsnorm_bwd_workspace_bytes
                    if ln:
                        t["db32"], t["db"] = torch.empty(N, device=dev), torch.empty_like(g)
                    t["ws"] = torch.empty(max(256, query(M, N, td)), dtype=torch.uint8, device=dev)
                    sets.append(t)

                def fwd(t):
                    if op == "plain":
                        R.rmsnorm_fwd_rstd(t["x"], g, w.eps, y=t["dx"], rstd=t["rstd"])
                    elif ln:
                        R.layernorm_fwd_stats(t["x"], g, beta, w.eps, y=t["dx"], mean=t["mean"],
                                              rstd=t["rstd"])
                    else:
                        R.fused_add_rmsnorm_fwd_rstd(t["x"], t["dy"], g, w.eps, out=t["dx"],
                                                     residual_out=t["dres"], rstd=t["rstd"])
                us = time_graph(lambda t: call_bwd(w, g, t), sets, steps, 5) * 1e3
                us_f = time_graph(fwd, sets, steps, 5) * 1e3
                b, bf = algorithmic_bytes(w), fwd_bytes(w)
                print(json.dumps({"op": op, "M": M, "N": N, "dtype": dtype, "bwd_us": round(us, 2),
                                  "bwd_GBps": round(b / us / 1e3, 1),
                                  "bwd_pct_of_8TBps": round(100 * b / us / 1e3 / HBM_PEAK_GBPS, 1),
                                  "fwd_us": round(us_f, 2), "fwd_GBps": round(bf / us_f / 1e3, 1)}),
                      flush=True)
                del sets
                torch.cuda.empty_cache()


# The shapes of the public-API comparison on [P854] (Benchmark contract, its
# timing table), with the pages' own MI355X times in microseconds: the
# FlyDSL backward and torch's, both through autograd.
API_SHAPES = [
    # op, M, N, dtype, pages' FlyDSL us, pages' torch us
    ("plain", 1, 4096, "bf16", 85.4, 42.8), ("fused", 1, 4096, "bf16", 98.6, 83.2),
    ("plain", 128, 4096, "bf16", 92.2, 57.5), ("fused", 128, 4096, "bf16", 114.5, 76.7),
    ("plain", 4096, 4096, "bf16", 157.2, 67.7), ("fused", 4096, 4096, "bf16", 160.2, 82.4),
    ("plain", 512, 2048, "bf16", 81.2, 48.5), ("fused", 512, 2048, "bf16", 100.3, 64.0),
    ("plain", 512, 3000, "f32", 77.6, 48.6), ("fused", 512, 3000, "f32", 94.8, 63.4),
    ("plain", 1024, 8192, "bf16", 81.1, 47.5), ("fused", 1024, 8192, "bf16", 102.0, 74.7),
]


def _autograd_graph_us(forward, impl, d, op, dev, with_backward, calls=10, replays=20):
    """GPU time per pass of `forward` (and, with_backward, of the backward
    through torch.autograd.grad) from one HIP graph of `calls` passes,
    replayed. The leaves are fresh tensors that no eager pass has touched,
    and the warm-up and the capture run on one side stream, so every autograd
    node of the captured passes belongs to the capturing stream."""
    x = d["x"].to(dev).requires_grad_()
    weight = d["gamma"].to(dev).requires_grad_()
    res = d["residual"].to(dev).requires_grad_() if op == "fused" else None
    douts = (d["dy"].to(dev),) if op == "plain" else (d["dy"].to(dev), d["dresidual_out"].to(dev))
    inputs = (x, weight) if op == "plain" else (x, res, weight)

    def one():
        o = forward(impl, x, weight, res)
        if with_backward:
            torch.autograd.grad(o, inputs, douts)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        for _ in range(3):
            one()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for _ in range(calls):
            one()
    torch.cuda.synchronize()
    ms = time_calls(lambda _: graph.replay(), [None], replays, 3)
    del graph
    return ms * 1e3 / calls


def api_compare(warmup=10, iters=100, windows=7):
    """Backward through the public autograd API, this library's wrappers
    against torch's eager RMSNorm (torch.nn.functional.rms_norm; for the
    fused-add form, torch's add then rms_norm), timed the way [P854]'s
    benchmark contract times them: the forward graph is built before timing;
    each backward allocates its gradients and includes the weight gradient's
    reduction and its cast to the parameter dtype; hot cache; HIP events
    around `iters` backward calls after `warmup`. The two implementations
    are timed in alternating windows in one process, so both see the same
    host state, and each figure is the median over `windows` windows. Each
    backward's GPU time is also given: one HIP graph of forward and backward
    replayed, less one of the forward alone. Gradients of the two are
    compared before timing. One JSON line per shape."""
    import torch.nn.functional as F
    from rmsnorm_bwd_amd.autograd import fused_add_rmsnorm, rmsnorm
    dev = torch.device("cuda:0")
    for op, M, N, dt, pages_dsl, pages_torch in API_SHAPES:
        w = workloads.custom(op, M, N, dt, 1e-6, dy_sigma=1e-2)
        d = workloads.make_inputs(w)

        def forward(impl, x, weight, res):
            if op == "plain":
                return (rmsnorm(x, weight, w.eps) if impl == "ours" else F.rms_norm(x, (N,), weight, w.eps),)
            if impl == "ours":
                return fused_add_rmsnorm(x, res, weight, w.eps)
            res_out = x + res
            return F.rms_norm(res_out, (N,), weight, w.eps), res_out

        def graph(impl):
            weight = d["gamma"].to(dev).requires_grad_()
            x = d["x"].to(dev).requires_grad_()
            res = d["residual"].to(dev).requires_grad_() if op == "fused" else None
            douts = (d["dy"].to(dev),) if op == "plain" else (d["dy"].to(dev), d["dresidual_out"].to(dev))
            inputs = (x, weight) if op == "plain" else (x, res, weight)
            return forward(impl, x, weight, res), douts, inputs, (x, weight, res)

        line = {"api_compare": f"{'rmsnorm_bwd' if op == 'plain' else 'fused_add_bwd'} {M}x{N} {dt}"}
        fns, grads = {}, {}
        for impl in ("ours", "torch"):
            outs, douts, inputs, raw = graph(impl)
            fns[impl] = (lambda o=outs, i=inputs, g=douts: torch.autograd.grad(o, i, g, retain_graph=True))
            grads[impl] = fns[impl]()
            fns[impl]()
        torch.cuda.synchronize()
        runs = {"ours": [], "torch": []}
        for k in range(windows):
            for impl in (("ours", "torch") if k % 2 == 0 else ("torch", "ours")):
                runs[impl].append(time_calls(lambda _: fns[impl](), [None], iters, warmup if k < 2 else 0))
        for impl in ("ours", "torch"):
            line[f"{impl}_us"] = round(statistics.median(runs[impl]) * 1e3, 2)
        # free the timing passes' autograd graphs before capturing new ones
        del fns, outs, douts, inputs, raw
        for impl in ("ours", "torch"):
            line[f"{impl}_gpu_us"] = round(_autograd_graph_us(forward, impl, d, op, dev, True)
                                           - _autograd_graph_us(forward, impl, d, op, dev, False), 2)
        g_o, g_t = grads["ours"], grads["torch"]

        def rdiff(a, b):
            a, b = a.double(), b.double()
            return float((a - b).abs().max() / b.abs().max().clamp_min(1e-30))
        line["dx_rel_diff"] = rdiff(g_o[0], g_t[0])
        line["dweight_rel_diff"] = rdiff(g_o[-1], g_t[-1])
        line["pages_flydsl_us"] = pages_dsl
        line["pages_torch_us"] = pages_torch
        print(json.dumps(line), flush=True)


def _stream_floor_lib():
    """The streaming-floor kernel's library (built beside the library)."""
    import ctypes
    from rmsnorm_bwd_amd import build as B
    if not os.path.exists(B.FLOOR_LIB):
        raise RuntimeError(f"{B.FLOOR_LIB} is missing: build with __graft_entry__.build()")
    L = ctypes.CDLL(B.FLOOR_LIB)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.rmsn_stream_floor.argtypes = [P, P, P, P, I64, I64, I, P]
    L.rmsn_stream_floor.restype = I
    return L


def floor(w, steps=100):
    """What streaming kernels of the backward's read/write mix reach at the
    workload's shape, on the same box, timed like the backward (one HIP-graph
    replay of `steps` calls over buffer sets rotated past the memory-side
    cache): torch's add (two reads, one write: the plain and LayerNorm
    backward's row traffic) and addcmul (three reads, one write: the fused
    backward with a dresidual_out), a device-to-device copy, and the
    backward's own window ring with its arithmetic replaced by out = a + b
    (+ c) (rmsn_stream_floor: same row plan, grid, ring depth, prologue and
    cache bits; no row reduction, no weight-gradient partials, no finalize).
    One JSON line."""
    dev = torch.device("cuda:0")
    T, s = w.torch_dtype, w.elem_bytes
    per = 4 * w.M * w.N * s
    nsets = max(2, min(steps, -(-ROTATE_BYTES // per)))
    sets = [[torch.randn(w.M, w.N, device=dev).to(T) for _ in range(4)] for _ in range(nsets)]
    mn = w.M * w.N * s
    out = {"floor": w.name, "M": w.M, "N": w.N, "dtype": w.dtype, "buffer_sets": nsets,
           "timing": "HIP graph replay, rotated sets"}
    ring = _stream_floor_lib()
    code = {"f32": 0, "f16": 1, "bf16": 2}[w.dtype]

    def ring_call(t, nr):
        st = ring.rmsn_stream_floor(t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr() if nr == 3 else None,
                                    t[3].data_ptr(), w.M, w.N, code, torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"rmsn_stream_floor: status {st}")
    for name, fn, nbytes in (
            ("copy", lambda t: t[3].copy_(t[0]), 2 * mn),
            ("add_2r1w", lambda t: torch.add(t[0], t[1], out=t[3]), 3 * mn),
            ("addcmul_3r1w", lambda t: torch.addcmul(t[0], t[1], t[2], out=t[3]), 4 * mn),
            ("ring_2r1w", lambda t: ring_call(t, 2), 3 * mn),
            ("ring_3r1w", lambda t: ring_call(t, 3), 4 * mn)):
        us = time_graph(fn, sets, steps, 5) * 1e3
        out[name + "_us"] = round(us, 2)
        out[name + "_GBps"] = round(nbytes / us / 1e3, 1)
        if name.startswith("ring"):
            # the ring moved every byte: its output is the fp32 sum, rounded once
            t = sets[0]
            fn(t)
            want = t[0].float() + t[1].float()
            if name == "ring_3r1w":
                want = want + t[2].float()
            torch.cuda.synchronize()
            out[name + "_exact"] = bool(torch.equal(t[3], want.to(T)))
    abytes = algorithmic_bytes(w)
    out["bwd_algorithmic_bytes"] = abytes
    key = "ring_3r1w" if w.op == "fused" else "ring_2r1w"
    out["bwd_at_ring_floor_rate_us"] = round(abytes / out[key + "_GBps"] / 1e3, 2)
    print(json.dumps(out), flush=True)
    del sets
    torch.cuda.empty_cache()


def ring_floor(w, sets, timer, steps, warmup):
    """The backward's row traffic alone through its own window ring
    (rmsn_stream_floor over the same buffer sets: x or added, dy and, for
    the fused variant, dresidual_out read, dx written; no reduction, no
    partials, no finalize), timed like the backward: what the ring itself
    delivers at this shape."""
    lib = _stream_floor_lib()
    code = {"f32": 0, "f16": 1, "bf16": 2}[w.dtype]

    def call(s):
        st = lib.rmsn_stream_floor(s["x"].data_ptr(), s["dy"].data_ptr(),
                                   s["dres"].data_ptr() if s["dres"] is not None else None,
                                   s["dx"].data_ptr(), w.M, w.N, code, torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"rmsn_stream_floor: status {st}")
    us = timer(call, sets, steps, warmup) * 1e3
    nbytes = (4 if w.op == "fused" else 3) * w.M * w.N * w.elem_bytes
    return {"us": round(us, 2), "row_GBps": round(nbytes / us / 1e3, 1),
            "what": "the row bytes through the same window ring, without the arithmetic"}


def _oracle_call(w, d):
    """A function running the CPU oracle's backward on rows [r0, r1) of the
    workload (the forward's statistics computed once beforehand), returning
    its fp64 weight gradient(s) for those rows."""
    import oracle
    if w.op == "plain":
        rstd, _ = oracle.rmsnorm_fwd(d["x"], d["gamma"], w.eps, want_y=False)
        return lambda r0, r1: oracle.rmsnorm_bwd(d["x"][r0:r1], d["gamma"], d["dy"][r0:r1],
                                                 rstd[r0:r1])[1:]
    if w.op == "layernorm":
        mean, rstd, _ = oracle.layernorm_fwd(d["x"], d["gamma"], d["beta"], w.eps, want_y=False)
        return lambda r0, r1: oracle.layernorm_bwd(d["x"][r0:r1], d["gamma"], d["dy"][r0:r1],
                                                   mean[r0:r1], rstd[r0:r1])[1:]
    added, rstd, _ = oracle.fused_add_rmsnorm_fwd(d["x"], d["residual"], d["gamma"], w.eps,
                                                  want_out=False)
    return lambda r0, r1: oracle.fused_add_rmsnorm_bwd(added[r0:r1], d["gamma"], d["dy"][r0:r1],
                                                       d["dresidual_out"][r0:r1], rstd[r0:r1])[1:]


def _time_median(run, budget_s, max_calls):
    """Median seconds of run() over whole calls repeated for about budget_s
    seconds (at least three calls), and the number of calls."""
    ts = []
    while len(ts) < 3 or (sum(ts) < budget_s and len(ts) < max_calls):
        t0 = time.perf_counter()
        run()
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts), ts


def host_threads(cap=16):
    """The CPUs this process may run on, at most `cap` (a GPU machine's CPU share
    is 16, whatever the host has)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def cpu_baseline(w, d, budget_s=8.0, max_calls=200):
    """The CPU oracle (fp64 C, single-threaded code, unchanged) on the same
    workload, timed two ways: one thread running whole calls, and the host
    threads (up to 16, never more than the rows) each running the oracle on
    its own contiguous shard of rows, the shards' fp64 weight gradients
    summed afterwards (the oracle call releases the interpreter lock, so the
    shards run in parallel). Each way repeats whole calls for about
    `budget_s` seconds and reports the median per call; `value` and `cores`
    are the faster of the two (for a few rows, handing shards to threads
    costs more than the work)."""
    from concurrent.futures import ThreadPoolExecutor
    call = _oracle_call(w, d)
    abytes = algorithmic_bytes(w)
    t1, ts1 = _time_median(lambda: call(0, w.M), budget_s, max_calls)
    nt = max(1, min(host_threads(), w.M))
    bounds = [(w.M * i // nt, w.M * (i + 1) // nt) for i in range(nt)]
    with ThreadPoolExecutor(nt) as ex:
        def sharded():
            parts = list(ex.map(lambda b: call(*b), bounds))
            return [sum(p[q] for p in parts) for q in range(len(parts[0]))]
        tn, tsn = _time_median(sharded, budget_s, max_calls)
    legs = {
        "one_thread": {"value": round(t1 * 1e6, 1), "unit": "us/call", "cores": 1,
                       "sample": f"{len(ts1)} whole calls ({sum(ts1):.1f} s), median",
                       "GBps": round(abytes / (t1 * 1e6) / 1e3, 2)},
        "all_threads": {"value": round(tn * 1e6, 1), "unit": "us/call", "cores": nt,
                        "sample": f"{len(tsn)} calls ({sum(tsn):.1f} s), each {nt} threads running the "
                                  f"oracle on 1/{nt} of the rows, median",
                        "GBps": round(abytes / (tn * 1e6) / 1e3, 2)},
    }
    best = legs["all_threads"] if tn <= t1 else legs["one_thread"]
    return {"value": best["value"], "unit": "us/call", "cores": best["cores"], "kind": "oracle",
            "sample": f"the full {w.M}x{w.N} {w.dtype} workload, fp64 C oracle; the faster of one thread "
                      f"({legs['one_thread']['value']} us) and {nt} threads on row shards "
                      f"({legs['all_threads']['value']} us), median of whole calls",
            "GBps": best["GBps"], **legs,
            "host": {"cpu_model": _cpu_model(), "logical_cpus": os.cpu_count()}}


def _cpu_model():
    """The host CPU's model name (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def load_traffic(w):
    """HBM bytes per launch from committed rocprofv3 PMC summaries, when they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    from hashlib import sha256
    src = b"".join(open(os.path.join(ROOT, "rmsnorm_bwd_amd", "csrc", f), "rb").read()
                   for f in ("kernels.hip", "long_rows.hip", "device.h", "plan.h", "capi.cpp"))
    if rec.get("source_sha256") != sha256(src).hexdigest():
        return None
    return rec.get("hbm_bytes_per_call")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=workloads.HEADLINE)
    ap.add_argument("--hot", action="store_true", help="time one buffer set only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--mode-sweep", action="store_true",
                    help="time the dgamma modes on an (M, N) grid (one JSON line per shape) and exit")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="time the backward and forward of --sweep-ops on an (M, N) grid "
                         "(one JSON line per shape) and exit")
    ap.add_argument("--sweep-n", default="1024,2048,4096,8192",
                    help="row lengths of --shape-sweep (comma-separated)")
    ap.add_argument("--sweep-dtype", default="bf16", choices=("bf16", "f16", "f32"),
                    help="element type of --shape-sweep")
    ap.add_argument("--sweep-m", default="1,128,512,1024,4096,16384,32768",
                    help="row counts of --shape-sweep (comma-separated)")
    ap.add_argument("--sweep-ops", default="plain,fused",
                    help="operations of --shape-sweep (comma-separated: plain, fused, layernorm)")
    ap.add_argument("--api-compare", action="store_true",
                    help="time the backward through autograd against torch's eager RMSNorm on the "
                         "pages' public-API shapes (one JSON line per shape) and exit")
    ap.add_argument("--floor", action="store_true",
                    help="time torch's copy, add and addcmul at the workload's shape (streaming "
                         "kernels of the backward's read/write mix) and exit")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the copy-bandwidth and one-row latency figures (profiled runs)")
    ap.add_argument("--graph", action="store_true",
                    help="time every loop as one replay of a HIP graph of the calls (kernels back "
                         "to back, as a profiler's kernel trace then sees them); value stays "
                         "the per-call time of that replay")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one device-to-device copy of MIB MiB (a kernel of "
                         "known traffic, to scale hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(dgamma would need one all-reduce per step across GPUs).", file=sys.stderr)
        sys.exit(2)

    if args.mode_sweep:
        mode_sweep()
        return
    if args.api_compare:
        api_compare()
        return
    if args.shape_sweep:
        shape_sweep(ns=[int(v) for v in args.sweep_n.split(",")],
                    ms=[int(v) for v in args.sweep_m.split(",")], dtype=args.sweep_dtype,
                    ops=args.sweep_ops.split(","))
        return
    if args.floor:
        floor(workloads.WORKLOADS[args.workload])
        return

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    w = workloads.WORKLOADS[args.workload]
    d = workloads.make_inputs(w)
    # row tensors a set holds on the device: x (or added), dy, dx, and
    # dresidual_out for the fused variant
    per_set = (4 if w.op == "fused" else 3) * w.M * w.N * w.elem_bytes
    nsets = 1 if args.hot else max(2, -(-ROTATE_BYTES // per_set))
    g, sets = make_sets(w, d, nsets)
    bwd = lambda s: call_bwd(w, g, s)  # noqa: E731
    timer = time_graph if args.graph else time_calls
    ms = timer(bwd, sets, args.steps, args.warmup)
    ms_hot = ms if args.hot else timer(bwd, sets[:1], args.steps, args.warmup)
    # the other timing method on the same calls, for comparison (skipped in
    # profiled runs, which trace only the chosen one)
    ms_other = None if args.no_extras else (time_calls if args.graph else time_graph)(bwd, sets, args.steps, 2)

    def fwd(s):
        if w.op == "plain":
            R.rmsnorm_fwd_rstd(s["x"], g, w.eps, y=s["dx"], rstd=s["rstd"])
        elif w.op == "layernorm":
            R.layernorm_fwd_stats(s["x"], g, s["beta"], w.eps, y=s["dx"], mean=s["mean"], rstd=s["rstd"])
        else:
            R.fused_add_rmsnorm_fwd_rstd(s["x"], s["dy"], g, w.eps, out=s["dx"],
                                         residual_out=s["dres"], rstd=s["rstd"])
    ms_fwd = timer(fwd, sets, args.steps, args.warmup)

    abytes = algorithmic_bytes(w)
    gbps = abytes / (ms * 1e-3) / 1e9
    # the copy and the one-row case are skipped under the counter runs, whose
    # only copy must be the calibration copy
    skip = args.copy_calibration or args.no_extras
    copy_gbps = None if skip else copy_bandwidth()
    latency = None if skip else latency_floor()
    ring = None if skip else ring_floor(w, sets, timer, args.steps, args.warmup)
    line = {
        "metric": "rmsnorm_bwd us/call + achieved HBM GB/s (% of peak), 4096x4096 bf16"
                  if w.name == workloads.HEADLINE
                  else f"{OP_NAMES[w.op]} us/call + achieved HBM GB/s (% of peak), {w.M}x{w.N} {w.dtype}",
        "value": round(ms * 1e3, 2),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type: every sum, product and reduction is fp32; the
        # rows are stored in config.dtype
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "op": w.op, "M": w.M, "N": w.N, "dtype": w.dtype,
                   "eps": w.eps, "buffer_sets": nsets,
                   "rotated_MiB": round(nsets * per_set / 2 ** 20),
                   "timing": ("hot" if args.hot else "rotated over > 512 MiB")
                   + ("; HIP graph replay" if args.graph else "; eager calls")},
        "achieved_GBps": round(gbps, 1),
        "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 1),
        "hot_cache_us": round(ms_hot * 1e3, 2),
        ("eager_us" if args.graph else "graph_us"): round(ms_other * 1e3, 2) if ms_other else None,
        "copy_GBps": round(copy_gbps, 1) if copy_gbps else None,
        "pct_of_copy": round(100 * gbps / copy_gbps, 1) if copy_gbps else None,
        "latency": latency,
        "ring_floor": ring,
        "pct_of_ring_floor": round(100 * ring["us"] / (ms * 1e3), 1) if ring else None,
        "fwd_rstd_us": round(ms_fwd * 1e3, 2),
        "fwd_rstd_GBps": round(fwd_bytes(w) / (ms_fwd * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic(w),
                     "kernel": f"one {'layernorm' if w.op == 'layernorm' else 'rmsnorm'}_bwd call "
                               "(main pass + weight-gradient finalize)",
                     "algorithmic_bytes": abytes},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, d)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
