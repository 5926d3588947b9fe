"""Seeded synthetic inputs and the named workloads (shapes, dtypes, eps,
value distributions) shared by the tests and the benchmark.

This module holds input generation only: no step of the RMSNorm or LayerNorm
arithmetic is here. Both the CPU oracle and the GPU library consume the exact bits it
produces.

Recipe: one ``numpy.random.Generator(PCG64(seed))`` per workload; each tensor,
in the order a workload lists them, is drawn as float32 ``standard_normal``
values in row-major order, mapped to ``mu + sigma * z`` in float32 (sigma is a
standard deviation), then rounded to the workload's dtype with torch's
round-to-nearest-even conversion. Large tensors are drawn in chunks, which
yields the same stream as one draw.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_CHUNK = 1 << 24


@dataclass(frozen=True)
class Workload:
    """One named problem: op ("plain" or "fused" RMSNorm, or "layernorm"),
    shape, dtype, eps, and the (mu, sigma) of every input in draw order."""
    name: str
    op: str
    M: int
    N: int
    dtype: str
    eps: float
    dists: tuple = field(default=())
    seed: int = 0

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    @property
    def elem_bytes(self):
        return 4 if self.dtype == "f32" else 2


def _plain(name, M, N, dtype, eps, dy_sigma):
    return Workload(name, "plain", M, N, dtype, eps,
                    (("x", 0.0, 1.0), ("gamma", 1.0, 0.1), ("dy", 0.0, dy_sigma)))


def _fused(name, M, N, dtype, eps):
    return Workload(name, "fused", M, N, dtype, eps,
                    (("x", 0.0, 1.0), ("residual", 0.0, 1.0), ("gamma", 1.0, 0.1),
                     ("dy", 0.0, 1e-2), ("dresidual_out", 0.0, 1e-2)))


def _layernorm(name, M, N, dtype, eps):
    # x with a nonzero mean, so that the mean matters
    return Workload(name, "layernorm", M, N, dtype, eps,
                    (("x", 0.5, 1.0), ("gamma", 1.0, 0.1), ("beta", 0.0, 0.1), ("dy", 0.0, 1e-2)))


# The workloads the library is specified, tested and measured on.
WORKLOADS = {w.name: w for w in (
    _plain("plain_8x256_f32", 8, 256, "f32", 1e-5, 1.0),
    _plain("plain_512x3000_f32", 512, 3000, "f32", 1e-5, 1.0),
    _plain("plain_512x2048_bf16", 512, 2048, "bf16", 1e-5, 1.0),
    _plain("plain_4096x4096_bf16", 4096, 4096, "bf16", 1e-6, 1e-2),
    _fused("fused_1024x8192_bf16", 1024, 8192, "bf16", 1e-6),
    _fused("fused_32768x8192_bf16", 32768, 8192, "bf16", 1e-6),
    _plain("plain_1x4096_bf16", 1, 4096, "bf16", 1e-6, 1e-2),
    _layernorm("layernorm_4096x4096_bf16", 4096, 4096, "bf16", 1e-6),
)}

HEADLINE = "plain_4096x4096_bf16"


def normal(gen, shape, mu, sigma, dtype):
    """Draw ``mu + sigma * z`` (z standard normal, float32) and round to dtype."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=dtype)
    done = 0
    while done < n:
        k = min(_CHUNK, n - done)
        z = gen.standard_normal(k, dtype=np.float32)
        v = np.float32(mu) + np.float32(sigma) * z
        out[done:done + k] = torch.from_numpy(v).to(dtype)
        done += k
    return out.reshape(shape)


def make_inputs(w, M=None, N=None, seed=None):
    """Return a dict of CPU tensors for workload ``w`` (shape overridable)."""
    M = w.M if M is None else M
    N = w.N if N is None else N
    gen = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    out = {}
    for name, mu, sigma in w.dists:
        shape = (N,) if name in ("gamma", "beta") else (M, N)
        out[name] = normal(gen, shape, mu, sigma, w.torch_dtype)
    return out


def custom(op, M, N, dtype, eps, seed=0, dy_sigma=1.0):
    """A workload of the plain, fused or LayerNorm kind at an arbitrary shape."""
    if op == "plain":
        w = _plain(f"plain_{M}x{N}_{dtype}", M, N, dtype, eps, dy_sigma)
    elif op == "layernorm":
        w = _layernorm(f"layernorm_{M}x{N}_{dtype}", M, N, dtype, eps)
    elif op == "fused":
        w = _fused(f"fused_{M}x{N}_{dtype}", M, N, dtype, eps)
    else:
        raise ValueError(f"unknown operation {op!r}")
    return Workload(w.name, w.op, w.M, w.N, w.dtype, w.eps, w.dists, seed)
