"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding on seeded inputs and compare it with the CPU oracle.

Tolerances (normwise infinity-relative error, max|got - ref| / max|ref|,
against the oracle's unrounded fp64 result):
  dx, y, out:  1e-5 for fp32, 2e-2 for fp16/bf16
  dgamma_f32:  1e-4 * sqrt(M)
  rstd:        1e-5, element by element
  residual_out: bit-exact
Half-precision dx/y are also held, element by element, within one unit in the
last place of the dtype plus 1e-5 of the tensor's scale: one rounding of an
fp32 result whose own error is far below an ulp.

dgamma_f32 is also held column by column to the error bound of an fp32 sum
(see sum_bound): the normwise 1e-4*sqrt(M) alone would let one row's
contribution go missing at large M, the bound does not.
"""
import math

import torch

import oracle
import rmsnorm_bwd_amd as R
import workloads

F64 = torch.float64
DEV = torch.device("cuda:0")

TOL = {torch.float32: 1e-5, torch.float16: 2e-2, torch.bfloat16: 2e-2}
MANT = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}


def rel(got, ref):
    got = got.detach().to("cpu", F64)
    ref = ref.to(F64)
    den = ref.abs().max().item() if ref.numel() else 0.0
    err = (got - ref).abs().max().item() if ref.numel() else 0.0
    return err / (den if den > 0 else 1.0)


def tol_dgamma(M):
    return 1e-4 * math.sqrt(max(M, 1))


def sum_depth(M):
    """Upper bound on the fp32 additions any one row's dgamma term passes
    through in the library: its row group's running sum (rows of a group,
    at most M with one block, at most ceil(M / 128) once the grid holds 128
    or more blocks, which every call of more than 8192 rows does), then the
    fold of at most 16 row groups and the sum over at most 256 block
    partials (in a fixed order, or by atomics in any order), plus the two
    roundings of forming the term."""
    per_group = M if M <= 8192 else -(-M // 128)
    return per_group + 16 + 256 + 2


def sum_bound(abs_sum, M):
    """Per-column bound on |fp32 sum - exact sum| for M terms of absolute sum
    abs_sum: first-order error analysis of summation, depth * 2^-24 *
    sum |t|, with a quarter's margin for second-order terms."""
    return 1.25 * sum_depth(M) * 2.0 ** -24 * abs_sum


def assert_sum_bound(name, got, ref, abs_sum, M):
    """Every column of an fp32 weight gradient within the summation bound of
    the oracle's fp64 value."""
    err = (got.detach().to("cpu", F64) - ref.to(F64)).abs()
    bound = sum_bound(abs_sum.to(F64), M) + 1e-30
    bad = err > bound
    assert not bad.any(), (f"{name}: {int(bad.sum())} columns beyond the fp32 summation bound "
                           f"(worst ratio {float((err / bound).max()):.3g})")


def term_abs_sum(x, dy, rstd):
    """sum_i |dy[i, j] * x[i, j] * rstd[i]| per column (fp64, CPU): the
    absolute sum of dgamma's terms."""
    return (dy.to(F64) * x.to(F64) * rstd.to(F64)[:, None]).abs().sum(0)


def assert_close(name, got, ref, dtype, scale=None):
    """Normwise check against the tolerance; `scale` replaces max|ref| as the
    denominator where the result is a cancellation of much larger terms."""
    if scale is None:
        e = rel(got, ref)
    else:
        e = (got.detach().to("cpu", F64) - ref.to(F64)).abs().max().item() / scale
    assert e <= TOL[dtype], f"{name}: normwise error {e:.3g} > {TOL[dtype]:.3g}"
    if dtype != torch.float32:
        g = got.detach().to("cpu", F64)
        r = ref.to(F64)
        mag = r.abs().clamp_min(torch.finfo(dtype).tiny)
        ulp = torch.exp2(torch.floor(torch.log2(mag)) - MANT[dtype])
        bound = ulp + 1e-5 * (scale if scale is not None else r.abs().max())
        bad = (g - r).abs() > bound
        assert not bad.any(), f"{name}: {int(bad.sum())} elements beyond 1 ulp"
    return e


def place(t, misalign=False):
    """Copy a CPU tensor to the GPU; with misalign, at an address one element
    past a 256-byte boundary (still element-aligned)."""
    if not misalign:
        return t.to(DEV).contiguous()
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
    v = buf[1:].view(t.shape)
    v.copy_(t.to(DEV))
    return v


def empty_like_dev(shape, dtype, misalign=False):
    if not misalign:
        return torch.empty(shape, dtype=dtype, device=DEV)
    n = 1
    for s in shape:
        n *= s
    return torch.empty(n + 1, dtype=dtype, device=DEV)[1:].view(shape)


def plain_case(w, flags=R.DGAMMA_AUTO, misalign=False, with_dgamma_t=True):
    """Run forward and backward of a plain workload on the GPU and return a
    dict of (gpu, oracle) results."""
    d = workloads.make_inputs(w)
    x, g, dy = d["x"], d["gamma"], d["dy"]
    M, N, T = w.M, w.N, w.torch_dtype
    r_ref, y_ref = oracle.rmsnorm_fwd(x, g, w.eps)
    xg, gg, dyg = place(x, misalign), place(g, misalign), place(dy, misalign)
    yg = empty_like_dev((M, N), T, misalign)
    y, rstd = R.rmsnorm_fwd_rstd(xg, gg, w.eps, y=yg)
    dxg = empty_like_dev((M, N), T, misalign)
    dgt = torch.empty(N, dtype=T, device=DEV) if with_dgamma_t else None
    dx, dg32, dgt = R.rmsnorm_bwd(xg, gg, dyg, r_ref.to(DEV), dx=dxg, dgamma=dgt, flags=flags)
    torch.cuda.synchronize()
    dx_ref, dg_ref = oracle.rmsnorm_bwd(x, g, dy, r_ref)
    return dict(M=M, N=N, T=T, y=(y, y_ref), rstd=(rstd, r_ref), dx=(dx, dx_ref),
                dg32=(dg32, dg_ref), dgt=dgt, inputs=(xg, gg, dyg, r_ref.to(DEV)),
                abs_sum=term_abs_sum(x, dy, r_ref))


def fused_case(w, flags=R.DGAMMA_AUTO, misalign=False, with_dres=True, with_dgamma_t=True):
    d = workloads.make_inputs(w)
    x, res, g, dy = d["x"], d["residual"], d["gamma"], d["dy"]
    dres = d["dresidual_out"] if with_dres else None
    M, N, T = w.M, w.N, w.torch_dtype
    a_ref, r_ref, o_ref = oracle.fused_add_rmsnorm_fwd(x, res, g, w.eps)
    xg, resg, gg, dyg = (place(t, misalign) for t in (x, res, g, dy))
    dresg = place(dres, misalign) if dres is not None else None
    out, res_out, rstd = R.fused_add_rmsnorm_fwd_rstd(
        xg, resg, gg, w.eps, out=empty_like_dev((M, N), T, misalign),
        residual_out=empty_like_dev((M, N), T, misalign))
    ag = place(a_ref, misalign)
    dgt = torch.empty(N, dtype=T, device=DEV) if with_dgamma_t else None
    dx, dg32, dgt = R.fused_add_rmsnorm_bwd(ag, gg, dyg, dresg, r_ref.to(DEV),
                                            dx=empty_like_dev((M, N), T, misalign), dgamma=dgt,
                                            flags=flags)
    torch.cuda.synchronize()
    dx_ref, dg_ref = oracle.fused_add_rmsnorm_bwd(a_ref, g, dy, dres, r_ref)
    return dict(M=M, N=N, T=T, y=(out, o_ref), rstd=(rstd, r_ref), dx=(dx, dx_ref),
                dg32=(dg32, dg_ref), dgt=dgt, added=(res_out, a_ref),
                inputs=(ag, gg, dyg, dresg, r_ref.to(DEV)), abs_sum=term_abs_sum(a_ref, dy, r_ref))


def check_case(c, check_fwd=True):
    T, M = c["T"], c["M"]
    if check_fwd and M > 0:
        rstd, r_ref = c["rstd"]
        er = ((rstd.cpu().double() - r_ref.double()).abs() / r_ref.double().abs()).max().item()
        assert er <= 1e-5, f"rstd: error {er:.3g}"
        assert_close("y", c["y"][0], c["y"][1], T)
        if "added" in c:
            assert torch.equal(c["added"][0].cpu(), c["added"][1]), "residual_out not bit-exact"
    if M > 0:
        if c["N"] == 1:
            # one column: dx = gamma*dy*eps*rstd^3 is what is left after
            # gamma*dy*rstd cancels almost entirely, so its error is measured
            # against the magnitude of those terms
            xg, gg, dyg = c["inputs"][:3]
            rg = c["inputs"][-1]
            scale = (dyg.double() * gg.double() * rg.double()[:, None]).abs().max().item()
            assert_close("dx", c["dx"][0], c["dx"][1], T, scale=scale)
        else:
            assert_close("dx", c["dx"][0], c["dx"][1], T)
    dg32, dg_ref = c["dg32"]
    e = rel(dg32, dg_ref)
    assert e <= tol_dgamma(M), f"dgamma: error {e:.3g} > {tol_dgamma(M):.3g}"
    if M > 0 and "abs_sum" in c:
        assert_sum_bound("dgamma", dg32, dg_ref, c["abs_sum"], M)
    if c["dgt"] is not None:
        # the dtype copy is exactly the RNE rounding of the fp32 result
        assert torch.equal(c["dgt"].cpu(), dg32.cpu().to(T))
