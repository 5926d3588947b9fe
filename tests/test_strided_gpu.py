"""GPU parity of the strided entry points: every row tensor may be a view
whose rows are N elements of unit stride under a row stride ld >= N (a slice
of wider rows, a column block). Results are held to the CPU oracle on the
same values laid out contiguously, and the gaps between rows of every output
view must keep their sentinel (nothing outside the rows is written).

Strides are chosen to cover both paths: byte strides that are multiples of
16 keep the 16-byte vector path, others take the element path; and every row
plan (rows inside one wavefront, several rows a block window, one row a
window, several chunks a thread).

Math: FlyDSL issue #769 ("[Feature] Add rmsnorm backward (+ forward saves
rstd) ..."), Implementation plan: Math, and PR sequence (LayerNorm); FlyDSL
PR #800 ("[rmsnorm] Add fused-add / residual backward (PR 2/3, #769)"),
fused-add commit; the review-fix commit's contiguity assertion is what the
strided entry points relax.
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_bwd_amd as R
import workloads
from parity_util import DEV, assert_close, rel, tol_dgamma

pytestmark = pytest.mark.gpu

T = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
SENTINEL = 7.0


def embed(t, pad):
    """A GPU view of CPU tensor t (M, N) inside rows of N + pad elements, the
    gaps filled with SENTINEL. Returns (view, whole buffer)."""
    M, N = t.shape
    buf = torch.full((M, N + pad), SENTINEL, dtype=t.dtype, device=DEV)
    v = buf[:, :N]
    v.copy_(t.to(DEV))
    return v, buf


def out_view(M, N, pad, dt):
    buf = torch.full((M, N + pad), SENTINEL, dtype=dt, device=DEV)
    return buf[:, :N], buf


def gaps_untouched(buf, N):
    return bool((buf[:, N:].float() == SENTINEL).all()) if buf.shape[1] > N else True


def draw(M, N, dt, seed, mu=0.0, sigma=1.0):
    gen = np.random.Generator(np.random.PCG64(seed))
    return workloads.normal(gen, (M, N), mu, sigma, T[dt]).reshape(M, N)


# (M, N, dtype, pads for the row tensors): vector-path pads keep 16-byte rows
BWD_CASES = [
    ("4096x4096_bf16_vec", 4096, 4096, "bf16", (8, 16, 24, 8)),     # one row a window
    ("300x1024_bf16_vec", 300, 1024, "bf16", (8, 0, 40, 16)),       # four rows a window
    ("200x256_f16_vec", 200, 256, "f16", (8, 8, 8, 8)),             # rows inside a wavefront
    ("100x640_f32_vec", 100, 640, "f32", (4, 12, 0, 4)),            # 160 chunks: two rows a window
    ("64x8192_bf16_vec", 64, 8192, "bf16", (64, 8, 8, 8)),          # two chunks a thread
    ("77x1000_bf16_elem", 77, 1000, "bf16", (1, 3, 5, 2)),          # element path
    ("50x4096_f32_elem", 50, 4096, "f32", (1, 0, 3, 0)),            # element path (one odd stride)
    ("20x20000_bf16_long_vec", 20, 20000, "bf16", (8, 16, 0, 8)),   # long rows, 16-byte chunks
    ("9x24577_f32_long_elem", 9, 24577, "f32", (1, 2, 0, 3)),       # long rows, element path
    ("600x24576_bf16_long_vec", 600, 24576, "bf16", (8, 24, 16, 8)),  # long rows, the next row loaded ahead
]


@pytest.mark.parametrize("name,M,N,dt,pads", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_rmsnorm_bwd_strided(name, M, N, dt, pads):
    print("case strided bwd", name, flush=True)
    td = T[dt]
    x, dy = draw(M, N, dt, 1), draw(M, N, dt, 2, 0.0, 1e-2)
    g = workloads.normal(np.random.Generator(np.random.PCG64(3)), (N,), 1.0, 0.1, td)
    r_ref, _ = oracle.rmsnorm_fwd(x, g, 1e-6, want_y=False)
    dx_ref, dg_ref = oracle.rmsnorm_bwd(x, g, dy, r_ref)
    xv, _ = embed(x, pads[0])
    dyv, _ = embed(dy, pads[1])
    dxv, dxbuf = out_view(M, N, pads[2], td)
    dgt = torch.empty(N, dtype=td, device=DEV)
    dx, dg32, dgt = R.rmsnorm_bwd(xv, g.to(DEV), dyv, r_ref.to(DEV), dx=dxv, dgamma=dgt)
    torch.cuda.synchronize()
    assert_close("dx", dx, dx_ref, td)
    assert rel(dg32, dg_ref) <= tol_dgamma(M)
    assert torch.equal(dgt.cpu(), dg32.cpu().to(td))
    assert gaps_untouched(dxbuf, N), "dx wrote between rows"


# the fused backward's own row plans: three chunks a thread, and from 4096
# rows the long-row kernel for rows of 12296-16384 16-bit elements
FUSED_CASES = BWD_CASES[1::2] + [
    ("300x12288_bf16_three_chunk", 300, 12288, "bf16", (8, 0, 16, 8)),
    ("4097x12296_bf16_next_row", 4097, 12296, "bf16", (8, 16, 24, 8)),
]


@pytest.mark.parametrize("name,M,N,dt,pads", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_bwd_strided(name, M, N, dt, pads):
    print("case strided fused bwd", name, flush=True)
    td = T[dt]
    x, res = draw(M, N, dt, 4), draw(M, N, dt, 5)
    dy, dres = draw(M, N, dt, 6, 0.0, 1e-2), draw(M, N, dt, 7, 0.0, 1e-2)
    g = workloads.normal(np.random.Generator(np.random.PCG64(8)), (N,), 1.0, 0.1, td)
    added, r_ref, _ = oracle.fused_add_rmsnorm_fwd(x, res, g, 1e-6, want_out=False)
    dx_ref, dg_ref = oracle.fused_add_rmsnorm_bwd(added, g, dy, dres, r_ref)
    av, _ = embed(added, pads[0])
    dyv, _ = embed(dy, pads[1])
    drv, _ = embed(dres, pads[3])
    dxv, dxbuf = out_view(M, N, pads[2], td)
    dx, dg32, _ = R.fused_add_rmsnorm_bwd(av, g.to(DEV), dyv, drv, r_ref.to(DEV), dx=dxv)
    torch.cuda.synchronize()
    assert_close("dx", dx, dx_ref, td)
    assert rel(dg32, dg_ref) <= tol_dgamma(M)
    assert gaps_untouched(dxbuf, N)


# the plain forward's 256-thread groups (rows of 4104-6144 16-bit elements
# from 4096 rows) and the forwards' 128-thread groups (2056-3072 elements from
# 3072 rows), single wavefronts (1032-1536 elements) and 32-thread groups
# (520-768 elements), on padded rows
FWD_CASES = BWD_CASES[::2] + [("4097x5120_bf16_half_rows", 4097, 5120, "bf16", (8, 16, 24, 8)),
                              ("3073x2560_bf16_quarter_rows", 3073, 2560, "bf16", (16, 8, 8, 24)),
                              ("2049x1280_bf16_wave_rows", 2049, 1280, "bf16", (8, 24, 16, 8)),
                              ("301x768_bf16_narrow_rows", 301, 768, "bf16", (8, 8, 24, 16))]


@pytest.mark.parametrize("name,M,N,dt,pads", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_strided(name, M, N, dt, pads):
    print("case strided fwd", name, flush=True)
    td = T[dt]
    eps = 1e-5
    x, res = draw(M, N, dt, 9), draw(M, N, dt, 10)
    g = workloads.normal(np.random.Generator(np.random.PCG64(11)), (N,), 1.0, 0.1, td)
    gg = g.to(DEV)
    # plain
    r_ref, y_ref = oracle.rmsnorm_fwd(x, g, eps)
    xv, _ = embed(x, pads[0])
    yv, ybuf = out_view(M, N, pads[2], td)
    y, rstd = R.rmsnorm_fwd_rstd(xv, gg, eps, y=yv)
    # fused
    added, r2_ref, o_ref = oracle.fused_add_rmsnorm_fwd(x, res, g, eps)
    rv, _ = embed(res, pads[1])
    ov, obuf = out_view(M, N, pads[3], td)
    rov, robuf = out_view(M, N, pads[0], td)
    out, res_out, rstd2 = R.fused_add_rmsnorm_fwd_rstd(xv, rv, gg, eps, out=ov, residual_out=rov)
    torch.cuda.synchronize()
    assert_close("y", y, y_ref, td)
    assert ((rstd.cpu().double() - r_ref.double()).abs() / r_ref.double()).max() <= 1e-5
    assert_close("out", out, o_ref, td)
    assert torch.equal(res_out.cpu(), added)
    assert ((rstd2.cpu().double() - r2_ref.double()).abs() / r2_ref.double()).max() <= 1e-5
    for buf in (ybuf, obuf, robuf):
        assert gaps_untouched(buf, N)


LN_CASES = BWD_CASES[:5] + [("300x14336_bf16_next_row", 300, 14336, "bf16", (8, 16, 24, 8)),
                            ("130x10240_bf16_three_chunks", 130, 10240, "bf16", (8, 24, 16, 8)),
                            ("3074x3072_bf16_quarter_rows", 3074, 3072, "bf16", (24, 8, 16, 8)),
                            ("130x1536_bf16_wave_rows", 130, 1536, "bf16", (8, 16, 8, 24)),
                            ("70x640_bf16_narrow_rows", 70, 640, "bf16", (16, 8, 24, 8))]


@pytest.mark.parametrize("name,M,N,dt,pads", LN_CASES, ids=[c[0] for c in LN_CASES])
def test_layernorm_strided(name, M, N, dt, pads):
    print("case strided layernorm", name, flush=True)
    td = T[dt]
    eps = 1e-5
    x, dy = draw(M, N, dt, 12, 0.5, 1.0), draw(M, N, dt, 13, 0.0, 1e-2)
    gen = np.random.Generator(np.random.PCG64(14))
    g = workloads.normal(gen, (N,), 1.0, 0.1, td)
    b = workloads.normal(gen, (N,), 0.0, 0.1, td)
    mean_ref, rstd_ref, y_ref = oracle.layernorm_fwd(x, g, b, eps)
    dx_ref, dg_ref, db_ref = oracle.layernorm_bwd(x, g, dy, mean_ref, rstd_ref)
    xv, _ = embed(x, pads[0])
    dyv, _ = embed(dy, pads[1])
    yv, ybuf = out_view(M, N, pads[3], td)
    dxv, dxbuf = out_view(M, N, pads[2], td)
    y, mean, rstd = R.layernorm_fwd_stats(xv, g.to(DEV), b.to(DEV), eps, y=yv)
    dx, dg32, db32, _, _ = R.layernorm_bwd(xv, g.to(DEV), dyv, mean_ref.to(DEV), rstd_ref.to(DEV),
                                           dx=dxv)
    torch.cuda.synchronize()
    assert_close("y", y, y_ref, td)
    assert_close("dx", dx, dx_ref, td)
    assert rel(dg32, dg_ref) <= tol_dgamma(M) and rel(db32, db_ref) <= tol_dgamma(M)
    assert gaps_untouched(ybuf, N) and gaps_untouched(dxbuf, N)


def test_three_dimensional_slice_and_autograd():
    """A 3-D slice of wider rows (its leading dimensions collapse into one row
    stride) goes through the autograd wrapper without a copy of x."""
    print("case strided 3-D autograd", flush=True)
    B, S, N, pad = 4, 6, 768, 32
    x = draw(B * S, N, "bf16", 15)
    g = workloads.normal(np.random.Generator(np.random.PCG64(16)), (N,), 1.0, 0.1, torch.bfloat16)
    up = draw(B * S, N, "bf16", 17, 0.0, 1e-2)
    big = torch.zeros(B, S, N + pad, dtype=torch.bfloat16, device=DEV)
    big[:, :, :N] = x.reshape(B, S, N).to(DEV)
    xv = big[:, :, :N].requires_grad_()
    assert not xv.is_contiguous()
    wg = g.to(DEV).requires_grad_()
    y = R.rmsnorm(xv, wg, 1e-6)
    y.backward(up.reshape(B, S, N).to(DEV))
    torch.cuda.synchronize()
    r_ref, y_ref = oracle.rmsnorm_fwd(x, g, 1e-6)
    dx_ref, dg_ref = oracle.rmsnorm_bwd(x, g, up, r_ref)
    assert_close("y", y.detach().reshape(-1, N), y_ref, torch.bfloat16)
    assert_close("dx", xv.grad.reshape(-1, N), dx_ref, torch.bfloat16)
    assert_close("dweight", wg.grad, dg_ref, torch.bfloat16)


def test_views_the_library_cannot_read_are_refused():
    x = torch.zeros(4, 6, 100, dtype=torch.bfloat16, device=DEV)[:, :5, :64]
    g = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        R.rmsnorm_fwd_rstd(x, g, 1e-5)
    with pytest.raises(ValueError):
        R.rmsnorm_fwd_rstd(torch.zeros(64, 8, dtype=torch.bfloat16, device=DEV).t(), torch.ones(
            64, dtype=torch.bfloat16, device=DEV)[:8].repeat(8), 1e-5)
