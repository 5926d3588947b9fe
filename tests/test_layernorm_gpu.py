"""GPU parity of the LayerNorm forward (saving mean and rstd) and backward
(dx, dgamma, dbeta) through the C ABI, against the CPU oracle.

Shapes cover every row plan: rows inside one wavefront, two and four rows per
block window, one to eight 16-byte chunks per thread, the element path (N not
a multiple of the vector width, and misaligned pointers), a single row, and
no rows. Inputs have a nonzero mean so that the mean handling matters. The
backward reads the oracle's saved statistics, as the RMSNorm parity tests
do; the GPU forward's statistics are checked on their own.

Tolerances: y and dx as for RMSNorm (1e-5 normwise for fp32, 2e-2 plus one
ulp element by element for half types); dgamma and dbeta 1e-4 * sqrt(M)
normwise; rstd 1e-5 per element; the mean within 1e-6 of the row's largest
|x| (an fp32 sum of N terms, whose error is relative to the terms, not to a
mean that may nearly cancel).

Math: FlyDSL issue #769 ("[Feature] Add rmsnorm backward (+ forward saves
rstd) ..."), PR sequence and status updates (the LayerNorm follow-up).
"""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_bwd_amd as R
import workloads
from parity_util import DEV, assert_close, empty_like_dev, place, rel, tol_dgamma

pytestmark = pytest.mark.gpu

T = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

CASES = [
    ("8x256_f32", 8, 256, "f32", 1e-5),        # rows inside one wavefront
    ("100x64_bf16", 100, 64, "bf16", 1e-5),    # 8 chunks: 16-lane groups
    ("257x640_f16", 257, 640, "f16", 1e-5),    # four rows a window, ragged M
    ("512x2048_bf16", 512, 2048, "bf16", 1e-5),  # two rows a window
    ("512x3000_f32", 512, 3000, "f32", 1e-5),  # two chunks a thread, ragged chunks
    ("4096x4096_bf16", 4096, 4096, "bf16", 1e-6),  # one row a window
    ("1024x8192_bf16", 1024, 8192, "bf16", 1e-6),  # two chunks a thread
    ("64x16384_f16", 64, 16384, "f16", 1e-6),  # four chunks a thread
    ("33x16384_f32", 33, 16384, "f32", 1e-6),  # eight chunks a thread
    ("300x1001_f32", 300, 1001, "f32", 1e-5),  # element path
    ("1x4096_bf16", 1, 4096, "bf16", 1e-6),    # one block writes the gradients
    ("150x1500_f16", 150, 1500, "f16", 1e-5),  # element path, 256 threads, 8 elements a thread
    ("200x4097_bf16", 200, 4097, "bf16", 1e-5),  # element path, 512 threads, 16 elements a thread
    ("300x10240_bf16", 300, 10240, "bf16", 1e-6),  # three chunks a thread (backward and forward)
    ("129x12288_f16", 129, 12288, "f16", 1e-6),  # three chunks a thread, the longest such row
    ("2050x8200_bf16", 2050, 8200, "bf16", 1e-6),  # three chunks a thread, the shortest such row
    ("3075x2560_bf16", 3075, 2560, "bf16", 1e-6),  # forward on 128-thread groups, ragged last window
    ("4098x3072_f16", 4098, 3072, "f16", 1e-6),  # forward on 128-thread groups, the longest such row
    ("3071x2056_bf16", 3071, 2056, "bf16", 1e-6),  # one row short: the forward keeps the plan
    ("1023x1536_bf16", 1023, 1536, "bf16", 1e-6),  # forward on one wavefront a row, ragged last window
    ("5x1032_f16", 5, 1032, "f16", 1e-6),  # forward on one wavefront a row, the shortest such row
    ("1x768_bf16", 1, 768, "bf16", 1e-6),  # forward on 32-thread groups, one row
    ("1031x520_f16", 1031, 520, "f16", 1e-6),  # forward on 32-thread groups, ragged last window
    ("1x640_f32", 1, 640, "f32", 1e-6),  # fp32 forward on one wavefront a row
    ("3073x1536_f32", 3073, 1536, "f32", 1e-6),  # fp32 forward on 128-thread groups, ragged last window
    ("130x384_f32", 130, 384, "f32", 1e-6),  # fp32 forward on 32-thread groups
    ("3071x1028_f32", 3071, 1028, "f32", 1e-6),  # one row short: the fp32 forward keeps the plan
    ("1025x384_bf16", 1025, 384, "bf16", 1e-6),  # forward with three chunks on 16-thread groups
    ("65x4100_f32", 65, 4100, "f32", 1e-6),  # fp32 LayerNorm keeps four chunks a thread here
    ("40x12296_bf16", 40, 12296, "bf16", 1e-6),  # one chunk past: four chunks a thread, next-row kernel
    ("4099x12296_bf16", 4099, 12296, "bf16", 1e-6),  # next-row kernel, ragged M
    ("300x16384_f16", 300, 16384, "f16", 1e-6),  # full rows, next-row kernel (M * N <= 2^26)
    ("4100x16384_bf16", 4100, 16384, "bf16", 1e-6),  # full rows past 2^26 elements: main kernel
    ("65x14336_bf16", 65, 14336, "bf16", 1e-6),  # next-row kernel, fewer rows than blocks
]


def _inputs(M, N, dt, seed=31, with_beta=True):
    gen = np.random.Generator(np.random.PCG64(seed))
    td = T[dt]
    x = workloads.normal(gen, (M, N), 0.5, 1.0, td).reshape(M, N)
    g = workloads.normal(gen, (N,), 1.0, 0.1, td)
    b = workloads.normal(gen, (N,), 0.0, 0.1, td) if with_beta else None
    dy = workloads.normal(gen, (M, N), 0.0, 1e-2, td).reshape(M, N)
    return x, g, b, dy


def run_case(M, N, dt, eps, flags=R.DGAMMA_AUTO, misalign=False, with_beta=True, seed=31, scale_exp=0):
    x, g, b, dy = _inputs(M, N, dt, seed, with_beta)
    td = T[dt]
    if scale_exp:
        xs = (x.double() * 2.0 ** scale_exp).to(td)
        assert torch.equal(xs.double() / 2.0 ** scale_exp, x.double())  # exact scaling
        x = xs
    mean_ref, rstd_ref, y_ref = oracle.layernorm_fwd(x, g, b, eps)
    dx_ref, dg_ref, db_ref = oracle.layernorm_bwd(x, g, dy, mean_ref, rstd_ref)
    xg, gg, dyg = place(x, misalign), place(g, misalign), place(dy, misalign)
    bg = place(b, misalign) if b is not None else None
    y, mean, rstd = R.layernorm_fwd_stats(xg, gg, bg, eps, y=empty_like_dev((M, N), td, misalign))
    dgt = torch.empty(N, dtype=td, device=DEV)
    dbt = torch.empty(N, dtype=td, device=DEV)
    dx, dg32, db32, dgt, dbt = R.layernorm_bwd(
        xg, gg, dyg, mean_ref.to(DEV), rstd_ref.to(DEV), dx=empty_like_dev((M, N), td, misalign),
        dgamma=dgt, dbeta=dbt, flags=flags)
    torch.cuda.synchronize()
    return dict(M=M, N=N, td=td, x=x, y=(y, y_ref), mean=(mean, mean_ref), rstd=(rstd, rstd_ref),
                dx=(dx, dx_ref), dg=(dg32, dg_ref), db=(db32, db_ref), dgt=dgt, dbt=dbt)


def check(c):
    td, M = c["td"], c["M"]
    if M > 0:
        rstd, r_ref = c["rstd"]
        er = ((rstd.cpu().double() - r_ref.double()).abs() / r_ref.double().abs()).max().item()
        assert er <= 1e-5, f"rstd: error {er:.3g}"
        mean, m_ref = c["mean"]
        scale = c["x"].double().abs().amax(dim=1)
        em = ((mean.cpu().double() - m_ref.double()).abs() / scale).max().item()
        assert em <= 1e-6, f"mean: error {em:.3g}"
        assert_close("y", c["y"][0], c["y"][1], td)
        assert_close("dx", c["dx"][0], c["dx"][1], td)
    for name, key, half in (("dgamma", "dg", "dgt"), ("dbeta", "db", "dbt")):
        got, ref = c[key]
        e = rel(got, ref)
        assert e <= tol_dgamma(M), f"{name}: error {e:.3g} > {tol_dgamma(M):.3g}"
        assert torch.equal(c[half].cpu(), got.cpu().to(td)), f"{name}: dtype copy is not the RNE of fp32"


@pytest.mark.parametrize("name,M,N,dt,eps", CASES, ids=[c[0] for c in CASES])
def test_layernorm_parity(name, M, N, dt, eps):
    print("case layernorm", name, flush=True)
    check(run_case(M, N, dt, eps))


def test_layernorm_without_beta():
    print("case layernorm no beta", flush=True)
    check(run_case(300, 2048, "bf16", 1e-5, with_beta=False))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_layernorm_misaligned_pointers(dt):
    print("case layernorm misaligned", dt, flush=True)
    check(run_case(77, 1024, dt, 1e-5, misalign=True))


def test_layernorm_deterministic_repeats_bit_for_bit():
    print("case layernorm deterministic", flush=True)
    M, N = 2048, 4096
    x, g, b, dy = _inputs(M, N, "bf16")
    mean, rstd, _ = oracle.layernorm_fwd(x, g, b, 1e-6, want_y=False)
    args = [t.to(DEV) for t in (x, g, dy, mean, rstd)]
    first = R.layernorm_bwd(*args, flags=R.DGAMMA_DETERMINISTIC)
    for _ in range(3):
        again = R.layernorm_bwd(*args, flags=R.DGAMMA_DETERMINISTIC)
        torch.cuda.synchronize()
        for a, b_ in zip(first[:3], again[:3]):
            assert torch.equal(a, b_)


def test_layernorm_atomic_mode_within_tolerance():
    print("case layernorm atomic", flush=True)
    check(run_case(1024, 4096, "bf16", 1e-6, flags=R.DGAMMA_ATOMIC))


@pytest.mark.parametrize("flags", [R.DGAMMA_DETERMINISTIC, R.DGAMMA_ATOMIC, R.DGAMMA_ONE_BLOCK])
def test_layernorm_next_row_kernel_every_dgamma_mode(flags):
    print("case layernorm next-row kernel, mode", flags, flush=True)
    check(run_case(130, 14336, "bf16", 1e-6, flags=flags))


# (1100, 24576): several rows a block through the one-read kernel
@pytest.mark.parametrize("M,N,dt", [(5, 20000, "bf16"), (3, 32768, "f32"), (260, 16400, "f16"), (4, 30003, "bf16"),
                                    (1100, 24576, "bf16")])
def test_layernorm_long_rows(M, N, dt):
    print("case layernorm long rows", M, N, dt, flush=True)
    check(run_case(M, N, dt, 1e-5))


@pytest.mark.parametrize("M,N,dt", [(64, 2048, "bf16"), (1, 4096, "f32"), (40, 256, "f16")])
def test_layernorm_one_block_mode(M, N, dt):
    print("case layernorm one-block mode", M, N, dt, flush=True)
    check(run_case(M, N, dt, 1e-5, flags=R.DGAMMA_ONE_BLOCK))


@pytest.mark.parametrize("N,dt", [(20000, "bf16"), (24576, "f16"), (20000, "f32")])
def test_layernorm_one_long_row_unaligned_gradient_outputs(N, dt):
    """One long row: one block writes dgamma and dbeta itself, four columns a
    store where the outputs allow; outputs that are only element-aligned
    take element stores and must hold the same bits."""
    print("case layernorm one long row, unaligned outputs", N, dt, flush=True)
    c = run_case(1, N, dt, 1e-5)
    check(c)
    td = T[dt]
    x, g, b, dy = _inputs(1, N, dt)
    mean, rstd = c["mean"][1].to(DEV), c["rstd"][1].to(DEV)
    bufs = [torch.empty(N + 1, dtype=t, device=DEV) for t in (torch.float32, torch.float32, td, td)]
    _, dg32, db32, dgt, dbt = R.layernorm_bwd(x.to(DEV), g.to(DEV), dy.to(DEV), mean, rstd,
                                              dgamma_f32=bufs[0][1:], dbeta_f32=bufs[1][1:],
                                              dgamma=bufs[2][1:], dbeta=bufs[3][1:])
    torch.cuda.synchronize()
    assert bufs[0][1:].data_ptr() % 16 != 0
    for got, ref in ((dg32, c["dg"][0]), (db32, c["db"][0]), (dgt, c["dgt"]), (dbt, c["dbt"])):
        assert torch.equal(got.cpu(), ref.cpu())


def test_layernorm_no_rows_gives_zero_gradients():
    N = 512
    g = torch.ones(N, dtype=torch.bfloat16, device=DEV)
    x = torch.empty(0, N, dtype=torch.bfloat16, device=DEV)
    empty = torch.empty(0, dtype=torch.float32, device=DEV)
    dg32 = torch.full((N,), 7.0, device=DEV)
    db32 = torch.full((N,), 7.0, device=DEV)
    dgt = torch.full((N,), 7.0, dtype=torch.bfloat16, device=DEV)
    dbt = torch.full((N,), 7.0, dtype=torch.bfloat16, device=DEV)
    R.layernorm_bwd(x, g, x, empty, empty, dgamma_f32=dg32, dbeta_f32=db32, dgamma=dgt, dbeta=dbt)
    torch.cuda.synchronize()
    for t in (dg32, db32, dgt, dbt):
        assert not t.any()


def test_layer_norm_autograd_against_oracle_and_fp64_torch():
    print("case layer_norm autograd", flush=True)
    shape, N, eps = (4, 6, 768), 768, 1e-5
    x, g, b, _ = _inputs(24, N, "bf16")
    gen = np.random.Generator(np.random.PCG64(3))
    up = workloads.normal(gen, (24, N), 0.0, 1e-2, torch.bfloat16).reshape(24, N)
    xg = x.reshape(shape).to(DEV).requires_grad_()
    wg = g.to(DEV).requires_grad_()
    bg = b.to(DEV).requires_grad_()
    y = R.layer_norm(xg, wg, bg, eps)
    y.backward(up.reshape(shape).to(DEV))
    torch.cuda.synchronize()
    mean, rstd, y_ref = oracle.layernorm_fwd(x, g, b, eps)
    dx_ref, dg_ref, db_ref = oracle.layernorm_bwd(x, g, up, mean, rstd)
    assert_close("y", y.detach().reshape(24, N), y_ref, torch.bfloat16)
    assert_close("dx", xg.grad.reshape(24, N), dx_ref, torch.bfloat16)
    assert_close("dweight", wg.grad, dg_ref, torch.bfloat16)
    assert_close("dbias", bg.grad, db_ref, torch.bfloat16)
    # fp32 end to end against torch's own layer_norm autograd in fp64
    x32 = x.float().reshape(shape)
    xa = x32.to(DEV).requires_grad_()
    wa = g.float().to(DEV).requires_grad_()
    ba = b.float().to(DEV).requires_grad_()
    R.layer_norm(xa, wa, ba, eps).backward(up.float().reshape(shape).to(DEV))
    x64 = x32.double().requires_grad_()
    w64 = g.double().requires_grad_()
    b64 = b.double().requires_grad_()
    torch.nn.functional.layer_norm(x64, (N,), w64, b64, eps).backward(up.double().reshape(shape))
    assert rel(xa.grad.cpu(), x64.grad) <= 1e-5
    assert rel(wa.grad.cpu(), w64.grad) <= tol_dgamma(24)
    assert rel(ba.grad.cpu(), b64.grad) <= tol_dgamma(24)


@pytest.mark.parametrize("k", [40, -40])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_layernorm_extreme_magnitudes(k, dt):
    """x (mean 0.5) scaled by 2^k, exact in binary, with eps = 0: the mean and
    the centred values sit 2^k from their usual size and rstd 2^-k; every
    output must keep its accuracy against the oracle on the scaled input."""
    print("case layernorm magnitude 2^%d" % k, dt, flush=True)
    check(run_case(48, 2048, dt, 0.0, seed=53, scale_exp=k))
