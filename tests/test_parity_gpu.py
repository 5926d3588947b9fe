"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the
seeded workloads (full sizes) and on edge cases: ragged and odd N, one row,
no rows, misaligned pointers, fp16, both dgamma modes, dresidual_out absent
and present, the fused forward writing residual_out in place.

Math: FlyDSL issue #769 ("[Feature] Add rmsnorm backward (+ forward saves
rstd) ..."), Implementation plan: Math; FlyDSL PR #800 ("[rmsnorm] Add
fused-add / residual backward (PR 2/3, #769)"), fused-add commit.
"""
import pytest
import torch

import oracle
import rmsnorm_bwd_amd as R
import workloads
from parity_util import (DEV, assert_close, assert_sum_bound, check_case, fused_case, place,
                         plain_case, rel, term_abs_sum, tol_dgamma)

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def _say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------------
# The named workloads at their full sizes
# --------------------------------------------------------------------------

PLAIN_FULL = ["plain_8x256_f32", "plain_512x3000_f32", "plain_512x2048_bf16",
              "plain_4096x4096_bf16", "plain_1x4096_bf16"]


@pytest.mark.parametrize("name", PLAIN_FULL)
def test_plain_workload_full(name):
    _say("case", name)
    check_case(plain_case(W[name]))


def test_fused_workload_1024x8192_full():
    _say("case fused_1024x8192_bf16")
    check_case(fused_case(W["fused_1024x8192_bf16"]))


@pytest.mark.slow
def test_fused_workload_32768x8192():
    """Full-size fused backward at 32768 x 8192 bf16, every element compared.
    The GPU runs the forward and the backward once on the whole tensor; the
    oracle then streams the rows in chunks of 1024 (forward for `out`,
    backward for dx), each chunk's fp64 results freed before the next, and
    every chunk of dx and `out` is held to the tolerances. residual_out and
    rstd are compared in full; dgamma in full, normwise and column by column
    to the fp32 summation bound, whose per-column terms are summed here
    chunk by chunk."""
    w = W["fused_32768x8192_bf16"]
    _say("case", w.name, "generating inputs")
    d = workloads.make_inputs(w)
    T, M, N = w.torch_dtype, w.M, w.N
    added, r_ref, _ = oracle.fused_add_rmsnorm_fwd(d["x"], d["residual"], d["gamma"], w.eps,
                                                    want_out=False)
    _say("oracle forward done")
    xg, resg, gg = place(d["x"]), place(d["residual"]), place(d["gamma"])
    out, res_out, rstd = R.fused_add_rmsnorm_fwd_rstd(xg, resg, gg, w.eps)
    del xg, resg
    ag, dyg, dresg = place(added), place(d["dy"]), place(d["dresidual_out"])
    dgt = torch.empty(N, dtype=T, device=DEV)
    dx, dg32, dgt = R.fused_add_rmsnorm_bwd(ag, gg, dyg, dresg, r_ref.to(DEV), dgamma=dgt)
    torch.cuda.synchronize()
    _say("gpu done")
    del ag, dyg, dresg
    assert torch.equal(res_out.cpu(), added)
    del res_out
    er = ((rstd.cpu().double() - r_ref.double()).abs() / r_ref.double()).max().item()
    assert er <= 1e-5
    _, dg_ref = oracle.fused_add_rmsnorm_bwd(added, d["gamma"], d["dy"], d["dresidual_out"],
                                             r_ref, want_dx=False)
    assert rel(dg32, dg_ref) <= tol_dgamma(M)
    assert torch.equal(dgt.cpu(), dg32.cpu().to(T))
    dx_h, out_h = dx.cpu(), out.cpu()
    del dx, out
    abs_sum = torch.zeros(N, dtype=torch.float64)
    CH = 1024
    for r0 in range(0, M, CH):
        rows = slice(r0, min(M, r0 + CH))
        a_s, r_s, o_s = oracle.fused_add_rmsnorm_fwd(d["x"][rows], d["residual"][rows], d["gamma"],
                                                     w.eps)
        assert torch.equal(a_s, added[rows]) and torch.equal(r_s, r_ref[rows])
        assert_close(f"out rows {r0}+", out_h[rows], o_s, T)
        del o_s
        dx_s, _ = oracle.fused_add_rmsnorm_bwd(a_s, d["gamma"], d["dy"][rows], d["dresidual_out"][rows],
                                               r_s, want_dgamma=False)
        assert_close(f"dx rows {r0}+", dx_h[rows], dx_s, T)
        del dx_s
        abs_sum += term_abs_sum(a_s, d["dy"][rows], r_s)
    _say("all", M, "rows compared")
    assert_sum_bound("dgamma", dg32, dg_ref, abs_sum, M)


# --------------------------------------------------------------------------
# Edge cases and the row-plan paths
# --------------------------------------------------------------------------

EDGE = [
    # (M, N, dtype): odd and ragged N take the element path; others cover
    # every vector row plan (16..512 threads per row) and several rows per wave
    (1, 1, "f32"), (3, 7, "bf16"), (37, 255, "f16"), (5, 3001, "bf16"), (9, 4097, "f32"),
    (300, 64, "bf16"), (1000, 128, "f32"), (129, 1024, "f16"), (64, 2048, "f16"),
    (33, 8192, "bf16"), (17, 16384, "bf16"), (6, 16384, "f32"), (2, 12288, "f32"),
    (1, 16383, "bf16"), (700, 768, "bf16"), (258, 5120, "f16"),
    # both sides of the one-block rule (N <= 1024 and M * N <= 8192, or
    # M <= 2 and N <= 8192)
    (32, 256, "bf16"), (33, 256, "bf16"), (8, 1024, "f32"), (9, 1024, "f32"),
    (2, 8192, "bf16"), (3, 4096, "bf16"), (2, 16384, "f32"), (2, 3000, "f32"),
    # a few blocks fill their window ring (and pause in the prologue) while
    # the rest hold fewer windows: 517 or 515 windows over 256 blocks
    (517, 4096, "bf16"), (1029, 2048, "bf16"), (517, 8192, "bf16"),
    # the element path's plans with several row windows a block
    (70, 1500, "bf16"), (600, 6001, "f16"), (300, 12289, "bf16"),
]


@pytest.mark.parametrize("M,N,dt", EDGE)
def test_plain_edge_shapes(M, N, dt):
    _say("case plain", M, N, dt)
    check_case(plain_case(workloads.custom("plain", M, N, dt, 1e-5, seed=M + N)))


# Short rows at large M: each block holds thousands of row windows and folds
# every one of their rows into its dgamma registers; M is not a multiple of
# the rows a window holds, so the last window is ragged.
MANY_ROWS = [(262147, 64, "bf16"), (100003, 256, "f32"), (32771, 1024, "f16")]


@pytest.mark.parametrize("M,N,dt", MANY_ROWS)
def test_plain_short_rows_at_large_M(M, N, dt):
    _say("case plain many rows", M, N, dt)
    check_case(plain_case(workloads.custom("plain", M, N, dt, 1e-5, seed=M + N)))


def test_fused_short_rows_at_large_M():
    _say("case fused many rows 131075 128 bf16")
    check_case(fused_case(workloads.custom("fused", 131075, 128, "bf16", 1e-6, seed=7)))


# Rows longer than 16384 elements: the two-pass long-row kernels (16-byte
# chunks where N and the pointers allow, single elements otherwise), one row
# per block of 512 threads; 257 rows put two rows on one block of 256.
LONG = [(3, 16385, "bf16"), (5, 20000, "f32"), (130, 32768, "bf16"), (7, 32768, "f32"),
        (9, 30001, "f16"), (257, 24576, "bf16"), (1, 32768, "f16"), (2, 20480, "bf16"),
        # several rows a block: the next row loaded during the current one
        # (16-bit), gamma held in registers (fp32 plain)
        (1300, 24576, "bf16"), (1100, 20000, "f32")]


@pytest.mark.parametrize("M,N,dt", LONG)
def test_long_rows(M, N, dt):
    _say("case long rows", M, N, dt)
    check_case(plain_case(workloads.custom("plain", M, N, dt, 1e-5, seed=M + N)))
    check_case(fused_case(workloads.custom("fused", M, N, dt, 1e-6, seed=M + 3 * N)))


@pytest.mark.parametrize("flags", [R.DGAMMA_DETERMINISTIC, R.DGAMMA_ATOMIC, R.DGAMMA_ONE_BLOCK])
def test_long_rows_every_dgamma_mode(flags):
    _say("case long rows, mode", flags)
    check_case(plain_case(workloads.custom("plain", 40, 24576, "bf16", 1e-5, seed=11), flags=flags))
    check_case(fused_case(workloads.custom("fused", 33, 20000, "f32", 1e-6, seed=12), flags=flags))


def test_long_rows_misaligned_and_in_place():
    _say("case long rows misaligned, in-place residual_out")
    check_case(plain_case(workloads.custom("plain", 4, 20000, "bf16", 1e-5), misalign=True))
    check_case(fused_case(workloads.custom("fused", 3, 18000, "f16", 1e-5), misalign=True))
    w = workloads.custom("fused", 6, 25000, "bf16", 1e-6)
    d = workloads.make_inputs(w)
    a_ref, r_ref, o_ref = oracle.fused_add_rmsnorm_fwd(d["x"], d["residual"], d["gamma"], w.eps)
    res = d["residual"].to(DEV)
    out, res_out, rstd = R.fused_add_rmsnorm_fwd_rstd(d["x"].to(DEV), res, d["gamma"].to(DEV), w.eps,
                                                      residual_out=res)
    torch.cuda.synchronize()
    assert torch.equal(res.cpu(), a_ref)
    assert_close("out", out, o_ref, torch.bfloat16)


def test_long_rows_deterministic_repeats_bit_for_bit():
    _say("case long rows deterministic repeat")
    c = plain_case(workloads.custom("plain", 300, 32768, "bf16", 1e-6, seed=5), flags=R.DGAMMA_DETERMINISTIC)
    check_case(c)
    xg, gg, dyg, rg = c["inputs"]
    for _ in range(2):
        dx, dg32, _ = R.rmsnorm_bwd(xg, gg, dyg, rg, flags=R.DGAMMA_DETERMINISTIC)
        torch.cuda.synchronize()
        assert torch.equal(dx, c["dx"][0]) and torch.equal(dg32, c["dg32"][0])


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("k", [40, -40])
@pytest.mark.parametrize("M,N", [(64, 4096), (7, 3001)])
def test_extreme_magnitudes(M, N, dt, k):
    """x scaled by 2^k, which is exact in binary, with eps = 0. The kernel
    forms dx as r*wdy - (r*r*c1)*x, whose per-row factor r*r is then 2^(-2k)
    times its usual size; dx and y must keep their accuracy against the oracle
    on the scaled input."""
    _say("case magnitude 2^%d" % k, M, N, dt)
    w = workloads.custom("plain", M, N, dt, 0.0, seed=k & 0xFF)
    d = workloads.make_inputs(w)
    T = w.torch_dtype
    x = (d["x"].double() * 2.0 ** k).to(T)
    assert torch.equal(x.double() / 2.0 ** k, d["x"].double())  # the scaling was exact
    r_ref, y_ref = oracle.rmsnorm_fwd(x, d["gamma"], 0.0)
    xg, gg, dyg = place(x), place(d["gamma"]), place(d["dy"])
    y, rstd = R.rmsnorm_fwd_rstd(xg, gg, 0.0)
    dx, dg32, _ = R.rmsnorm_bwd(xg, gg, dyg, r_ref.to(DEV))
    torch.cuda.synchronize()
    er = ((rstd.cpu().double() - r_ref.double()).abs() / r_ref.double()).max().item()
    assert er <= 1e-5
    assert_close("y", y, y_ref, T)
    dx_ref, dg_ref = oracle.rmsnorm_bwd(x, d["gamma"], d["dy"], r_ref)
    assert_close("dx", dx, dx_ref, T)
    assert rel(dg32, dg_ref) <= tol_dgamma(M)


@pytest.mark.parametrize("k", [40, -40])
def test_fused_extreme_magnitudes(k):
    """x and residual scaled by 2^k (exact in binary), eps = 0: their sum,
    rounded once, is the unscaled sum times 2^k, and the backward (with a
    dresidual_out) must keep its accuracy against the oracle."""
    _say("case fused magnitude 2^%d" % k)
    M, N = 64, 4096
    w = workloads.custom("fused", M, N, "bf16", 0.0, seed=k & 0xFF)
    d = workloads.make_inputs(w)
    T = w.torch_dtype
    xs, rs = ((d[n].double() * 2.0 ** k).to(T) for n in ("x", "residual"))
    a_ref, r_ref, o_ref = oracle.fused_add_rmsnorm_fwd(xs, rs, d["gamma"], 0.0)
    out, res_out, rstd = R.fused_add_rmsnorm_fwd_rstd(place(xs), place(rs), place(d["gamma"]), 0.0)
    dx, dg32, _ = R.fused_add_rmsnorm_bwd(place(a_ref), place(d["gamma"]), place(d["dy"]),
                                          place(d["dresidual_out"]), r_ref.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(res_out.cpu(), a_ref)
    er = ((rstd.cpu().double() - r_ref.double()).abs() / r_ref.double()).max().item()
    assert er <= 1e-5
    assert_close("out", out, o_ref, T)
    dx_ref, dg_ref = oracle.fused_add_rmsnorm_bwd(a_ref, d["gamma"], d["dy"], d["dresidual_out"], r_ref)
    assert_close("dx", dx, dx_ref, T)
    assert rel(dg32, dg_ref) <= tol_dgamma(M)


# A fused backward with a dresidual_out runs a smaller grid from 4096 rows
# on; these shapes put it at long and mid-length rows, ragged in M, compared
# in full.
FUSED_CAPPED = [(4099, 4096, "bf16"), (5000, 2048, "bf16"), (4097, 3000, "f32")]


@pytest.mark.parametrize("M,N,dt", FUSED_CAPPED)
def test_fused_capped_grid_shapes(M, N, dt):
    _say("case fused capped grid", M, N, dt)
    check_case(fused_case(workloads.custom("fused", M, N, dt, 1e-6, seed=M + 5 * N)))


@pytest.mark.parametrize("M,N,dt", EDGE[::2])
def test_fused_edge_shapes(M, N, dt):
    _say("case fused", M, N, dt)
    check_case(fused_case(workloads.custom("fused", M, N, dt, 1e-6, seed=M * 3 + N)))


# The fused backward runs rows of 1025 to 1536 16-byte chunks (8200-12288
# 16-bit or 4100-6144 fp32 elements) with three chunks a thread: both ends
# of that range, both element sizes, ragged M, a capped grid, and the first
# row length past it (four chunks a thread).
THREE_CHUNK = [(300, 10240, "bf16"), (129, 12288, "f16"), (260, 8200, "bf16"), (70, 6144, "f32"),
               (65, 4100, "f32"), (4099, 12288, "bf16"), (40, 12296, "bf16")]


@pytest.mark.parametrize("M,N,dt", THREE_CHUNK)
def test_fused_three_chunk_rows(M, N, dt):
    _say("case fused three-chunk", M, N, dt)
    check_case(fused_case(workloads.custom("fused", M, N, dt, 1e-6, seed=M + 7 * N)))


# The plain and fused forwards run 16-bit rows of 8200-12288 elements on
# three chunks a thread up to 2^26 elements a call and on the plan's four
# beyond: 12288-element rows at 5461 rows (2^26 - 4096 elements) and 5462
# (just past). The first m0 rows are held to the oracle; the rest repeat them
# down the tensor, and a row's outputs depend on that row and gamma alone, so
# every repetition must equal its first occurrence bit for bit.
@pytest.mark.parametrize("op", ["plain", "fused"])
@pytest.mark.parametrize("M", [5461, 5462])
def test_forward_three_chunk_size_limit(op, M):
    N, m0 = 12288, 43
    _say("case forward three-chunk limit", op, M, N)
    w = workloads.custom(op, m0, N, "bf16", 1e-6, seed=M + 13)
    d = workloads.make_inputs(w)
    reps = -(-M // m0)

    def tile(t):
        return t.to(DEV).repeat(reps, 1)[:M].contiguous()

    g = d["gamma"].to(DEV)
    if op == "plain":
        r_ref, y_ref = oracle.rmsnorm_fwd(d["x"], d["gamma"], w.eps)
        y, rstd = R.rmsnorm_fwd_rstd(tile(d["x"]), g, w.eps)
        rows = [("y", y)]
    else:
        added, r_ref, y_ref = oracle.fused_add_rmsnorm_fwd(d["x"], d["residual"], d["gamma"], w.eps)
        y, res_out, rstd = R.fused_add_rmsnorm_fwd_rstd(tile(d["x"]), tile(d["residual"]), g, w.eps)
        rows = [("out", y), ("residual_out", res_out)]
        assert torch.equal(res_out[:m0].cpu(), added), "residual_out differs from the rounded sum"
    torch.cuda.synchronize()
    assert_close(rows[0][0], y[:m0], y_ref, torch.bfloat16)
    er = ((rstd[:m0].cpu().double() - r_ref.double()).abs() / r_ref.double().abs()).max().item()
    assert er <= 1e-5, f"rstd: error {er:.3g}"
    full = (M // m0) * m0
    for name, t in rows + [("rstd", rstd)]:
        v = t[:full].view(M // m0, m0, *t.shape[1:])
        assert torch.equal(v, v[:1].expand_as(v)), f"{name}: a repetition differs from the first rows"
        assert torch.equal(t[full:], t[:M - full]), f"{name}: the ragged tail differs from the first rows"


# The plain forward runs 16-bit rows of 4104-6144 elements on 256-thread
# groups (three chunks a thread, two rows a block) from 4096 rows: ragged M
# (an odd last window), both 16-bit types, both ends of the range, and 4095
# rows (the plan's two chunks on 512 threads). The backward of each runs too.
HALF_ROWS = [(4096, 5120, "bf16"), (4097, 6144, "f16"), (4101, 4104, "bf16"), (4095, 6144, "bf16")]


@pytest.mark.parametrize("M,N,dt", HALF_ROWS)
def test_plain_forward_half_row_groups(M, N, dt):
    _say("case plain forward half rows", M, N, dt)
    check_case(plain_case(workloads.custom("plain", M, N, dt, 1e-6, seed=M + 5 * N)))


# Every forward runs 16-bit rows of 2056-3072 elements on 128-thread groups
# (three chunks a thread, four rows a block) from 3072 rows: M not a multiple
# of four (a ragged last window), both 16-bit types, both ends of the range,
# and 3071 rows (the plan's one chunk on 512 threads). The backward of each
# runs too.
QUARTER_ROWS = [("plain", 3072, 2560, "bf16"), ("plain", 4097, 2056, "f16"), ("fused", 3074, 3072, "bf16"),
                ("fused", 4099, 2304, "f16"), ("plain", 3071, 3072, "bf16"), ("fused", 3071, 2056, "bf16")]


@pytest.mark.parametrize("op,M,N,dt", QUARTER_ROWS)
def test_forward_quarter_row_groups(op, M, N, dt):
    _say("case forward quarter rows", op, M, N, dt)
    w = workloads.custom(op, M, N, dt, 1e-6, seed=M + 3 * N)
    check_case(plain_case(w) if op == "plain" else fused_case(w))


# The plain and LayerNorm forwards, and the fused one from 2048 rows, run
# 16-bit rows of 1032-1536 elements on one wavefront a row (three chunks a
# thread, four rows a block): one row, ragged M, both 16-bit types, both ends
# of the range, and the fused forward one row short of 2048 (the plan's one
# chunk on 256 threads). The backward of each runs too.
WAVE_ROWS = [("plain", 1, 1536, "bf16"), ("plain", 4099, 1032, "f16"), ("plain", 301, 1280, "bf16"),
             ("fused", 2048, 1536, "bf16"), ("fused", 2051, 1032, "f16"), ("fused", 2047, 1536, "bf16")]


@pytest.mark.parametrize("op,M,N,dt", WAVE_ROWS)
def test_forward_wave_row_groups(op, M, N, dt):
    _say("case forward wave rows", op, M, N, dt)
    w = workloads.custom(op, M, N, dt, 1e-6, seed=M + 9 * N)
    check_case(plain_case(w) if op == "plain" else fused_case(w))


# The forwards run 16-bit rows of 520-768 elements on 32-thread groups (three
# chunks a thread, eight rows a block): the plain one from 256 rows, the
# fused one from 4096 rows; M not a multiple of eight, both 16-bit types,
# both ends of the range, and one row short of each limit (the plan's one
# chunk on 128 threads). The backward of each runs too.
NARROW_ROWS = [("plain", 256, 768, "bf16"), ("plain", 4099, 520, "f16"), ("plain", 255, 768, "bf16"),
               ("fused", 4096, 768, "bf16"), ("fused", 4101, 640, "f16"), ("fused", 4095, 768, "bf16")]


@pytest.mark.parametrize("op,M,N,dt", NARROW_ROWS)
def test_forward_narrow_row_groups(op, M, N, dt):
    _say("case forward narrow rows", op, M, N, dt)
    w = workloads.custom(op, M, N, dt, 1e-6, seed=M + 17 * N)
    check_case(plain_case(w) if op == "plain" else fused_case(w))


# Every forward runs 16-bit rows of 264-384 elements with three chunks a
# thread instead of four on 16-thread groups (sixteen rows a block): one row,
# M not a multiple of sixteen, both 16-bit types, both ends of the range, and
# 392 elements (one chunk past: four chunks a thread). The backward of each
# runs too.
SHORT_ROWS = [("plain", 1, 384, "bf16"), ("plain", 4099, 264, "f16"), ("plain", 300, 392, "bf16"),
              ("fused", 300, 320, "bf16"), ("fused", 17, 384, "f16")]


@pytest.mark.parametrize("op,M,N,dt", SHORT_ROWS)
def test_forward_short_rows_three_chunks(op, M, N, dt):
    _say("case forward short rows", op, M, N, dt)
    w = workloads.custom(op, M, N, dt, 1e-6, seed=M + 19 * N)
    check_case(plain_case(w) if op == "plain" else fused_case(w))


# The fused backward runs 16-bit rows of 12296-16384 elements on the
# long-row kernel, which loads a block's next row during the current one:
# ragged M on the capped grid and below it, both 16-bit types, both ends of
# the range, fewer rows than blocks.
FUSED_NEXT_ROW = [(4099, 12296, "bf16"), (4096, 16384, "f16"), (4100, 14336, "bf16"), (2048, 16384, "bf16"),
                  (300, 12296, "f16"), (33, 16384, "bf16")]


@pytest.mark.parametrize("M,N,dt", FUSED_NEXT_ROW)
def test_fused_next_row_kernel_rows(M, N, dt):
    _say("case fused next-row", M, N, dt)
    check_case(fused_case(workloads.custom("fused", M, N, dt, 1e-6, seed=M + 11 * N)))


def test_fused_next_row_kernel_every_dgamma_mode():
    """The atomic and one-block sums on the same inputs: dx bit-equal to the
    default call's (it does not depend on how dgamma is summed), dgamma
    within the tolerance of the oracle."""
    _say("case fused next-row, modes")
    c = fused_case(workloads.custom("fused", 4097, 12296, "bf16", 1e-6, seed=21))
    check_case(c)
    ag, gg, dyg, dresg, rg = c["inputs"]
    for flags in (R.DGAMMA_ATOMIC, R.DGAMMA_ONE_BLOCK):
        dx, dg32, _ = R.fused_add_rmsnorm_bwd(ag, gg, dyg, dresg, rg, flags=flags)
        torch.cuda.synchronize()
        assert torch.equal(dx, c["dx"][0]), f"flags {flags}: dx differs from the default call"
        assert rel(dg32, c["dg32"][1]) <= tol_dgamma(c["M"]), f"flags {flags}: dgamma"


@pytest.mark.parametrize("M,N,dt", [(64, 4096, "bf16"), (7, 3000, "f32"), (40, 250, "f16")])
def test_misaligned_pointers_take_the_element_path(M, N, dt):
    _say("case misaligned", M, N, dt)
    check_case(plain_case(workloads.custom("plain", M, N, dt, 1e-5), misalign=True))
    check_case(fused_case(workloads.custom("fused", M, N, dt, 1e-5), misalign=True))


@pytest.mark.parametrize("M,N,dt", [(1, 4096, "bf16"), (8, 1024, "bf16"), (32, 256, "bf16"),
                                     (1, 3000, "f32"), (8, 256, "f16"),
                                     # one long row: the long-row kernels' one-block stores
                                     (1, 20000, "bf16"), (1, 32768, "f32"), (1, 24576, "f16")])
def test_one_block_call_with_unaligned_gradient_outputs(M, N, dt):
    """A call whose rows fit one block writes dgamma itself, four columns a
    store when its outputs allow; outputs that are only element-aligned take
    element stores and must hold the same bits."""
    _say("case one block, unaligned dgamma outputs", M, N, dt)
    w = workloads.custom("plain", M, N, dt, 1e-5, seed=N)
    d = workloads.make_inputs(w)
    T = w.torch_dtype
    x, g, dy = place(d["x"]), place(d["gamma"]), place(d["dy"])
    r_ref, _ = oracle.rmsnorm_fwd(d["x"], d["gamma"], w.eps)
    rstd = r_ref.to(DEV)
    _, dg32_a, dgt_a = R.rmsnorm_bwd(x, g, dy, rstd, dgamma=torch.empty(N, dtype=T, device=DEV))
    f32buf = torch.empty(N + 1, dtype=torch.float32, device=DEV)
    tbuf = torch.empty(N + 1, dtype=T, device=DEV)
    _, dg32_u, dgt_u = R.rmsnorm_bwd(x, g, dy, rstd, dgamma_f32=f32buf[1:], dgamma=tbuf[1:])
    torch.cuda.synchronize()
    assert f32buf[1:].data_ptr() % 16 != 0
    assert torch.equal(dg32_u.cpu(), dg32_a.cpu()) and torch.equal(dgt_u.cpu(), dgt_a.cpu())
    assert torch.equal(dgt_u.cpu(), dg32_u.cpu().to(T))
    _, dg_ref = oracle.rmsnorm_bwd(d["x"], d["gamma"], d["dy"], r_ref)
    assert rel(dg32_u, dg_ref) <= tol_dgamma(M)


@pytest.mark.parametrize("with_dres", [False, True])
@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
def test_fused_with_and_without_dresidual(with_dres, dt):
    _say("case fused dres", with_dres, dt)
    check_case(fused_case(workloads.custom("fused", 96, 1536, dt, 1e-6), with_dres=with_dres))


@pytest.mark.parametrize("eps", [1e-5, 1e-6, 1e-2, 0.0])
def test_eps_is_honoured(eps):
    _say("case eps", eps)
    check_case(plain_case(workloads.custom("plain", 64, 512, "f32", eps)))


def test_no_rows():
    _say("case M=0")
    for op in ("plain", "fused"):
        N = 64
        g = torch.randn(N, device=DEV, dtype=torch.bfloat16)
        x = torch.empty(0, N, device=DEV, dtype=torch.bfloat16)
        rstd = torch.empty(0, device=DEV)
        dg32 = torch.full((N,), 7.0, device=DEV)
        dgt = torch.full((N,), 7.0, device=DEV, dtype=torch.bfloat16)
        if op == "plain":
            R.rmsnorm_bwd(x, g, x, rstd, dgamma_f32=dg32, dgamma=dgt)
            y, r = R.rmsnorm_fwd_rstd(x, g, 1e-5)
        else:
            R.fused_add_rmsnorm_bwd(x, g, x, None, rstd, dgamma_f32=dg32, dgamma=dgt)
            R.fused_add_rmsnorm_fwd_rstd(x, x, g, 1e-5)
        torch.cuda.synchronize()
        assert torch.count_nonzero(dg32) == 0 and torch.count_nonzero(dgt.float()) == 0


def test_batched_input_flattens_leading_dims():
    _say("case 3-D input")
    w = workloads.custom("plain", 24, 640, "bf16", 1e-5)
    d = workloads.make_inputs(w)
    r_ref, _ = oracle.rmsnorm_fwd(d["x"], d["gamma"], w.eps)
    x3 = d["x"].view(4, 6, 640).to(DEV)
    dy3 = d["dy"].view(4, 6, 640).to(DEV)
    dx, dg32, _ = R.rmsnorm_bwd(x3, d["gamma"].to(DEV), dy3, r_ref.to(DEV))
    torch.cuda.synchronize()
    dx_ref, dg_ref = oracle.rmsnorm_bwd(d["x"], d["gamma"], d["dy"], r_ref)
    assert dx.shape == (4, 6, 640)
    assert_close("dx", dx.view(24, 640), dx_ref, torch.bfloat16)
    assert rel(dg32, dg_ref) <= tol_dgamma(24)


# --------------------------------------------------------------------------
# dgamma modes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["plain_4096x4096_bf16", "plain_512x3000_f32"])
def test_deterministic_mode_repeats_bit_for_bit(name):
    _say("case deterministic", name)
    c = plain_case(W[name], flags=R.DGAMMA_DETERMINISTIC)
    check_case(c)
    xg, gg, dyg, rg = c["inputs"]
    for _ in range(3):
        dx, dg32, _ = R.rmsnorm_bwd(xg, gg, dyg, rg, flags=R.DGAMMA_DETERMINISTIC)
        torch.cuda.synchronize()
        assert torch.equal(dx, c["dx"][0]) and torch.equal(dg32, c["dg32"][0])


@pytest.mark.parametrize("name", ["plain_4096x4096_bf16", "plain_512x2048_bf16"])
def test_atomic_mode_within_tolerance(name):
    _say("case atomic", name)
    check_case(plain_case(W[name], flags=R.DGAMMA_ATOMIC))


@pytest.mark.parametrize("M,N,dt", [(1, 4096, "bf16"), (64, 2048, "bf16"), (300, 3000, "f32"),
                                     (33, 256, "f16"), (5, 1001, "bf16")])
def test_one_block_mode_at_any_size(M, N, dt):
    """The explicit one-block mode: one workgroup walks every row and writes
    the gradients itself, also where the default would use many blocks."""
    _say("case one-block mode", M, N, dt)
    check_case(plain_case(workloads.custom("plain", M, N, dt, 1e-5, seed=M * 7 + N), flags=R.DGAMMA_ONE_BLOCK))
    check_case(fused_case(workloads.custom("fused", M, N, dt, 1e-6, seed=M * 5 + N), flags=R.DGAMMA_ONE_BLOCK))


@pytest.mark.parametrize("M,N,dt", [(1, 4096, "bf16"), (8, 1024, "f32"), (32, 256, "bf16"), (3, 7, "f16")])
def test_deterministic_mode_where_the_default_runs_one_block(M, N, dt):
    """The explicit deterministic mode keeps its two-stage sum (block
    partials, then the fixed-order finalize) on problems the default runs
    in one block, and repeats bit for bit."""
    _say("case deterministic at one-block shapes", M, N, dt)
    c = plain_case(workloads.custom("plain", M, N, dt, 1e-5, seed=N + 3), flags=R.DGAMMA_DETERMINISTIC)
    check_case(c)
    xg, gg, dyg, rg = c["inputs"]
    dx, dg32, _ = R.rmsnorm_bwd(xg, gg, dyg, rg, flags=R.DGAMMA_DETERMINISTIC)
    torch.cuda.synchronize()
    assert torch.equal(dx, c["dx"][0]) and torch.equal(dg32, c["dg32"][0])


def test_atomic_mode_fused():
    _say("case atomic fused")
    check_case(fused_case(W["fused_1024x8192_bf16"], flags=R.DGAMMA_ATOMIC))


# --------------------------------------------------------------------------
# Aliasing, guards and errors
# --------------------------------------------------------------------------

def test_fused_forward_in_place_residual():
    _say("case in-place residual_out")
    w = workloads.custom("fused", 50, 1000, "bf16", 1e-6)
    d = workloads.make_inputs(w)
    a_ref, r_ref, o_ref = oracle.fused_add_rmsnorm_fwd(d["x"], d["residual"], d["gamma"], w.eps)
    res = d["residual"].to(DEV)
    out, res_out, rstd = R.fused_add_rmsnorm_fwd_rstd(d["x"].to(DEV), res, d["gamma"].to(DEV),
                                                      w.eps, residual_out=res)
    torch.cuda.synchronize()
    assert res_out.data_ptr() == res.data_ptr()
    assert torch.equal(res.cpu(), a_ref)
    assert_close("out", out, o_ref, torch.bfloat16)


def test_dtype_mismatch_is_refused():
    # the pages' guard: one dtype across operands, else bytes are reinterpreted
    x = torch.randn(4, 64, device=DEV, dtype=torch.bfloat16)
    g = torch.ones(64, device=DEV, dtype=torch.float16)
    with pytest.raises(TypeError):
        R.rmsnorm_fwd_rstd(x, g, 1e-5)
    with pytest.raises(TypeError):
        R.fused_add_rmsnorm_fwd_rstd(x, x.half(), g.bfloat16(), 1e-5)
    with pytest.raises(ValueError):
        R.rmsnorm_fwd_rstd(x, torch.ones(63, device=DEV, dtype=torch.bfloat16), 1e-5)
    with pytest.raises(ValueError):
        R.rmsnorm_fwd_rstd(x.t(), torch.ones(4, device=DEV, dtype=torch.bfloat16), 1e-5)


def test_device_check_flag_refuses_host_memory():
    N = 256
    x = torch.randn(4, N, device=DEV)
    g = torch.ones(N, device=DEV)
    rstd = torch.ones(4, device=DEV)
    host_dy = torch.randn(4, N)
    ws = torch.empty(R.rmsnorm_bwd_workspace_bytes(4, N, R.F32), dtype=torch.uint8, device=DEV)
    dx = torch.empty_like(x)
    dg = torch.empty(N, device=DEV)
    import ctypes
    st = R.lib().rmsnorm_bwd(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(g.data_ptr()),
                             ctypes.c_void_p(host_dy.data_ptr()), ctypes.c_void_p(rstd.data_ptr()),
                             ctypes.c_void_p(dx.data_ptr()), ctypes.c_void_p(dg.data_ptr()), None,
                             ctypes.c_void_p(ws.data_ptr()), ws.numel(), 4, N, R.F32,
                             R.CHECK_DEVICE, None)
    assert st == 7  # RMSN_ERR_DEVICE, nothing launched
    # with device memory everywhere, the checked call runs
    dx2, dg2, _ = R.rmsnorm_bwd(x, g, x, rstd, flags=R.CHECK_DEVICE)
    torch.cuda.synchronize()
    assert torch.isfinite(dx2).all() and torch.isfinite(dg2).all()


def test_binding_refuses_host_outputs_and_workspace():
    """The binding checks, before any launch, that the fp32 weight-gradient
    outputs and a caller's workspace are on x's device (a host pointer would
    otherwise reach the kernel)."""
    N, M = 256, 4
    x = torch.randn(M, N, device=DEV)
    g = torch.ones(N, device=DEV)
    rstd = torch.ones(M, device=DEV)
    with pytest.raises(ValueError):
        R.rmsnorm_bwd(x, g, x, rstd, dgamma_f32=torch.empty(N))
    with pytest.raises(ValueError):
        R.rmsnorm_bwd(x, g, x, rstd, workspace=torch.zeros(1 << 16, dtype=torch.uint8))
    with pytest.raises(ValueError):
        R.layernorm_bwd(x, g, x, rstd, rstd, dbeta_f32=torch.empty(N))
    # a float32 workspace is sized in bytes, not elements
    need = R.rmsnorm_bwd_workspace_bytes(64, 4096, torch.float32)
    xs = torch.randn(64, 4096, device=DEV)
    gs = torch.ones(4096, device=DEV)
    rs = torch.ones(64, device=DEV)
    ws = torch.zeros((need + 3) // 4, dtype=torch.float32, device=DEV)
    dx, dg, _ = R.rmsnorm_bwd(xs, gs, xs, rs, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(dx).all() and torch.isfinite(dg).all()


def test_concurrent_streams_each_get_their_own_workspace():
    """Backward calls queued on two streams at once (default priority), with
    no workspace passed: the binding keeps one workspace per stream, so the
    calls do not share partials; each result is held to the oracle."""
    _say("case two streams")
    cases = []
    for seed, M in ((101, 2048), (102, 1536)):
        w = workloads.custom("plain", M, 4096, "bf16", 1e-6, seed=seed)
        d = workloads.make_inputs(w)
        r, _ = oracle.rmsnorm_fwd(d["x"], d["gamma"], w.eps, want_y=False)
        cases.append((w, d, r))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    dev_in = [(d["x"].to(DEV), d["gamma"].to(DEV), d["dy"].to(DEV), r.to(DEV)) for _, d, r in cases]
    torch.cuda.synchronize()
    for _ in range(3):
        outs = []
        for s, (x, g, dy, r) in zip(streams, dev_in):
            with torch.cuda.stream(s):
                outs.append(R.rmsnorm_bwd(x, g, dy, r))
        torch.cuda.synchronize()
    for (w, d, r), (dx, dg32, _) in zip(cases, outs):
        dx_ref, dg_ref = oracle.rmsnorm_bwd(d["x"], d["gamma"], d["dy"], r)
        assert_close("dx", dx, dx_ref, w.torch_dtype)
        assert rel(dg32, dg_ref) <= tol_dgamma(w.M)
