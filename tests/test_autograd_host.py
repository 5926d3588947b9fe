"""Host-side guards of the autograd wrappers (no GPU call is reached)."""
import pytest
import torch

import rmsnorm_bwd_amd as R


def test_rmsnorm_rejects_wrong_weight_length():
    with pytest.raises(ValueError):
        R.rmsnorm(torch.zeros(2, 8), torch.ones(7))


def test_fused_add_rejects_mismatched_shapes():
    with pytest.raises(ValueError):
        R.fused_add_rmsnorm(torch.zeros(2, 8), torch.zeros(3, 8), torch.ones(8))
    with pytest.raises(ValueError):
        R.fused_add_rmsnorm(torch.zeros(2, 8), torch.zeros(2, 8), torch.ones(9))


# The binding's row-view rule, on host tensors (no library call): (M, ld) of
# a tensor whose rows are its last dimension.

def test_row_view_of_contiguous_and_sliced_tensors():
    t = torch.zeros(6, 5, 8)
    assert R._view(t, 8, "f", "x") == (30, 8)
    assert R._view(torch.zeros(1, 8), 8, "f", "x") == (1, 8)
    assert R._view(torch.zeros(0, 8), 8, "f", "x") == (0, 8)
    wide = torch.zeros(7, 20)
    assert R._view(wide[:, 4:12], 8, "f", "x") == (7, 20)      # column block of wider rows
    assert R._view(wide[2:5, :8], 8, "f", "x") == (3, 20)      # row slice, still strided
    three = torch.zeros(3, 4, 20)[:, :, :8]                    # leading dims collapse: ld 20
    assert R._view(three, 8, "f", "x") == (12, 20)
    every_other = torch.zeros(3, 4, 20)[:, ::2, :8]            # strides 80, 40 collapse: ld 40
    assert R._view(every_other, 8, "f", "x") == (6, 40)
    # one column per row: any row stride works as N = 1
    assert R._view(torch.zeros(5, 3)[:, :1], 1, "f", "x") == (5, 3)


def test_row_view_refusals():
    with pytest.raises(ValueError):
        R._view(torch.zeros(4, 8), 7, "f", "x")                # wrong row length
    with pytest.raises(ValueError):
        R._view(torch.zeros(8, 4).t(), 8, "f", "x")            # rows not of unit stride
    with pytest.raises(ValueError):
        R._view(torch.zeros(3, 4, 20)[:, :2, :8], 8, "f", "x")  # strides 80, 20: no one row stride
    with pytest.raises(ValueError):
        R._view(torch.zeros(()), 1, "f", "x")                   # no row dimension


def test_row_stride_of_outputs_must_match_x_shape():
    x = torch.zeros(4, 8)
    assert R._ld(None, x.shape, 8, "f", "dx") == 8
    assert R._ld(torch.zeros(4, 8), x.shape, 8, "f", "dx") == 8
    assert R._ld(torch.zeros(4, 16)[:, :8], x.shape, 8, "f", "dx") == 16
    with pytest.raises(ValueError):
        R._ld(torch.zeros(8, 4), x.shape, 8, "f", "dx")


def test_device_index_rule():
    assert R._didx(torch.device("cpu")) == -1
    assert R._didx(torch.device("cuda", 0)) == 0
    assert R._didx(torch.device("cuda", 3)) == 3
    assert torch.zeros(1).get_device() == R._didx(torch.zeros(1).device)


def test_workspace_cache_keeps_the_most_recent_streams():
    R._workspaces.clear()
    cpu = torch.device("cpu")
    first = R._cached_workspace(cpu, 1000, 1)
    assert first.numel() >= 1000
    assert R._cached_workspace(cpu, 500, 1) is first          # reused when large enough
    bigger = R._cached_workspace(cpu, 5000, 1)
    assert bigger is not first and bigger.numel() >= 5000     # grown when not
    for s in range(2, 2 + 2 * R._WS_STREAMS):
        R._cached_workspace(cpu, 256, s)
    assert len(R._workspaces) == R._WS_STREAMS
    assert (None, 1) not in R._workspaces                     # the oldest stream gave its up
    assert (None, 1 + 2 * R._WS_STREAMS) in R._workspaces
    R._workspaces.clear()
