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
