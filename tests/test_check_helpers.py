"""CPU checks of the GPU tests' comparison helpers (no GPU needed)."""

import numpy as np
import pytest
import torch

from gpu_util import check_bf16, check_bf16_floor


def _bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def test_floor_bar_accepts_the_exact_result_rounded_to_bf16():
    # outputs of magnitude 4..8: bf16 spacing 2^-5, rounding alone up to 2^-6
    want = np.linspace(4.0, 7.99, 4001)
    got = _bf16(want)
    assert np.abs(got - want).max() > 1e-2          # the fixed bar would reject it
    with pytest.raises(AssertionError):
        check_bf16(got, want)
    check_bf16_floor(got, want)


def test_floor_bar_rejects_an_error_beyond_the_floor():
    want = np.linspace(-3.0, 3.0, 1001)
    got = _bf16(want)
    got[500] += 0.02                                  # one element 2e-2 off
    with pytest.raises(AssertionError):
        check_bf16_floor(got, want)
    # every element 2e-3 off where the floor is tiny (|O| <= 0.1): the mean bar
    want = np.linspace(-0.1, 0.1, 1001)
    got = _bf16(want) + 2e-3
    with pytest.raises(AssertionError):
        check_bf16_floor(got, want)


def test_floor_bar_rejects_non_finite_output():
    want = np.zeros(8)
    got = want.copy()
    got[3] = np.nan
    with pytest.raises(AssertionError):
        check_bf16_floor(got, want)
