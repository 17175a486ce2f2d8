"""The parity bar itself (CPU): what ``gpu_util.assert_close`` accepts and
rejects, on hand-made outputs around a known exact value."""
import numpy as np
import pytest
import torch

from gpu_util import TOL, assert_close, rounding_slack


def test_rounding_slack_is_half_the_gap_toward_ref():
    got = torch.tensor([1.0, 1.0, 16.0], dtype=torch.bfloat16)
    ref = np.array([1.001, 0.999, 15.9])
    s = rounding_slack(got, ref)
    # bf16 spacing above 1 is 2^-7, below 1 it is 2^-8; below 16 it is 2^-4
    assert np.allclose(s, [2.0 ** -8, 2.0 ** -9, 2.0 ** -5])


def test_correctly_rounded_large_outputs_pass_both_bars():
    """Outputs that are the exact values rounded to bf16 pass, however large the
    values (the rounding alone averages far above the 2e-3 mean bar here)."""
    g = torch.Generator().manual_seed(5)
    ref = (torch.rand(64, 64, generator=g, dtype=torch.float64) * 8 + 12).numpy()
    got = torch.from_numpy(ref).to(torch.bfloat16)
    assert np.abs(got.double().numpy() - ref).mean() > TOL[torch.bfloat16][1]
    assert_close("x", got, ref, torch.bfloat16)


def test_an_output_off_by_more_than_the_bar_fails():
    ref = np.full((8,), 0.5)
    got = torch.full((8,), 0.5, dtype=torch.bfloat16)
    got[3] = 0.5 + 2 ** -5      # 0.031 off, with a spacing of 2^-8 near 0.5
    with pytest.raises(AssertionError, match="error"):
        assert_close("x", got, ref, torch.bfloat16)


def test_a_uniform_small_bias_fails_the_mean_bar():
    """Every element 0.004 off (within the max bar, past the mean bar, and more
    than rounding can explain at magnitude 0.1)."""
    ref = np.full((256,), 0.1)
    got = torch.full((256,), 0.104, dtype=torch.bfloat16)
    with pytest.raises(AssertionError, match="mean-abs"):
        assert_close("x", got, ref, torch.bfloat16)


def test_non_finite_outputs_fail():
    ref = np.zeros(4)
    got = torch.tensor([0.0, float("nan"), 0.0, 0.0], dtype=torch.float16)
    with pytest.raises(AssertionError, match="non-finite"):
        assert_close("x", got, ref, torch.float16)
