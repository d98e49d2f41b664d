"""CPU checks of the GPU parity helpers' own arithmetic (no GPU).

The bf16 bar compares a kernel's bf16 output with the oracle's output rounded
to bf16, so the rounding helper must be round-to-nearest-even: it is checked
against torch's float32 -> bfloat16 conversion on float32 inputs (exact there,
no double rounding), on planted ties, and the bar itself on planted errors.
"""
import numpy as np
import pytest
import torch

from parity import Tally, round_bf16, ulp_bf16


def test_round_bf16_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-30, 30, 200_000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(round_bf16(x.astype(np.float64)), want)


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even significand (1)
    assert round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert round_bf16(np.array([-(1 + 2.0 ** -8)]))[0] == -1.0
    assert round_bf16(np.array([0.0]))[0] == 0.0


def test_ulp_bf16():
    assert ulp_bf16(np.array([1.0]))[0] == 2.0 ** -7
    assert ulp_bf16(np.array([1.99]))[0] == 2.0 ** -7
    assert ulp_bf16(np.array([-4.0]))[0] == 2.0 ** -5
    assert ulp_bf16(np.array([0.0]))[0] == 0.0


def test_bar_rounded_and_strict():
    ref = np.array([4.4, 0.1, -2.3])
    # a kernel output one bf16 step away from the rounded reference at 4.4
    # (spacing 2^-5 there) passes the rounded bar but not the strict one
    got = round_bf16(ref)
    got[0] += 2.0 ** -5
    t = Tally()
    t.add(got, ref, np.zeros(3))
    with pytest.raises(AssertionError):
        t.check("bf16", "planted", out_bf16=True, strict=True)
    # the mean bound of 1e-3 is not widened: three elements, one off by 2^-5
    with pytest.raises(AssertionError):
        t.check("bf16", "planted", out_bf16=True)
    t2 = Tally()
    big = np.concatenate([ref, np.full(100, 0.25)])
    g2 = round_bf16(big)
    g2[0] += 2.0 ** -5
    t2.add(g2, big, np.zeros(big.size))
    t2.check("bf16", "planted, diluted", out_bf16=True)
    with pytest.raises(AssertionError):
        t2.check("bf16", "planted, diluted", out_bf16=True, strict=True)
