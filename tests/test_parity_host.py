"""CPU tests of the parity helpers the GPU tests use to decide pass or fail:
the bfloat16 rounding bound, the element-wise bound of assert_close and the
derived allowances.  A mistake here would pass wrong kernels or fail right
ones on every GPU test at once, so each rule is pinned to what it states."""
import math

import numpy as np
import pytest
import torch

from parity import (MANY_ROWS_PER_KEY, RTOL_BF16_TERMS, TOL_F32, assert_close, bf16_grad_rtol,
                    fp32_score_tol, half_ulp_bf16)


def test_half_ulp_bf16_bounds_round_to_nearest_even():
    # brute force over float32 values spread across many binades: torch's
    # float32 -> bfloat16 conversion (one rounding, to nearest even) never
    # moves a value by more than the bound, and the bound is reached at the
    # midpoints between two bfloat16 neighbours
    g = torch.Generator().manual_seed(0)
    x = (torch.rand(200000, generator=g) * 2 - 1) * torch.exp2(torch.randint(-30, 30, (200000,), generator=g).float())
    r = x.to(torch.bfloat16).to(torch.float64).numpy()
    x = x.to(torch.float64).numpy()
    err = np.abs(r - x)
    assert np.all(err <= half_ulp_bf16(np.maximum(np.abs(x), np.abs(r))))
    assert np.all(err <= half_ulp_bf16(x))
    for e in (-20, -1, 0, 3, 17):
        mid = 2.0 ** e * (1 + 2.0 ** -8)    # halfway between 2^e and its upper neighbour
        assert half_ulp_bf16(mid) == 2.0 ** (e - 8)
        got = float(torch.tensor(mid, dtype=torch.float32).to(torch.bfloat16).float())
        assert abs(got - mid) == half_ulp_bf16(mid)
    assert half_ulp_bf16(0.0) == 0.0
    assert half_ulp_bf16(-3.0) == half_ulp_bf16(3.0) == 2.0 ** -7


def test_assert_close_bound_is_tol_plus_rtol_times_magnitude():
    # powers of two, so that ref + bound is exact in float64
    ref = np.array([0.0, 1.0, -4.0, 128.0])
    tol, rtol = 2.0 ** -10, 2.0 ** -7
    bound = tol + rtol * np.abs(ref)
    assert_close("at the bound", ref + bound, ref, tol, rtol)
    assert_close("at the bound, below", ref - bound, ref, tol, rtol)
    for i in range(ref.size):
        got = ref + bound
        got[i] += 2.0 ** -30 * max(1.0, abs(ref[i]))
        with pytest.raises(AssertionError):
            assert_close(f"past the bound at {i}", got, ref, tol, rtol)


def test_assert_close_rtol_applies_only_from_its_threshold():
    ref = np.array([1.0, 30.0])
    got = ref + np.array([0.15, 1.5])
    # bounds 0.1 + 2^-4 |ref| = 0.1625 and 1.975: both pass
    assert_close("both", got, ref, 0.1, 2.0 ** -4)
    # from 20 on only: the first element is held to 0.1
    with pytest.raises(AssertionError):
        assert_close("small element held to tol", got, ref, 0.1, 2.0 ** -4, rtol_from=20.0)
    assert_close("only the large element", got[1:], ref[1:], 0.1, 2.0 ** -4, rtol_from=20.0)
    # an explicit magnitude replaces |ref|
    assert_close("mag", got, ref, 0.1, 2.0 ** -4, mag=np.array([30.0, 30.0]), rtol_from=20.0)


def test_assert_close_adds_the_bf16_output_rounding():
    ref = np.array([9.0, 0.25])
    got = torch.tensor([9.0 + 2.0 ** -5, 0.25], dtype=torch.float32)
    # 2^-5 exceeds tol 2e-2 but is within 2e-2 + half an ulp at 9 (2^-5)
    with pytest.raises(AssertionError):
        assert_close("fp32 result", got, ref, 2e-2)
    assert_close("as a bf16 result", got, ref, 2e-2, rounded_bf16=True)
    assert_close("bf16 tensor", got.to(torch.bfloat16), ref, 2e-2)


def test_assert_close_rejects_non_finite_and_shape_mismatch_and_accepts_empty():
    with pytest.raises(AssertionError):
        assert_close("nan", np.array([np.nan]), np.array([0.0]), 1.0)
    with pytest.raises(AssertionError):
        assert_close("inf", np.array([np.inf]), np.array([np.inf]), 1.0)
    with pytest.raises(AssertionError):
        assert_close("shape", np.zeros(3), np.zeros(4), 1.0)
    assert assert_close("empty", np.zeros(0), np.zeros(0), 1e-5) == 0.0


def test_bf16_gradient_allowance_only_for_many_rows_per_key():
    assert bf16_grad_rtol(torch.float32, 10000, 1) == 0.0
    assert bf16_grad_rtol(torch.bfloat16, 4096, 4096) == 0.0
    assert bf16_grad_rtol(torch.bfloat16, MANY_ROWS_PER_KEY * 5 - 1, 5) == 0.0
    assert bf16_grad_rtol(torch.bfloat16, MANY_ROWS_PER_KEY * 5, 5) == RTOL_BF16_TERMS
    # shared K/V heads: every query head of the group adds its rows to each key
    assert bf16_grad_rtol(torch.bfloat16, MANY_ROWS_PER_KEY * 5 // 4, 5, group=4) == RTOL_BF16_TERMS


def test_fp32_score_bound_follows_the_score_magnitude():
    q = torch.ones(1, 1, 4, 64)
    k = torch.ones(1, 1, 6, 64)
    v = torch.ones(1, 1, 6, 64)
    scale = 1 / math.sqrt(64)
    # scores of 0.8: the estimate 8 * sqrt(64) * 2^-24 * 0.8 is below 1e-5
    assert fp32_score_tol(q * 0.1, k, v, scale) == TOL_F32
    big = fp32_score_tol(q * 1000, k, v, scale)
    assert big == pytest.approx(8 * 8 * 2.0 ** -24 * 8000)
    assert fp32_score_tol(q * 1000, k, v * 3, scale) == pytest.approx(3 * big)
