"""CPU checks of the bf16 comparison rule and of the rounding emulation that
decides the input scale of the many-head backward tests."""
from __future__ import annotations

import numpy as np
import pytest

import bwd_rounding
from parity import BF16_MAX_ABS, bf16_bound, bf16_check, bf16_ulp


def test_bound_adds_half_an_ulp_of_the_exact_value():
    x = np.array([0.0, 0.7, 1.0, 3.9, 4.0, 7.99, 8.0, 12.0, -9.0])
    np.testing.assert_allclose(bf16_bound(x), BF16_MAX_ABS + 0.5 * bf16_ulp(x))
    assert bf16_ulp(np.array([8.0]))[0] == 2.0 ** -4 and bf16_ulp(np.array([4.0]))[0] == 2.0 ** -5
    assert bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7 and bf16_ulp(np.array([0.0]))[0] == 0.0


def test_correct_rounding_alone_meets_the_bound():
    """The exact values, rounded to bf16, always pass; an fp32 value 2.1e-2
    off before rounding fails where the rounding happens to go the same way."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * 6
    assert bf16_check(bwd_rounding.to_bf16(x), x, True)[2] <= 0
    _, _, worst, n_allow = bf16_check(bwd_rounding.to_bf16(x + 0.021), x, True)
    assert worst > 0 and n_allow > 0


def test_check_counts_allowance_elements():
    want = np.array([9.0, 9.0, 1.0])
    got = np.array([9.04, 9.0, 1.0])       # 0.04 > 2e-2 but within 2e-2 + 1/32
    mx, _, worst, n_allow = bf16_check(got, want, True)
    assert abs(mx - 0.04) < 1e-12 and worst < 0 and n_allow == 1
    assert bf16_check(got, want, False)[2] > 0   # fp32 outputs get no allowance


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", bwd_rounding.MANY_HEADS)
def test_many_heads_rounding_alone_meets_the_bound(shape, causal):
    """With N(0,1) inputs, rounding P and dS to bf16 (everything else exact)
    keeps the backward of 8 and 16 query heads per kv head inside the bound,
    so the GPU tests of those shapes can hold the kernel to it."""
    rep = bwd_rounding.emulation_report(shape, causal)
    assert all(r[2] <= 0 and r[1] <= 2e-3 for r in rep.values()), {k: v[:3] for k, v in rep.items()}


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", bwd_rounding.ODD_GROUPS)
def test_odd_group_sweep_rounding_alone_meets_the_bound(shape, causal):
    """The backward sweep cases with 3, 6 and 5 query heads per kv head, on
    the sweep's own inputs (N(0,1)): rounding P and dS alone stays inside the
    bound, so the GPU sweep can hold the kernels to it at full input scale."""
    rep = bwd_rounding.emulation_report(shape, causal, seed=bwd_rounding.sweep_seed(shape))
    assert all(r[2] <= 0 and r[1] <= 2e-3 for r in rep.values()), {k: v[:3] for k, v in rep.items()}


def test_allowance_only_from_8_would_be_unattainable():
    """Why the output-rounding allowance applies at every magnitude: with it
    only where half an ulp exceeds 2e-2 (|x| >= 8), rounding P and dS alone
    breaks the bound for 16 query heads per kv head, causal, N(0,1)."""
    def strict(x):
        half = 0.5 * bf16_ulp(x)
        return np.where(half > BF16_MAX_ABS, BF16_MAX_ABS + half, BF16_MAX_ABS)

    rep = bwd_rounding.emulation_report((2, 200, 16, 1, 128), True, bound=strict)
    assert rep["dV"][2] > 0, rep
