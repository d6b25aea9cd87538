"""The parity helper's bf16 rounding allowance: it is the rounding error bound,
and it only replaces the 2e-2 bar where a correctly rounded value cannot meet it."""

import numpy as np
import torch

from conftest import elementwise_bound, half_ulp_bf16, tol_check


def test_half_ulp_bounds_bf16_rounding_and_is_tight():
    x = (np.random.default_rng(0).standard_normal(200000) * 8).astype(np.float32).astype(np.float64)
    r = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    err = np.abs(r - x)
    h = half_ulp_bf16(x)
    assert np.all(err <= h)
    assert np.max(err / h) > 0.99          # tight: some values sit near a midpoint
    assert half_ulp_bf16(np.array([1.0]))[0] == 2.0 ** -8
    assert half_ulp_bf16(np.array([8.5]))[0] == 2.0 ** -5


def test_bound_is_exactly_max_abs_below_8():
    ref = np.linspace(-7.999, 7.999, 10001)
    assert np.all(elementwise_bound(ref, 2e-2, True) == 2e-2)
    big = np.array([8.0, -9.5, 15.9, 16.0, 100.0])
    b = elementwise_bound(big, 2e-2, True)
    assert np.all(b == half_ulp_bf16(big)) and np.all(b > 2e-2)
    # a correctly rounded bf16 value always meets the bound
    x = (np.random.default_rng(1).standard_normal(100000) * 20).astype(np.float64)
    r = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.all(np.abs(r - x) <= elementwise_bound(x, 2e-2, True))


def test_tol_check_rejects_real_errors():
    ref = np.linspace(-4, 4, 1000)
    tol_check(ref + 0.015, ref, 2e-2, 1e-2)
    for bad in (ref + 0.021, ref * 1.02, np.where(np.arange(1000) == 7, ref + 0.025, ref)):
        try:
            tol_check(bad, ref, 2e-2, 1e-2, out_bf16=True)
        except AssertionError:
            continue
        raise AssertionError("tolerance check accepted a real error")
