"""The parity helper's bf16 rounding allowance is exactly the rounding error bound."""

import numpy as np
import torch

from conftest import half_ulp_bf16, tol_check


def test_half_ulp_bounds_bf16_rounding_and_is_tight():
    x = (np.random.default_rng(0).standard_normal(200000) * 8).astype(np.float32).astype(np.float64)
    r = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    err = np.abs(r - x)
    h = half_ulp_bf16(x)
    assert np.all(err <= h)
    assert np.max(err / h) > 0.99          # tight: some values sit near a midpoint
    assert half_ulp_bf16(np.array([1.0]))[0] == 2.0 ** -8
    assert half_ulp_bf16(np.array([8.5]))[0] == 2.0 ** -5


def test_tol_check_rejects_real_errors():
    ref = np.linspace(-4, 4, 1000)
    tol_check(ref + 0.015, ref, 2e-2, 1e-2)
    for bad in (ref + 0.03, ref * 1.02):
        try:
            tol_check(bad, ref, 2e-2, 1e-2, out_bf16=True)
        except AssertionError:
            continue
        raise AssertionError("tolerance check accepted a real error")
