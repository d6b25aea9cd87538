"""The parity helper's bf16 rounding allowance: it is the rounding error bound,
and it only replaces the 2e-2 bar where a correctly rounded value cannot meet it."""

import numpy as np
import pytest
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


def _fp8_round_p(p):
    """P rounded as the fp8 forward rounds it: times 2^8, to OCP e4m3 (torch's
    round to nearest), back, divided by 2^8."""
    t = torch.from_numpy(np.ascontiguousarray(p * 256.0, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy() / 256.0


def test_fp8_o_bound_holds_for_simulated_rounding_and_is_not_vacuous():
    """The fp8 forward's bar (parity_util.check_fp8_o) against a CPU model of its
    rounding: P relative to the exact row max, rounded to e4m3 after scaling by
    2^8, the row sum over the unrounded P.  The model meets the bar; the same
    model with each row's previous key dropped, or with the values of
    neighbouring keys swapped (P and V paired on different keys), exceeds it."""
    from parity_util import check_fp8_o
    from workloads import fp8_inputs
    import oracle
    B, T, H, KV, D, W = 1, 300, 2, 1, 128, 100
    (q8, k8, v8), (dq, dk, dv) = fp8_inputs(B, T, H, KV, D, seed=3)
    q, k, v = (x.to(torch.float64).numpy() * d for x, d in ((q8, dq), (k8, dk), (v8, dv)))
    ro, _ = oracle.attn_fwd(q, k, v, W)
    ra, _ = oracle.attn_fwd(q, k, np.abs(v), W)

    def model(drop_prev=False, swap_keys=False):
        o = np.zeros_like(ro)
        for h in range(H):
            s = q[0, :, h] @ k[0, :, h // (H // KV)].T / np.sqrt(D)
            i, j = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
            vis = (j <= i) & (i - j <= W)
            if drop_prev:
                vis &= j != i - 1
            s = np.where(vis, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            l = p.sum(axis=1, keepdims=True)
            vh = v[0, :, h // (H // KV)]
            if swap_keys:
                vh = vh[np.arange(T) ^ 1 if T % 2 == 0 else np.minimum(np.arange(T) ^ 1, T - 1)]
            o[0, :, h] = (_fp8_round_p(p) @ vh) / l
        return torch.from_numpy(o).to(torch.bfloat16).double().numpy()

    check_fp8_o(model(), ro, ra, v, W, "model")
    with pytest.raises(AssertionError):
        check_fp8_o(model(drop_prev=True), ro, ra, v, W, "model missing each row's previous key")
    with pytest.raises(AssertionError):
        check_fp8_o(model(swap_keys=True), ro, ra, v, W, "model with neighbouring keys' values swapped")
