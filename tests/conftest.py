import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")
    config.addinivalue_line("markers", "slow: full-size parity at the workload shapes")


def half_ulp_bf16(x):
    """Half a unit in the last place of bfloat16 (8-bit significand) at |x|: the
    largest error of rounding x to the nearest bf16 value."""
    import numpy as np
    _, e = np.frexp(np.abs(np.asarray(x, dtype=np.float64)))
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 9))


def tol_check(got, ref, max_abs, rel_fro, what="", out_bf16=False):
    """The parity bar: max-abs error and relative Frobenius error, both bounded.

    With out_bf16 the result is stored as bfloat16, which cannot represent the
    exact value closer than half an ulp; the max-abs bound then applies to the
    error before that final rounding: |got - ref| <= max_abs + half_ulp_bf16(ref)
    per element (at |ref| < 4 the allowance is at most 2^-7)."""
    import numpy as np
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in result"
    err = np.abs(got - ref)
    mae = float(err.max()) if err.size else 0.0
    bound = max_abs + (half_ulp_bf16(ref) if out_bf16 else 0.0)
    excess = float((err - bound).max()) if err.size else -1.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))
    assert excess <= 0 and rel <= rel_fro, (f"{what}: max_abs={mae:.3e} (bound {max_abs}"
                                             f"{' + half bf16 ulp' if out_bf16 else ''}, worst excess {excess:.3e}),"
                                             f" rel_fro={rel:.3e} (<= {rel_fro})")
    return mae, rel
