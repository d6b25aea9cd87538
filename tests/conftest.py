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


def elementwise_bound(ref, max_abs, out_bf16):
    """Per-element max-abs bound.  A bf16 result cannot be stored closer to the
    exact value than half a bf16 ulp, which exceeds 2e-2 only where |ref| >= 8
    (half an ulp is 2^-5 there).  So for bf16 results the bound is
    max(max_abs, half_ulp_bf16(ref)): exactly max_abs wherever a correctly rounded
    value can meet it, and the rounding bound itself where none can."""
    import numpy as np
    if not out_bf16:
        return max_abs
    return np.maximum(max_abs, half_ulp_bf16(ref))


def tol_check(got, ref, max_abs, rel_fro, what="", out_bf16=False):
    """The parity bar: max-abs error (per element, see elementwise_bound) and
    relative Frobenius error ||got - ref|| / ||ref||, both bounded.  Returns the
    raw (max-abs, rel-Frobenius) errors and prints them."""
    import numpy as np
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in result"
    err = np.abs(got - ref)
    mae = float(err.max()) if err.size else 0.0
    bound = elementwise_bound(ref, max_abs, out_bf16)
    excess = float((err - bound).max()) if err.size else -1.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))
    print(f"  {what}: max_abs={mae:.3e} rel_fro={rel:.3e}", file=sys.stderr, flush=True)
    where = ""
    if excess > 0:
        i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        where = f", worst at {tuple(int(x) for x in i)}: got {got[i]:.6g} ref {ref[i]:.6g}"
    assert excess <= 0 and rel <= rel_fro, (f"{what}: max_abs={mae:.3e} (bound {max_abs}"
                                             f"{' or half a bf16 ulp where |ref| >= 8' if out_bf16 else ''}, "
                                             f"worst excess {excess:.3e}{where}), rel_fro={rel:.3e} (<= {rel_fro})")
    return mae, rel
