import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP library")
    config.addinivalue_line("markers", "slow: full-size parity at the workload shapes")


def tol_check(got, ref, max_abs, rel_fro, what=""):
    """The parity bar: max-abs error and relative Frobenius error, both bounded."""
    import numpy as np
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in result"
    err = np.abs(got - ref)
    mae = float(err.max()) if err.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got - ref))
    assert mae <= max_abs and rel <= rel_fro, f"{what}: max_abs={mae:.3e} (<= {max_abs}), rel_fro={rel:.3e} (<= {rel_fro})"
    return mae, rel
