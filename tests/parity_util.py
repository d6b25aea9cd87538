"""Helpers for GPU-vs-oracle parity tests: tolerances, slicing one kv group out of
a batch so the oracle only computes what is sampled, and tensor conversion."""

import numpy as np
import torch

from conftest import tol_check

# Parity bars: bf16 I/O with fp32 accumulation, and fp32 throughout.
TOL = {
    "bf16": dict(max_abs=2e-2, rel_fro=1e-2),
    "f32": dict(max_abs=1e-4, rel_fro=1e-4),
}
# LSE is fp32 in both paths; its error comes from the bf16 rounding of the inputs
# already seen by both sides plus fp32 accumulation.
LSE_TOL = {"bf16": 1e-3, "f32": 1e-5}


def lse_tol_after_bf16_inputs(D, gain=1.0):
    """LSE bound when the attention inputs are the bf16-rounded output of the
    QK-norm step on the GPU but exact on the oracle side.  Rounding q and k to
    bf16 moves each score by at most scale * sum_d |q_d k_d| * 2^-8 <=
    (1/sqrt(D)) * |q| |k| * 2^-8 = sqrt(D) gain^2 2^-8 (|q| = |k| = gain sqrt(D)
    after RMSNorm), and LSE is 1-Lipschitz in the max-norm of the scores."""
    return LSE_TOL["bf16"] + (D ** 0.5) * gain * gain * 2.0 ** -8


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def group_slice(q, k, v, do, b, g, G):
    """Inputs of kv head g of sequence b: q/do heads [g*G, (g+1)*G), k/v head g."""
    hs = slice(g * G, (g + 1) * G)
    return (q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1],
            None if do is None else do[b:b + 1, :, hs])


def check(got, ref, dtype, what):
    return tol_check(f64(got) if isinstance(got, torch.Tensor) else got, ref, what=what, out_bf16=dtype == "bf16",
                     **TOL[dtype])


def check_lse(got, ref, dtype, what, tol=None):
    g = f64(got) if isinstance(got, torch.Tensor) else got
    tol = LSE_TOL[dtype] if tol is None else tol
    err = float(np.abs(g - ref).max()) if g.size else 0.0
    assert np.all(np.isfinite(g)), f"{what}: non-finite lse"
    assert err <= tol, f"{what}: lse max_abs={err:.3e} > {tol:.3e}"
    return err
