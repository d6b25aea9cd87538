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
# LSE is fp32 in both paths; its error comes from fp32 accumulation only (both
# sides see the same stored inputs).
LSE_TOL = {"bf16": 1e-3, "f32": 1e-5}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def stored(x, dtype):
    """The oracle's float64 result as the library stores it in the I/O dtype
    (round to nearest even): QK-norm + RoPE writes q' and k' back into bf16 (or
    fp32) tensors, and the attention that follows reads those stored values.  A
    chained comparison feeds the oracle's own q', k', rounded this way, to the
    oracle's attention; nothing here comes from the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)
    return t.double().numpy()


def group_slice(q, k, v, do, b, g, G):
    """Inputs of kv head g of sequence b: q/do heads [g*G, (g+1)*G), k/v head g."""
    hs = slice(g * G, (g + 1) * G)
    return (q[b:b + 1, :, hs], k[b:b + 1, :, g:g + 1], v[b:b + 1, :, g:g + 1],
            None if do is None else do[b:b + 1, :, hs])


def check(got, ref, dtype, what):
    return tol_check(f64(got) if isinstance(got, torch.Tensor) else got, ref, what=what, out_bf16=dtype == "bf16",
                     **TOL[dtype])


def check_lse(got, ref, dtype, what, tol=None):
    import sys
    g = f64(got) if isinstance(got, torch.Tensor) else got
    tol = LSE_TOL[dtype] if tol is None else tol
    err = float(np.abs(g - ref).max()) if g.size else 0.0
    print(f"  {what}: max_abs={err:.3e}", file=sys.stderr, flush=True)
    assert np.all(np.isfinite(g)), f"{what}: non-finite lse"
    assert err <= tol, f"{what}: lse max_abs={err:.3e} > {tol:.3e}"
    return err


def check_fp8_o(got, ref, ref_abs, v, window, what):
    """Element-wise bar of the fp8 forward's o (derived in the header of its
    kernel): each probability P_ij enters P V rounded to e4m3 after scaling by
    2^8, a relative error of at most 2^-4, or an absolute 2^-18 (relative to the
    row max) below e4m3's normal range; the row sum is exact fp32.  So
        |o_id - o_exact,id| <= 2^-4 sum_j P_ij |v_jd| + n_i 2^-18 max_j |v_jd|
    for row i with n_i visible keys, plus the bf16 rounding of o (one ulp of the
    exact value: half an ulp of a value that may sit a binade higher) and 1e-6 of
    fp32 accumulation.  ref_abs = sum_j P_ij |v_jd| is the oracle's forward of the
    same q, k with |v| in place of v; v: the float64 values [B][T][KV][D]."""
    import sys
    g = f64(got) if isinstance(got, torch.Tensor) else got
    B, T, H, D = ref.shape
    vmax = np.abs(v).max(axis=(0, 1, 2))  # per column d
    i = np.arange(T)
    n = i + 1 if window < 0 else np.minimum(i + 1, window + 1)
    e = np.floor(np.log2(np.maximum(np.abs(ref), 1e-30)))
    bound = 2.0 ** -4 * ref_abs + n[None, :, None, None] * 2.0 ** -18 * vmax[None, None, None, :] \
        + 2.0 ** (e - 7) + 1e-6
    err = np.abs(g - ref)
    rel_fro = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30))
    worst = float((err / bound).max()) if err.size else 0.0
    print(f"  {what}: max_abs={float(err.max()):.3e} rel_fro={rel_fro:.3e} worst err/bound={worst:.3f}",
          file=sys.stderr, flush=True)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    assert worst <= 1.0, f"{what}: error {float(err.max()):.3e} exceeds the fp8 bound (ratio {worst:.3f})"
    return err
