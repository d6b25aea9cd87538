"""GPU parity of every hot-path call against the CPU oracle, element by element,
at sizes the oracle finishes in seconds that still span several tiles and a
ragged tail, plus the edge cases: T = 1, windows 0 / 1 / tile-1 / tile / tile+1 /
T-1 / larger than T, GQA groups, empty and full caches, invalid cache lengths,
NaN-poisoned cache slots, and run-twice determinism."""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_qknorm_amd as nc
from conftest import tol_check
from parity_util import LSE_TOL, TOL, check, check_fp8_o, check_lse, f64, stored
from workloads import attn_inputs, decode_inputs, fp8_inputs, prefill_inputs, replicate_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(*ts):
    return [t.to(DEV) for t in ts]


# ------------------------------------------------------------------ QK-norm + RoPE

@pytest.mark.parametrize("dtype,B,T,H,KV,D,base,gain,offset", [
    ("f32", 1, 64, 2, 2, 64, 10000.0, 1.0, False),
    ("f32", 2, 37, 4, 2, 128, 100000.0, math.sqrt(1.2), True),
    ("bf16", 3, 130, 6, 6, 128, 100000.0, 1.0, False),
    ("bf16", 64, 1, 10, 10, 128, 100000.0, 1.0, True),     # decode: one token at pos = cache length
    ("bf16", 2, 50, 12, 4, 64, 10000.0, math.sqrt(1.2), True),
])
def test_qknorm_rope(dtype, B, T, H, KV, D, base, gain, offset):
    say(f"qknorm_rope {dtype} B={B} T={T} H={H} KV={KV} D={D}")
    q, k, v, _ = attn_inputs(B, T, H, KV, D, dtype, seed=11)
    pos = torch.from_numpy(np.random.default_rng(3).integers(0, 8192, size=B).astype(np.int32)) if offset else None
    ref_q, ref_k = oracle.qknorm_rope(f64(q), f64(k), None if pos is None else pos.numpy(), base, 1e-6, gain)
    qd, kd, vd = to_dev(q, k, v)
    v_before = vd.clone()
    nc.qknorm_rope_(qd, kd, None if pos is None else pos.to(DEV), rope_base=base, eps=1e-6, qk_gain=gain)
    torch.cuda.synchronize()
    check(qd, ref_q, dtype, "q")
    check(kd, ref_k, dtype, "k")
    assert torch.equal(vd, v_before)


@pytest.mark.parametrize("dtype,B,T,H,KV,D,base,gain,offset", [
    ("f32", 1, 64, 2, 2, 64, 10000.0, 1.0, False),
    ("f32", 2, 37, 4, 2, 128, 100000.0, math.sqrt(1.2), True),
    ("bf16", 3, 130, 6, 6, 128, 100000.0, 1.0, False),
    ("bf16", 64, 1, 10, 10, 128, 100000.0, 1.0, True),
    ("bf16", 2, 50, 12, 4, 64, 10000.0, math.sqrt(1.2), True),
])
def test_qknorm_rope_bwd(dtype, B, T, H, KV, D, base, gain, offset):
    say(f"qknorm_rope_bwd {dtype} B={B} T={T} H={H} KV={KV} D={D}")
    q, k, _, _ = attn_inputs(B, T, H, KV, D, dtype, seed=21)
    gq, gk, _, _ = attn_inputs(B, T, H, KV, D, dtype, seed=22)
    pos = torch.from_numpy(np.random.default_rng(4).integers(0, 8192, size=B).astype(np.int32)) if offset else None
    ref_q, ref_k = oracle.qknorm_rope_bwd(f64(q), f64(k), f64(gq), f64(gk), None if pos is None else pos.numpy(),
                                          base, 1e-6, gain)
    qd, kd, gqd, gkd = to_dev(q, k, gq, gk)
    q_before, k_before = qd.clone(), kd.clone()
    nc.qknorm_rope_bwd_(gqd, gkd, qd, kd, None if pos is None else pos.to(DEV), rope_base=base, eps=1e-6,
                        qk_gain=gain)
    torch.cuda.synchronize()
    check(gqd, ref_q, dtype, "dq_in")
    check(gkd, ref_k, dtype, "dk_in")
    assert torch.equal(qd, q_before) and torch.equal(kd, k_before)


@pytest.mark.parametrize("dtype,B,T,H,KV,D", [("bf16", 2, 100, 4, 2, 128), ("bf16", 1, 77, 6, 6, 64),
                                               ("f32", 2, 50, 3, 1, 64), ("f32", 1, 9, 2, 2, 128)])
def test_qknorm_rope_rstd(dtype, B, T, H, KV, D):
    """The variant that also stores 1/r: q', k' bit-equal to ncattn_qknorm_rope's,
    1/r of every row against the oracle (q rows, then k rows, per token)."""
    q, k, _, _ = attn_inputs(B, T, H, KV, D, dtype, seed=60 + T)
    pos = torch.arange(B, dtype=torch.int32) * 1000 + 3
    qa, ka = to_dev(q, k)
    qb, kb = to_dev(q, k)
    nc.qknorm_rope_(qa, ka, pos.to(DEV), rope_base=1e4, eps=1e-6, qk_gain=math.sqrt(1.2))
    _, _, rstd = nc.qknorm_rope_rstd_(qb, kb, pos.to(DEV), rope_base=1e4, eps=1e-6, qk_gain=math.sqrt(1.2))
    torch.cuda.synchronize()
    assert torch.equal(qa, qb) and torch.equal(ka, kb)
    ref = np.concatenate([oracle.rms_rstd(f64(q), 1e-6), oracle.rms_rstd(f64(k), 1e-6)], axis=2)
    np.testing.assert_allclose(f64(rstd), ref, rtol=1e-5)


# ------------------------------------------------------------------ fp8 forward
FP8_CASES = [
    # B, T, H, KV, W, softmax_scale
    (2, 200, 4, 2, -1, None),
    (1, 333, 8, 1, 100, None),
    (3, 130, 6, 6, 64, 0.05),
    (1, 1, 2, 1, -1, None),
    (2, 64, 4, 4, 0, None),
    (2, 129, 4, 2, 63, None),
    (1, 1000, 4, 2, 511, None),
    (1, 2048, 6, 2, -1, None),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "-".join(str(x) for x in c))
def test_fwd_fp8(case):
    """fp8 (OCP e4m3) q, k, v with per-tensor descales: o against the oracle's
    forward on the values they stand for, within the bound the fp8 rounding of P
    allows (check_fp8_o); lse to the fp32 bar; and the same o and lse on a second
    run."""
    B, T, H, KV, W, sc = case
    say(f"fwd_fp8 {case}")
    (q8, k8, v8), (dq, dk, dv) = fp8_inputs(B, T, H, KV, 128, seed=500 + T)
    qv, kv, vv = (x.to(torch.float64).numpy() * d for x, d in ((q8, dq), (k8, dk), (v8, dv)))
    ro, rlse = oracle.attn_fwd(qv, kv, vv, W, sc)
    ra, _ = oracle.attn_fwd(qv, kv, np.abs(vv), W, sc)
    qd, kd, vd = to_dev(q8, k8, v8)
    o, lse = nc.fwd_fp8(qd, kd, vd, dq, dk, dv, window=(W, 0), softmax_scale=sc)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    check_fp8_o(o, ro, ra, vv, W, "o")
    check_lse(lse, rlse, "bf16", "lse")
    o2, lse2 = nc.fwd_fp8(qd, kd, vd, dq, dk, dv, window=(W, 0), softmax_scale=sc)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "fp8 forward not deterministic"


@pytest.mark.parametrize("W", [-1, 300])
def test_fwd_fp8_scores_growing_along_the_keys(W):
    """Scores that rise by about 0.23 (natural units) per key, so that every
    64-key tile's row max exceeds the exponent reference by far more than 0.8 in
    base 2 and the reference moves (O and the row sum rescaled) on every tile:
    o and lse against the oracle on the values the fp8 bytes stand for."""
    B, T, H, KV, D = 1, 700, 2, 1, 128
    say(f"fwd_fp8 growing scores W={W}")
    q = np.zeros((B, T, H, D), np.float32)
    q[..., :64] = 2.0
    k = np.zeros((B, T, KV, D), np.float32)
    k[..., :64] = (0.02 * np.arange(T, dtype=np.float32))[None, :, None, None]
    rng = np.random.default_rng(77)
    v = rng.standard_normal((B, T, KV, D), dtype=np.float32)
    v8 = (torch.from_numpy(v) / (float(np.abs(v).max()) / 448.0)).to(torch.float8_e4m3fn)
    q8 = torch.from_numpy(q).to(torch.float8_e4m3fn)
    k8 = torch.from_numpy(k).to(torch.float8_e4m3fn)
    dq, dk, dv = 1.0, 1.0, float(np.abs(v).max()) / 448.0
    qv, kv, vv = (x.to(torch.float64).numpy() * d for x, d in ((q8, dq), (k8, dk), (v8, dv)))
    assert float(kv.max()) > 12.0  # e4m3 keeps the growth: scores reach ~150
    ro, rlse = oracle.attn_fwd(qv, kv, vv, W, None)
    ra, _ = oracle.attn_fwd(qv, kv, np.abs(vv), W, None)
    qd, kd, vd = to_dev(q8, k8, v8)
    o, lse = nc.fwd_fp8(qd, kd, vd, dq, dk, dv, window=(W, 0))
    torch.cuda.synchronize()
    check_fp8_o(o, ro, ra, vv, W, "o")
    check_lse(lse, rlse, "bf16", "lse")


def test_fwd_fp8_unsupported_head_dim():
    q8 = torch.zeros(1, 8, 2, 64, dtype=torch.float8_e4m3fn, device=DEV)
    with pytest.raises(nc.NcattnError, match="EUNSUPPORTED"):
        nc.fwd_fp8(q8, q8, q8, 1.0, 1.0, 1.0)


FUSED_CASES = [
    # dtype, B, T, H, KV, D, W, base, gain, pos_offset
    ("bf16", 2, 200, 4, 2, 128, -1, 100000.0, 1.0, False),
    ("bf16", 2, 333, 8, 1, 128, 100, 100000.0, math.sqrt(1.2), True),
    ("bf16", 1, 1, 2, 1, 128, -1, 100000.0, 1.0, True),
    ("bf16", 3, 130, 6, 6, 128, 64, 10000.0, 1.0, True),
    ("bf16", 1, 777, 6, 2, 128, 256, 100000.0, math.sqrt(1.2), False),
    ("bf16", 2, 200, 4, 2, 64, -1, 10000.0, 1.0, True),
    ("bf16", 1, 333, 8, 1, 64, 100, 100000.0, math.sqrt(1.2), False),
    ("f32", 2, 100, 4, 2, 64, 17, 10000.0, math.sqrt(1.2), True),
    ("f32", 1, 150, 3, 3, 128, -1, 100000.0, 1.0, False),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "-".join(str(x)[:6] for x in c))
def test_fwd_qknorm_rope(case):
    """The fused call: q and k normalised and rotated in place, then the forward
    on them; checked against the oracle's QK-norm + RoPE followed by its forward."""
    dtype, B, T, H, KV, D, W, base, gain, offset = case
    say(f"fwd_qknorm_rope {case}")
    q, k, v, _ = attn_inputs(B, T, H, KV, D, dtype, seed=300 + T)
    pos = torch.from_numpy(np.random.default_rng(5).integers(0, 8192, size=B).astype(np.int32)) if offset else None
    xq, xk = oracle.qknorm_rope(f64(q), f64(k), None if pos is None else pos.numpy(), base, 1e-6, gain)
    ro, rlse = oracle.attn_fwd(stored(xq, dtype), stored(xk, dtype), f64(v), W)
    qd, kd, vd = to_dev(q, k, v)
    v_before = vd.clone()
    rstd = nc.rstd_like(qd, kd)
    o, lse = nc.fwd_qknorm_rope_(qd, kd, vd, None if pos is None else pos.to(DEV), rope_base=base, eps=1e-6,
                                 qk_gain=gain, window=(W, 0), rstd=rstd)
    torch.cuda.synchronize()
    check(qd, xq, dtype, "q'")
    check(kd, xk, dtype, "k'")
    ref_rstd = np.concatenate([oracle.rms_rstd(f64(q), 1e-6), oracle.rms_rstd(f64(k), 1e-6)], axis=2)
    np.testing.assert_allclose(f64(rstd), ref_rstd, rtol=1e-5)
    check(o, ro, dtype, "o")
    check_lse(lse, rlse, dtype, "lse")
    assert torch.equal(vd, v_before)
    # the same result as the two calls it fuses
    q2, k2 = to_dev(q, k)
    nc.qknorm_rope_(q2, k2, None if pos is None else pos.to(DEV), rope_base=base, eps=1e-6, qk_gain=gain)
    o2, lse2 = nc.fwd(q2, k2, vd, window=(W, 0))
    torch.cuda.synchronize()
    assert torch.equal(kd, k2), "k' differs from the unfused call"
    check(o, f64(o2), dtype, "o vs unfused")


BWD_FUSED_CASES = [
    # dtype, B, T, H, KV, D, W, base, gain, pos_offset
    ("bf16", 2, 200, 4, 2, 128, -1, 100000.0, 1.0, False),
    ("bf16", 2, 333, 8, 1, 128, 100, 100000.0, math.sqrt(1.2), True),
    ("bf16", 1, 1, 2, 1, 128, -1, 100000.0, 1.0, True),
    ("bf16", 3, 130, 6, 6, 128, 64, 10000.0, 1.0, True),
    ("bf16", 1, 300, 6, 2, 64, 64, 10000.0, 1.0, True),
    ("bf16", 3, 130, 4, 4, 64, -1, 100000.0, math.sqrt(1.2), False),
    ("f32", 2, 100, 4, 2, 64, 17, 10000.0, math.sqrt(1.2), True),
    ("f32", 1, 150, 3, 3, 128, -1, 100000.0, 1.0, False),
]


@pytest.mark.parametrize("case", BWD_FUSED_CASES, ids=lambda c: "-".join(str(x)[:6] for x in c))
def test_bwd_qknorm_rope(case):
    """The fused backward: gradients of the raw q, k (and of v) through QK-norm +
    RoPE and attention, against the oracle's attention backward followed by its
    QK-norm + RoPE backward, and against the two separate calls."""
    dtype, B, T, H, KV, D, W, base, gain, offset = case
    say(f"bwd_qknorm_rope {case}")
    q, k, v, do = attn_inputs(B, T, H, KV, D, dtype, seed=400 + T)
    pos = torch.from_numpy(np.random.default_rng(6).integers(0, 8192, size=B).astype(np.int32)) if offset else None
    pn = None if pos is None else pos.numpy()
    xq, xk = oracle.qknorm_rope(f64(q), f64(k), pn, base, 1e-6, gain)
    sq, sk = stored(xq, dtype), stored(xk, dtype)
    ro, _ = oracle.attn_fwd(sq, sk, f64(v), W)
    rdy_q, rdy_k, rdv = oracle.attn_bwd(sq, sk, f64(v), f64(do), W, o=stored(ro, dtype))
    rdq, rdk = oracle.qknorm_rope_bwd(f64(q), f64(k), rdy_q, rdy_k, pn, base, 1e-6, gain)
    qr, kr, vd, dod = to_dev(q, k, v, do)
    pd = None if pos is None else pos.to(DEV)
    qn, kn = qr.clone(), kr.clone()
    _, _, rstd = nc.qknorm_rope_rstd_(qn, kn, pd, rope_base=base, eps=1e-6, qk_gain=gain)
    o, lse = nc.fwd(qn, kn, vd, window=(W, 0))
    before = [t.clone() for t in (qn, kn, rstd)]
    # from the post-norm rows and their 1/r only: the raw rows are not passed
    dq, dk, dv = nc.bwd_qknorm_rope(qn, kn, vd, o, lse, dod, rstd, pd, rope_base=base, qk_gain=gain, window=(W, 0))
    torch.cuda.synchronize()
    check(dq, rdq, dtype, "dq_raw")
    check(dk, rdk, dtype, "dk_raw")
    check(dv, rdv, dtype, "dv")
    assert all(torch.equal(a, b) for a, b in zip((qn, kn, rstd), before))
    # the attention backward followed by the norm's backward gives the same
    # gradients up to rounding: dv bit for bit; dq, dk each within the bar of the
    # exact values, so within twice the bar of each other (the two calls round the
    # post-norm gradients to the I/O dtype in between, the fused call does not)
    g = nc.bwd(qn, kn, vd, o, lse, dod, window=(W, 0))
    nc.qknorm_rope_bwd_(g[0], g[1], qr, kr, pd, rope_base=base, eps=1e-6, qk_gain=gain)
    torch.cuda.synchronize()
    assert torch.equal(dv, g[2])
    twice = {kk: 2 * vv for kk, vv in TOL[dtype].items()}
    for name, a, b in (("dq_raw", dq, g[0]), ("dk_raw", dk, g[1])):
        tol_check(f64(a), f64(b), what=f"{name} vs two calls", out_bf16=dtype == "bf16", **twice)


# ------------------------------------------------------------------ forward / backward

FWD_CASES = [
    # dtype, B, T, H, KV, D, W
    ("bf16", 2, 200, 4, 2, 128, -1),
    ("bf16", 2, 200, 4, 2, 128, 0),
    ("bf16", 2, 200, 4, 2, 128, 1),
    ("bf16", 2, 200, 4, 2, 128, 63),
    ("bf16", 2, 200, 4, 2, 128, 64),
    ("bf16", 2, 200, 4, 2, 128, 65),
    ("bf16", 2, 200, 4, 2, 128, 127),
    ("bf16", 2, 200, 4, 2, 128, 128),
    ("bf16", 2, 200, 4, 2, 128, 199),
    ("bf16", 2, 200, 4, 2, 128, 5000),
    ("bf16", 1, 1, 2, 1, 128, -1),
    ("bf16", 1, 64, 2, 2, 128, -1),
    ("bf16", 1, 129, 3, 1, 128, 20),
    ("bf16", 3, 520, 2, 2, 128, -1),
    ("bf16", 1, 777, 6, 2, 128, 256),
    ("bf16", 1, 300, 8, 1, 128, -1),   # eight query heads on one kv head: dK/dV sum over the group
    ("bf16", 2, 333, 8, 1, 128, 100),
    # many (sequence, head) blocks per CU
    ("bf16", 64, 300, 8, 2, 128, -1),
    ("bf16", 64, 300, 8, 2, 128, 100),
    # head_dim 64 (GPT-2's 768 / 12): the same edges
    ("bf16", 2, 200, 4, 2, 64, -1),
    ("bf16", 2, 200, 4, 2, 64, 0),
    ("bf16", 2, 200, 4, 2, 64, 1),
    ("bf16", 2, 200, 4, 2, 64, 63),
    ("bf16", 2, 200, 4, 2, 64, 65),
    ("bf16", 2, 200, 4, 2, 64, 128),
    ("bf16", 2, 200, 4, 2, 64, 199),
    ("bf16", 2, 200, 4, 2, 64, 5000),
    ("bf16", 1, 1, 2, 1, 64, -1),
    ("bf16", 3, 520, 2, 2, 64, -1),
    ("bf16", 1, 777, 6, 2, 64, 256),
    ("bf16", 1, 300, 8, 1, 64, -1),
    ("bf16", 64, 300, 12, 12, 64, 100),
    ("f32", 1, 64, 2, 2, 64, -1),
    ("f32", 2, 100, 4, 2, 64, 17),
    ("f32", 1, 150, 2, 1, 128, -1),
    ("f32", 1, 150, 3, 3, 128, 40),
]


def _ids(c):
    return "-".join(str(x) for x in c)


@pytest.mark.parametrize("case", FWD_CASES, ids=[_ids(c) for c in FWD_CASES])
def test_fwd_bwd(case):
    dtype, B, T, H, KV, D, W = case
    say(f"fwd/bwd {case}")
    q, k, v, do = attn_inputs(B, T, H, KV, D, dtype, seed=100 + T + W)
    ro, rlse = oracle.attn_fwd(f64(q), f64(k), f64(v), W)
    # the backward is handed the forward's output as stored (the I/O dtype)
    rdq, rdk, rdv = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), W, o=stored(ro, dtype))
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o, lse = nc.fwd(qd, kd, vd, window=(W, 0))
    torch.cuda.synchronize()
    check(o, ro, dtype, "o")
    check_lse(lse, rlse, dtype, "lse")
    dq, dk, dv = nc.bwd(qd, kd, vd, o, lse, dod, window=(W, 0))
    torch.cuda.synchronize()
    check(dq, rdq, dtype, "dq")
    check(dk, rdk, dtype, "dk")
    check(dv, rdv, dtype, "dv")


def test_long_sequence_window_sampled():
    """T = 32768 (256 query tiles, 512 key tiles), window 1024, on sampled rows.
    With inputs taken as post-norm the windowed attention is translation
    invariant, so the oracle runs on the slice [c - 2W, c + W + 128): query rows
    [c, c + 128) see their whole windows inside it (o, lse, dq), and every query
    that sees keys [c, c + 128) lies inside it with its whole window (dk, dv)."""
    B, T, H, KV, D, W, R = 1, 32768, 2, 1, 128, 1024, 128
    q, k, v, do = attn_inputs(B, T, H, KV, D, "bf16", seed=77)
    qd, kd, vd, dod = to_dev(q, k, v, do)
    o, lse = nc.fwd(qd, kd, vd, window=(W, 0))
    dq, dk, dv = nc.bwd(qd, kd, vd, o, lse, dod, window=(W, 0))
    torch.cuda.synchronize()
    for c in (T // 2 + 37, T - R):
        say(f"long sequence: rows [{c}, {c + R})")
        a, e = c - 2 * W, min(T, c + W + R)
        sq, sk, sv, sdo = (f64(t[:, a:e]) for t in (q, k, v, do))
        ro, rlse = oracle.attn_fwd(sq, sk, sv, W)
        rdq, rdk, rdv = oracle.attn_bwd(sq, sk, sv, sdo, W, o=stored(ro, "bf16"))
        r = slice(c - a, c - a + R)
        check(o[:, c:c + R], ro[:, r], "bf16", "o")
        check_lse(lse[:, :, c:c + R], rlse[:, :, r], "bf16", "lse")
        check(dq[:, c:c + R], rdq[:, r], "bf16", "dq")
        check(dk[:, c:c + R], rdk[:, r], "bf16", "dk")
        check(dv[:, c:c + R], rdv[:, r], "bf16", "dv")


def _random_cases(n, seed=2024, D=128):
    """Seeded random shapes (bf16): ragged T in [1, 400], group sizes 1-4, windows
    unbounded or drawn up to T + 50 (so some exceed T)."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 401))
        KV, G = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        W = -1 if rng.random() < 0.4 else int(rng.integers(0, T + 51))
        cases.append(("bf16", B, T, KV * G, KV, D, W))
    return cases


RANDOM_CASES = _random_cases(12) + _random_cases(6, seed=2028, D=64)


def _random_f32_cases(n, seed=2027):
    """Seeded random shapes for the fp32 kernels: head_dim 64 or 128, T in
    [1, 260], group sizes 1-3, random windows."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B, T = int(rng.integers(1, 3)), int(rng.integers(1, 261))
        KV, G = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        D = 64 if rng.random() < 0.5 else 128
        W = -1 if rng.random() < 0.4 else int(rng.integers(0, T + 51))
        cases.append(("f32", B, T, KV * G, KV, D, W))
    return cases


RANDOM_CASES += _random_f32_cases(6)


@pytest.mark.parametrize("case", RANDOM_CASES, ids=[_ids(c) for c in RANDOM_CASES])
def test_fwd_bwd_random_shapes(case):
    test_fwd_bwd(case)


@pytest.mark.parametrize("D", [128, 64])
def test_fwd_bwd_closed_forms_on_gpu(D):
    """W = 0 gives O = v, dQ = dK = 0, dV = sum of the group's dO (exact up to rounding)."""
    q, k, v, do = to_dev(*attn_inputs(2, 300, 4, 2, D, "bf16", seed=9))
    o, lse = nc.fwd(q, k, v, window=(0, 0))
    torch.cuda.synchronize()
    assert torch.equal(o, v.repeat_interleave(2, dim=2))
    dq, dk, dv = nc.bwd(q, k, v, o, lse, do, window=(0, 0))
    torch.cuda.synchronize()
    # dS = P (dP - D) vanishes exactly in exact arithmetic; fp32 rounding of dP and D leaves ~1e-6
    assert float(dq.abs().max()) <= 1e-5 and float(dk.abs().max()) <= 1e-5
    ref = f64(do).reshape(2, 300, 2, 2, D).sum(axis=3)
    check(dv, ref, "bf16", "dv(W=0)")


@pytest.mark.parametrize("D", [128, 64])
def test_fwd_bwd_scores_far_above_first_tile(D):
    """Rows whose first key tile scores about -44 and whose later keys score about
    +44 (natural log units): the probabilities against the first tile's reference
    would overflow fp32, so the forward must take its exact-maximum second pass.
    Checked against the oracle like any other case, backward included.  (q is
    100 u, k is +-5 u plus unit noise, for a random unit vector u: a large common
    part in k would make the bf16 rounding of dS dominate dQ, which the exact
    cancellation sum_j dS_ij = 0 leaves small.)"""
    B, T, H, KV = 1, 300, 2, 2
    rng = np.random.default_rng(77)
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    sign = np.where(np.arange(T) < 100, -1.0, 1.0)[None, :, None, None]
    q = 100.0 * u + 0.5 * rng.standard_normal((B, T, H, D))
    k = sign * 5.0 * u + rng.standard_normal((B, T, KV, D))
    v = rng.standard_normal((B, T, KV, D))
    do = rng.standard_normal((B, T, H, D))
    q, k, v, do = (torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16) for x in (q, k, v, do))
    for W in (-1, 150):
        say(f"large score growth W={W}")
        ro, rlse = oracle.attn_fwd(f64(q), f64(k), f64(v), W)
        rdq, rdk, rdv = oracle.attn_bwd(f64(q), f64(k), f64(v), f64(do), W, o=stored(ro, "bf16"))
        assert float(rlse.max() - rlse.min()) > 60.0  # the construction does what it says
        qd, kd, vd, dod = to_dev(q, k, v, do)
        o, lse = nc.fwd(qd, kd, vd, window=(W, 0))
        torch.cuda.synchronize()
        check(o, ro, "bf16", "o")
        check_lse(lse, rlse, "bf16", "lse")
        dq, dk, dv = nc.bwd(qd, kd, vd, o, lse, dod, window=(W, 0))
        torch.cuda.synchronize()
        # The gradients here reach ~100 (q is 100 u), so the absolute bound,
        # stated for unit-scale data, is applied to the gradients divided by their
        # largest reference magnitude (rounded up to a power of 2); the relative Frobenius bound is unchanged.
        for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
            m = 2.0 ** max(0, math.ceil(math.log2(float(np.abs(ref).max()))))  # exact binary scaling
            tol_check(f64(got) / m, ref / m, what=name, out_bf16=True, **TOL["bf16"])


@pytest.mark.parametrize("D", [128, 64])
def test_determinism(D):
    q, k, v, do = to_dev(*attn_inputs(2, 700, 6, 2, D, "bf16", seed=5))
    for W in (-1, 100):
        o1, l1 = nc.fwd(q, k, v, window=(W, 0))
        o2, l2 = nc.fwd(q, k, v, window=(W, 0))
        g1 = nc.bwd(q, k, v, o1, l1, do, window=(W, 0))
        g2 = nc.bwd(q, k, v, o1, l1, do, window=(W, 0))
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        for a, b in zip(g1, g2):
            assert torch.equal(a, b)


def test_window_reaching_every_key_is_full_causal():
    """window_left >= T - 1 (up to INT_MAX) is the same attention as -1: bit-equal
    results from the forward, the backward (same workspace size) and decode."""
    q, k, v, do = to_dev(*attn_inputs(2, 333, 6, 2, 128, "bf16", seed=6))
    o_ref, l_ref = nc.fwd(q, k, v, window=(-1, 0))
    g_ref = nc.bwd(q, k, v, o_ref, l_ref, do, window=(-1, 0))
    for W in (332, 333, 2 ** 31 - 64, 2 ** 31 - 1):
        say(f"window {W}")
        o, l = nc.fwd(q, k, v, window=(W, 0))
        g = nc.bwd(q, k, v, o_ref, l_ref, do, window=(W, 0))
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref), W
        for a, b in zip(g, g_ref):
            assert torch.equal(a, b), W
    qd, kn, vn, kc, vc, lens = decode_inputs(5, 4, 2, 128, 1, 290, 300, seed=22, poison=True)
    ref = nc.decode(*to_dev(qd, kn, vn, kc.clone(), vc.clone(), lens), window=-1)
    for W in (299, 2 ** 31 - 1):
        o = nc.decode(*to_dev(qd, kn, vn, kc.clone(), vc.clone(), lens), window=W)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), W


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("W", [-1, 0, 1, 100, 127, 128, 129, 400])
def test_decode_small(W, D):
    say(f"decode small W={W} D={D}")
    B, H, KV, Tm = 6, 4, 2, 300
    q, kn, vn, kc, vc, lens = decode_inputs(B, H, KV, D, 1, 290, Tm, seed=21, poison=False)
    lens = torch.tensor([0, 1, 127, 128, 129, 299], dtype=torch.int32)
    # poison every slot from each sequence's length on (the oracle never reads them)
    for b in range(B):
        kc[b, int(lens[b]):] = float("nan")
        vc[b, int(lens[b]):] = float("nan")
    ro, rlse, rkc, rvc = oracle.decode(f64(q), f64(kn), f64(vn), f64(kc), f64(vc), lens.numpy(), W)
    qd, knd, vnd, kcd, vcd, ld = to_dev(q, kn, vn, kc, vc, lens)
    o, lse = nc.decode(qd, knd, vnd, kcd, vcd, ld, window=W, return_lse=True)
    torch.cuda.synchronize()
    check(o, ro, "bf16", "o")
    check_lse(lse, rlse, "bf16", "lse")
    # the new slot is written bit-exactly, every other slot is untouched (NaNs included)
    kc_after, vc_after = kcd.cpu(), vcd.cpu()
    for b in range(B):
        s = int(lens[b])
        assert torch.equal(kc_after[b, s], kn[b, 0]) and torch.equal(vc_after[b, s], vn[b, 0])
    mask = torch.ones(B, Tm, dtype=torch.bool)
    mask[torch.arange(B), lens.long()] = False
    for a, b_ in ((kc_after, kc), (vc_after, vc)):
        x, y = a[mask].view(torch.int16), b_[mask].view(torch.int16)
        assert torch.equal(x, y)


@pytest.mark.parametrize("W,D", [(-1, 128), (4096, 128), (-1, 64)])
def test_decode_long_cache(W, D):
    """Caches of 65600 slots with up to 65535 keys in use (512 split chunks for one
    sequence), slots past each length NaN-poisoned."""
    say(f"decode long cache W={W} D={D}")
    B, H, KV, Tm = 2, 4, 2, 65600
    q, kn, vn, kc, vc, lens = decode_inputs(B, H, KV, D, 1, 100, Tm, seed=23, poison=False)
    lens = torch.tensor([65535, 40001], dtype=torch.int32)
    for b in range(B):
        kc[b, int(lens[b]):] = float("nan")
        vc[b, int(lens[b]):] = float("nan")
    ro, rlse, _, _ = oracle.decode(f64(q), f64(kn), f64(vn), f64(kc), f64(vc), lens.numpy(), W)
    qd, knd, vnd, kcd, vcd, ld = to_dev(q, kn, vn, kc, vc, lens)
    o, lse = nc.decode(qd, knd, vnd, kcd, vcd, ld, window=W, return_lse=True)
    torch.cuda.synchronize()
    check(o, ro, "bf16", "o")
    check_lse(lse, rlse, "bf16", "lse")
    kc_after, vc_after = kcd.cpu(), vcd.cpu()
    for b in range(B):
        s = int(lens[b])
        assert torch.equal(kc_after[b, s], kn[b, 0]) and torch.equal(vc_after[b, s], vn[b, 0])
        assert torch.equal(kc_after[b, :s].view(torch.int16), kc[b, :s].view(torch.int16))


def _random_decode_cases(n, seed=2026, D=128):
    """Seeded random decode shapes: 1-8 sequences, cached lengths anywhere in
    [0, T_max - 1], group sizes 1-4, random windows."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B, KV, G = int(rng.integers(1, 9)), int(rng.integers(1, 4)), int(rng.integers(1, 5))
        Tm = int(rng.integers(2, 600))
        W = -1 if rng.random() < 0.4 else int(rng.integers(0, Tm + 51))
        cases.append((B, KV * G, KV, Tm, W, D))
    return cases


RANDOM_DECODE_CASES = _random_decode_cases(8) + _random_decode_cases(4, seed=2029, D=64)


@pytest.mark.parametrize("case", RANDOM_DECODE_CASES, ids=[_ids(c) for c in RANDOM_DECODE_CASES])
def test_decode_random_shapes(case):
    B, H, KV, Tm, W, D = case
    say(f"decode {case}")
    q, kn, vn, kc, vc, lens = decode_inputs(B, H, KV, D, 0, Tm - 1, Tm, seed=40 + Tm, poison=True)
    ro, rlse, _, _ = oracle.decode(f64(q), f64(kn), f64(vn), f64(kc), f64(vc), lens.numpy(), W)
    qd, knd, vnd, kcd, vcd, ld = to_dev(q, kn, vn, kc, vc, lens)
    o, lse = nc.decode(qd, knd, vnd, kcd, vcd, ld, window=W, return_lse=True)
    torch.cuda.synchronize()
    check(o, ro, "bf16", "o")
    check_lse(lse, rlse, "bf16", "lse")
    kc_after, vc_after = kcd.cpu(), vcd.cpu()
    mask = torch.ones(B, Tm, dtype=torch.bool)
    for b in range(B):
        s_ = int(lens[b])
        assert torch.equal(kc_after[b, s_], kn[b, 0]) and torch.equal(vc_after[b, s_], vn[b, 0])
        mask[b, s_] = False
    for a, b_ in ((kc_after, kc), (vc_after, vc)):
        assert torch.equal(a[mask].view(torch.int16), b_[mask].view(torch.int16))


@pytest.mark.parametrize("W,D", [(0, 128), (100, 128), (511, 128), (-1, 128), (300, 64)])
def test_decode_many_groups(W, D):
    """512 (sequence, kv head) pairs with grouped query heads (G = 2): lengths across
    the whole cache (0 and T_max - 1 included), NaN-poisoned slots past them, two
    invalid lengths in the same batch (NaN rows, cache untouched)."""
    B, H, KV, Tm = 64, 16, 8, 700
    say(f"decode many groups W={W} D={D}")
    q, kn, vn, kc, vc, lens = decode_inputs(B, H, KV, D, 0, Tm - 1, Tm, seed=70 + D, poison=True)
    lens[0], lens[1] = 0, Tm - 1
    kc[1] = torch.nan_to_num(kc[1].float(), nan=0.5).to(kc.dtype)   # every slot of row 1 is read
    vc[1] = torch.nan_to_num(vc[1].float(), nan=-0.25).to(vc.dtype)
    lens[2], lens[3] = -1, Tm      # invalid
    ok = torch.ones(B, dtype=torch.bool)
    ok[2] = ok[3] = False
    ro, rlse, _, _ = oracle.decode(f64(q[ok]), f64(kn[ok]), f64(vn[ok]), f64(kc[ok]), f64(vc[ok]),
                                   lens[ok].numpy(), W)
    qd, knd, vnd, kcd, vcd, ld = to_dev(q, kn, vn, kc, vc, lens)
    o, lse = nc.decode(qd, knd, vnd, kcd, vcd, ld, window=W, return_lse=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    check(o[ok], ro, "bf16", "o")
    check_lse(lse[ok], rlse, "bf16", "lse")
    assert torch.isnan(o[~ok].float()).all() and torch.isnan(lse[~ok]).all()
    kc_after = kcd.cpu()
    for b in range(B):
        s_ = int(lens[b])
        if 0 <= s_ < Tm:
            assert torch.equal(kc_after[b, s_], kn[b, 0])
            keep = torch.ones(Tm, dtype=torch.bool)
            keep[s_] = False
            assert torch.equal(kc_after[b, keep].view(torch.int16), kc[b, keep].view(torch.int16))
        else:
            assert torch.equal(kc_after[b].view(torch.int16), kc[b].view(torch.int16))


@pytest.mark.parametrize("D", [128, 64])
def test_decode_matches_fwd_row(D):
    """Decode at position s equals row s of the forward over the prefix (the
    incremental computation equals the full one)."""
    B, T, H, KV = 3, 333, 6, 2
    q, k, v, _ = attn_inputs(B, T, H, KV, D, "bf16", seed=8)
    qd, kd, vd = to_dev(q, k, v)
    for W in (-1, 64):
        o_full, lse_full = nc.fwd(qd, kd, vd, window=(W, 0))
        s = T - 1
        kc = torch.zeros(B, T + 5, KV, D, dtype=torch.bfloat16, device=DEV)
        vc = torch.zeros_like(kc)
        kc[:, :s] = kd[:, :s]
        vc[:, :s] = vd[:, :s]
        lens = torch.full((B,), s, dtype=torch.int32, device=DEV)
        o, lse = nc.decode(qd[:, s:s + 1].contiguous(), kd[:, s:s + 1].contiguous(), vd[:, s:s + 1].contiguous(),
                           kc, vc, lens, window=W, return_lse=True)
        torch.cuda.synchronize()
        d = (o.float() - o_full[:, s:s + 1].float()).abs().max().item()
        assert d <= 1.6e-2, d
        assert (lse - lse_full[:, :, s]).abs().max().item() <= 1e-3


def test_decode_invalid_lengths_give_nan_and_leave_cache():
    B, H, KV, D, Tm = 3, 2, 2, 128, 64
    q, kn, vn, kc, vc, _ = decode_inputs(B, H, KV, D, 1, 10, Tm, seed=2, poison=False)
    lens = torch.tensor([-1, 5, Tm], dtype=torch.int32)
    qd, knd, vnd, kcd, vcd, ld = to_dev(q, kn, vn, kc, vc, lens)
    o, lse = nc.decode(qd, knd, vnd, kcd, vcd, ld, return_lse=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    assert torch.isnan(o[0]).all() and torch.isnan(o[2]).all() and torch.isfinite(o[1]).all()
    assert torch.isnan(lse[0]).all() and torch.isnan(lse[2]).all()
    kca = kcd.cpu()
    assert torch.equal(kca[0], kc[0]) and torch.equal(kca[2], kc[2])
    assert torch.equal(kca[1, 5], kn[1, 0])


def test_decode_deterministic():
    q, kn, vn, kc, vc, lens = to_dev(*decode_inputs(8, 4, 4, 128, 256, 2000, 2048, seed=4, poison=False))
    for W in (-1, 1024):
        o1 = nc.decode(q, kn, vn, kc, vc, lens, window=W)
        o2 = nc.decode(q, kn, vn, kc, vc, lens, window=W)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)


# ------------------------------------------------------------------ chunked prefill

PREFILL_CASES = [
    # B, Tn, H, KV, min_len, max_len, T_max, W[, D = 128]
    (3, 1, 4, 2, 0, 100, 160, -1),
    (3, 7, 4, 2, 0, 100, 160, -1),
    (2, 64, 2, 2, 0, 200, 300, 50),
    (2, 130, 6, 2, 60, 300, 512, -1),
    (2, 200, 2, 1, 0, 0, 256, 0),
    (2, 65, 4, 4, 500, 700, 800, 128),
    (1, 257, 2, 2, 1, 1, 258, 1000),
    (3, 7, 4, 2, 0, 100, 160, -1, 64),
    (2, 130, 6, 2, 60, 300, 512, 77, 64),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[_ids(c) for c in PREFILL_CASES])
def test_prefill(case):
    B, Tn, H, KV, lo, hi, T_max, W = case[:8]
    D = case[8] if len(case) > 8 else 128
    say(f"prefill {case}")
    q, kn, vn, kc, vc, lens = prefill_inputs(B, Tn, H, KV, D, lo, hi, T_max, seed=31 + Tn)
    ro, rlse, rkc, rvc = oracle.prefill(f64(q), f64(kn), f64(vn), f64(kc), f64(vc), lens.numpy(), W)
    qd, knd, vnd, kcd, vcd, lensd = to_dev(q, kn, vn, kc, vc, lens)
    o, lse = nc.prefill(qd, knd, vnd, kcd, vcd, lensd, window=W, return_lse=True)
    torch.cuda.synchronize()
    check(o, ro, "bf16", "o")
    check_lse(lse, rlse, "bf16", "lse")
    # the chunk lands in the cache bit for bit; every other slot keeps its bits (NaN poison included)
    for b in range(B):
        s_ = int(lens[b])
        assert torch.equal(kcd[b, s_:s_ + Tn].cpu().view(torch.int16), kn[b].view(torch.int16))
        assert torch.equal(vcd[b, s_:s_ + Tn].cpu().view(torch.int16), vn[b].view(torch.int16))
        keep = torch.ones(T_max, dtype=torch.bool)
        keep[s_:s_ + Tn] = False
        assert torch.equal(kcd[b, keep].cpu().view(torch.int16), kc[b, keep].view(torch.int16))
        assert torch.equal(vcd[b, keep].cpu().view(torch.int16), vc[b, keep].view(torch.int16))


def _random_prefill_cases(n, seed=2025):
    """Seeded random chunked-prefill shapes: chunks of 1-150 tokens onto cached
    lengths anywhere in [0, T_max - Tn], group sizes 1-4, random windows."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B, Tn = int(rng.integers(1, 4)), int(rng.integers(1, 151))
        KV, G = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        T_max = int(rng.integers(Tn + 1, 700))
        hi = int(rng.integers(0, T_max - Tn + 1))
        lo = int(rng.integers(0, hi + 1))
        W = -1 if rng.random() < 0.4 else int(rng.integers(0, T_max + 51))
        cases.append((B, Tn, KV * G, KV, lo, hi, T_max, W))
    return cases


RANDOM_PREFILL_CASES = _random_prefill_cases(8)


@pytest.mark.parametrize("case", RANDOM_PREFILL_CASES, ids=[_ids(c) for c in RANDOM_PREFILL_CASES])
def test_prefill_random_shapes(case):
    test_prefill(case)


@pytest.mark.parametrize("D", [128, 64])
def test_prefill_from_empty_cache_is_the_forward(D):
    """With empty caches, prefill of a whole sequence runs the forward kernel on the
    same rows: the outputs are bitwise those of ncattn_fwd."""
    B, T, H, KV = 2, 300, 4, 2
    q, k, v, _ = to_dev(*attn_inputs(B, T, H, KV, D, "bf16", seed=41))
    for W in (-1, 77):
        o_f, lse_f = nc.fwd(q, k, v, window=(W, 0))
        kc = torch.zeros(B, T + 20, KV, D, dtype=torch.bfloat16, device=DEV)
        vc = torch.zeros_like(kc)
        lens = torch.zeros(B, dtype=torch.int32, device=DEV)
        o_p, lse_p = nc.prefill(q, k, v, kc, vc, lens, window=W, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o_p, o_f) and torch.equal(lse_p, lse_f)


def test_prefill_invalid_lengths_give_nan_and_leave_cache():
    B, Tn, H, KV, T_max = 3, 10, 2, 2, 64
    q, kn, vn, kc, vc, lens = prefill_inputs(B, Tn, H, KV, 128, 0, 20, T_max, seed=8, poison=False)
    lens = torch.tensor([5, T_max - Tn + 1, -1], dtype=torch.int32)
    qd, knd, vnd, kcd, vcd, lensd = to_dev(q, kn, vn, kc, vc, lens)
    o, lse = nc.prefill(qd, knd, vnd, kcd, vcd, lensd, window=-1, return_lse=True)
    torch.cuda.synchronize()
    ro, rlse, _, _ = oracle.prefill(f64(q[:1]), f64(kn[:1]), f64(vn[:1]), f64(kc[:1]), f64(vc[:1]), [5], -1)
    check(o[:1], ro, "bf16", "o valid row")
    assert torch.isnan(o[1:].float()).all() and torch.isnan(lse[1:]).all()
    for b in (1, 2):
        assert torch.equal(kcd[b].cpu(), kc[b]) and torch.equal(vcd[b].cpu(), vc[b])


# ------------------------------------------------------------ cache replication

def _bits_equal(a, b):
    """Bitwise equality of two CPU tensors of one dtype (NaN payloads included)."""
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


REPLICATE_CASES = [
    # N, T_src, T_max, KV, D, dtype, prompt length
    (3, 37, 64, 3, 64, "f32", 29),
    (5, 16, 16, 2, 8, "bf16", 16),         # the whole source, T_src == T_max, 32-byte rows
    (4, 20, 40, 2, 128, "bf16", 0),        # empty prompt: nothing copied
    (64, 1024, 1536, 10, 128, "bf16", 777),  # the Engine decode batch and heads
    (2, 9, 9, 1, 4, "f32", 1),             # 16-byte rows, a single prompt row
]


@pytest.mark.parametrize("N,T_src,T_max,KV,D,dtype,s", REPLICATE_CASES)
def test_cache_replicate(N, T_src, T_max, KV, D, dtype, s):
    say(f"cache_replicate N={N} T_src={T_src} T_max={T_max} KV={KV} D={D} {dtype} s={s}")
    ks, vs, kd, vd, sl = replicate_inputs(N, T_src, T_max, KV, D, s, seed=9 + N, dtype=dtype)
    ksd, vsd, kdd, vdd, sld = to_dev(ks, vs, kd, vd, sl)
    dl = torch.full((N,), 12345, dtype=torch.int32, device=DEV)
    nc.cache_replicate(ksd, vsd, sld, kdd, vdd, dl)
    torch.cuda.synchronize()
    # the oracle moves the values in their own dtype's float32 image (exact for bf16)
    rk, rv, rl = oracle.cache_replicate(ks.float().numpy(), vs.float().numpy(), s, kd.float().numpy(),
                                        vd.float().numpy())
    assert dl.cpu().tolist() == rl.tolist()
    exp_k = torch.from_numpy(rk).to(kd.dtype)
    exp_v = torch.from_numpy(rv).to(vd.dtype)
    assert _bits_equal(kdd.cpu(), exp_k) and _bits_equal(vdd.cpu(), exp_v)
    assert _bits_equal(ksd.cpu(), ks) and _bits_equal(vsd.cpu(), vs)   # sources only read


@pytest.mark.parametrize("bad", [-1, 21, -2 ** 31])
def test_cache_replicate_invalid_length_copies_nothing(bad):
    N, T_src, T_max, KV, D = 3, 20, 32, 2, 128
    ks, vs, kd, vd, _ = replicate_inputs(N, T_src, T_max, KV, D, bad, seed=31)
    ksd, vsd, kdd, vdd = to_dev(ks, vs, kd, vd)
    sld = torch.tensor([bad], dtype=torch.int32, device=DEV)
    dl = torch.zeros(N, dtype=torch.int32, device=DEV)
    nc.cache_replicate(ksd, vsd, sld, kdd, vdd, dl)
    torch.cuda.synchronize()
    assert dl.cpu().tolist() == [-1] * N
    assert _bits_equal(kdd.cpu(), kd) and _bits_equal(vdd.cpu(), vd)


def test_cache_replicate_then_decode():
    """Prefill once, replicate, decode every sample: each row's decode matches the
    oracle decode over the replicated cache (the Engine's prefill-then-sample flow)."""
    N, T_src, T_max, H, KV, D, s = 8, 300, 512, 4, 2, 128, 250
    ks, vs, kd, vd, sl = replicate_inputs(N, T_src, T_max, KV, D, s, seed=33)
    ksd, vsd, kdd, vdd, sld = to_dev(ks, vs, kd, vd, sl)
    dl = torch.empty(N, dtype=torch.int32, device=DEV)
    nc.cache_replicate(ksd, vsd, sld, kdd, vdd, dl)
    q, kn, vn, _, _, _ = decode_inputs(N, H, KV, D, 1, 2, 4, seed=34, poison=False)
    qd, knd, vnd = to_dev(q, kn, vn)
    rk, rv, rl = oracle.cache_replicate(f64(ks), f64(vs), s, f64(kd), f64(vd))
    for W in (-1, 100):
        kc, vc = kdd.clone(), vdd.clone()
        o, lse = nc.decode(qd, knd, vnd, kc, vc, dl, window=W, return_lse=True)
        torch.cuda.synchronize()
        ro, rlse, _, _ = oracle.decode(f64(q), f64(kn), f64(vn), rk, rv, rl, W)
        check(o, ro, "bf16", f"decode after replicate W={W}")
        check_lse(lse, rlse, "bf16", f"decode lse after replicate W={W}")
