"""Pins for the CPU oracle: each check compares it with something other than
itself -- torch's float64 SDPA/autograd/rms_norm (library routines for the
textbook definitions), central finite differences, closed forms, brute-force
counts, a complex-multiplication RoPE and hand-worked golden fixtures.

The last group plants plausible mistakes in copies of oracle functions and
checks that the pins catch each one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def sdpa_ref(q, k, v, W, scale=None):
    """torch float64 SDPA with an explicit inclusive-window causal mask and GQA."""
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    T = q.shape[1]
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = j <= i
    if W >= 0:
        mask = mask & (i - j <= W)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                       enable_gqa=q.shape[2] != k.shape[2])
    return o.permute(0, 2, 1, 3).numpy()


def rand(*shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------- RMSNorm

def test_rmsnorm_matches_torch_rms_norm():
    x = rand(3, 5, 2, 64)
    got = oracle.rms_norm(x, eps=1e-6)
    ref = F.rms_norm(torch.from_numpy(x), (64,), eps=1e-6).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_rmsnorm_closed_forms():
    x = rand(4, 128)
    eps, g = 1e-6, math.sqrt(1.2)
    y = oracle.rms_norm(x, eps=eps, gain=g)
    m = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), g * np.sqrt(m / (m + eps)), rtol=1e-12)
    # constant row c * 1 -> g * sign(c) * 1 (up to eps)
    c = np.full((1, 64), -3.5)
    np.testing.assert_allclose(oracle.rms_norm(c, eps=0.0, gain=g), -g * np.ones((1, 64)), rtol=1e-14)
    # scale invariance for c > 0 (eps = 0)
    np.testing.assert_allclose(oracle.rms_norm(7.0 * x, eps=0.0), oracle.rms_norm(x, eps=0.0), rtol=1e-13)


def test_rms_rstd_against_torch_rms_norm_and_closed_forms():
    """x * rstd(x) is torch's rms_norm of x; a constant row c gives 1/sqrt(c^2 + eps)."""
    x = rand(3, 5, 2, 128)
    r = oracle.rms_rstd(x, eps=1e-6)
    assert r.shape == x.shape[:-1]
    ref = F.rms_norm(torch.from_numpy(x), (128,), eps=1e-6).numpy()
    np.testing.assert_allclose(x * r[..., None], ref, rtol=1e-13, atol=1e-13)
    c = np.full((2, 64), -3.5)
    np.testing.assert_allclose(oracle.rms_rstd(c, eps=0.25), 1.0 / math.sqrt(3.5 ** 2 + 0.25), rtol=1e-15)


# ----------------------------------------------------------------- RoPE

def test_rope_golden_hand_values():
    g = json.load(open(os.path.join(GOLDEN, "rope_hand.json")))
    for case in g["cases"]:
        x = np.array(case["x"], dtype=np.float64).reshape(1, 1, 1, 4)
        pos = np.array([[case["pos"]]], dtype=np.float64)
        got = oracle.apply_rope(x, pos, g["base"]).reshape(-1)
        np.testing.assert_allclose(got, case["expect"], rtol=0, atol=1e-14, err_msg=case["why"])


def test_rope_equals_complex_multiplication():
    # independent formulation: z_j = x_j + i x_{j+D/2}, z_j <- z_j * exp(i pos w_j)
    B, T, Hh, D, base = 2, 9, 3, 64, 100000.0
    x = rand(B, T, Hh, D)
    pos = rng.integers(0, 9000, size=(B, T)).astype(np.float64)
    w = np.array([base ** (-(2.0 * j) / D) for j in range(D // 2)])
    z = x[..., : D // 2] + 1j * x[..., D // 2:]
    z = z * np.exp(1j * pos[:, :, None, None] * w)
    ref = np.concatenate([z.real, z.imag], axis=-1)
    np.testing.assert_allclose(oracle.apply_rope(x, pos, base), ref, rtol=1e-12, atol=1e-12)


def test_rope_invariants():
    D, base = 128, 100000.0
    x = rand(1, 6, 2, D)
    pos = np.arange(6, dtype=np.float64)[None] * 1000.0
    y = oracle.apply_rope(x, pos, base)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(oracle.apply_rope(x, 0 * pos, base), x, rtol=0, atol=0)
    # R(a) R(b) = R(a + b)
    a = oracle.apply_rope(oracle.apply_rope(x, pos, base), pos + 17.0, base)
    np.testing.assert_allclose(a, oracle.apply_rope(x, 2 * pos + 17.0, base), atol=1e-10)
    # relative position: <R(q, m), R(k, n)> depends only on n - m
    qv, kv = rand(1, 1, 1, D), rand(1, 1, 1, D)
    d1 = np.sum(oracle.apply_rope(qv, np.array([[5.0]]), base) * oracle.apply_rope(kv, np.array([[12.0]]), base))
    d2 = np.sum(oracle.apply_rope(qv, np.array([[105.0]]), base) * oracle.apply_rope(kv, np.array([[112.0]]), base))
    assert abs(d1 - d2) < 1e-11


def test_qknorm_rope_commutes_and_offsets():
    q, k = rand(2, 5, 4, 64), rand(2, 5, 2, 64)
    off = np.array([0, 300])
    qn, kn = oracle.qknorm_rope(q, k, off, base=10000.0, eps=1e-6, gain=1.0)
    pos = off[:, None] + np.arange(5)[None]
    # RoPE then norm gives the same result (norm and rotation commute)
    alt = oracle.rms_norm(oracle.apply_rope(q, pos, 10000.0), 1e-6)
    np.testing.assert_allclose(qn, alt, atol=1e-13)
    np.testing.assert_allclose(kn[1, 2], oracle.apply_rope(oracle.rms_norm(k, 1e-6), pos, 10000.0)[1, 2], atol=1e-14)


# ----------------------------------------------------------------- forward

@pytest.mark.parametrize("T,H,KV,D,W", [(16, 2, 2, 8, -1), (16, 4, 2, 8, 3), (33, 6, 2, 16, 0),
                                        (33, 3, 1, 16, 7), (20, 2, 2, 8, 19), (1, 2, 1, 8, -1)])
def test_fwd_matches_torch_sdpa(T, H, KV, D, W):
    q, k, v = rand(2, T, H, D), rand(2, T, KV, D), rand(2, T, KV, D)
    o, lse = oracle.attn_fwd(q, k, v, W)
    np.testing.assert_allclose(o, sdpa_ref(q, k, v, W), rtol=1e-12, atol=1e-12)
    # LSE against torch.logsumexp of the masked scores
    G = H // KV
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    s = qt @ kt.transpose(-1, -2) / math.sqrt(D)
    i, j = torch.arange(T)[:, None], torch.arange(T)[None, :]
    vis = (j <= i) & ((i - j <= W) if W >= 0 else torch.ones_like(j <= i))
    ref_lse = torch.logsumexp(s.masked_fill(~vis, float("-inf")), dim=-1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_fwd_closed_forms():
    T, H, D = 24, 2, 16
    q, k, v = rand(1, T, H, D), rand(1, T, H, D), rand(1, T, H, D)
    # W = 0: every query sees only itself
    o, lse = oracle.attn_fwd(q, k, v, 0)
    np.testing.assert_allclose(o, v, atol=1e-14)
    np.testing.assert_allclose(lse, np.einsum("bthd,bthd->bht", q, k) / math.sqrt(D), atol=1e-13)
    # q = 0: O_i is the mean of the visible v_j and LSE_i = log(n_visible(i))
    W = 5
    o, lse = oracle.attn_fwd(np.zeros_like(q), k, v, W)
    for i in range(T):
        lo = max(0, i - W)
        np.testing.assert_allclose(o[0, i], v[0, lo:i + 1].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(lse[0, :, i], math.log(i + 1 - lo), atol=1e-13)
    # W >= T - 1 equals full causal exactly
    a, _ = oracle.attn_fwd(q, k, v, T - 1)
    b, _ = oracle.attn_fwd(q, k, v, -1)
    np.testing.assert_array_equal(a, b)
    # T = 1 => O = v
    o1, _ = oracle.attn_fwd(q[:, :1], k[:, :1], v[:, :1], -1)
    np.testing.assert_allclose(o1, v[:, :1], atol=1e-15)


def test_fwd_gqa_equals_mha_on_repeated_kv():
    q, k, v = rand(2, 12, 6, 8), rand(2, 12, 2, 8), rand(2, 12, 2, 8)
    a, la = oracle.attn_fwd(q, k, v, 4)
    b, lb = oracle.attn_fwd(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), 4)
    np.testing.assert_allclose(a, b, atol=1e-14)
    np.testing.assert_allclose(la, lb, atol=1e-14)


def test_pair_count_brute_force():
    for T in (1, 2, 7, 64, 130):
        for W in (-1, 0, 1, 5, 63, 129, 500):
            brute = sum(1 for i in range(T) for j in range(T) if j <= i and (W < 0 or i - j <= W))
            assert oracle.n_visible_pairs(T, W) == brute == int(oracle.visible_mask(T, W).sum())
    assert oracle.n_visible_pairs(2048, -1) == 2048 * 2049 // 2
    # closed form for W < T: W+1 keys for the T-W rows past the ramp, 1..W for the ramp
    assert oracle.n_visible_pairs(2048, 1024) == (2048 - 1024) * 1025 + 1024 * 1025 // 2
    fwd, bwd = oracle.attn_flops(8, 2048, 6, 128, 1024)
    assert (fwd, bwd) == (4 * 128 * 1574400 * 48, 8 * 128 * 1574400 * 48)


def _counted_attention(q, k, v, do, W):
    """Scalar-loop attention forward and backward that counts every multiply and
    every add of the four contractions it performs (QK^T, PV; dV, dP, dQ, dK),
    two per multiply-accumulate.  Softmax arithmetic is not counted (the MFU
    convention counts matmul work only).  Returns (o, dq, dk, dv, fwd_flops,
    bwd_flops); o and the gradients are checked against the oracle so that the
    count belongs to a real computation of the same function."""
    B, T, H, D = q.shape
    KV = k.shape[2]
    G = H // KV
    scale = 1.0 / math.sqrt(D)
    o = np.zeros_like(q)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    ff = fb = 0
    for b in range(B):
        for h in range(H):
            g = h // G
            for i in range(T):
                keys = [j for j in range(i + 1) if W < 0 or i - j <= W]
                s = {}
                for j in keys:
                    acc = 0.0
                    for d in range(D):
                        acc += q[b, i, h, d] * k[b, j, g, d]
                        ff += 2
                    s[j] = acc * scale
                m = max(s.values())
                z = sum(math.exp(x - m) for x in s.values())
                p = {j: math.exp(s[j] - m) / z for j in keys}
                for j in keys:
                    for d in range(D):
                        o[b, i, h, d] += p[j] * v[b, j, g, d]
                        ff += 2
                dp = {}
                for j in keys:
                    acc = 0.0
                    for d in range(D):
                        dv[b, j, g, d] += p[j] * do[b, i, h, d]
                        acc += do[b, i, h, d] * v[b, j, g, d]
                        fb += 4
                    dp[j] = acc
                delta = sum(p[j] * dp[j] for j in keys)
                for j in keys:
                    ds = p[j] * (dp[j] - delta)
                    for d in range(D):
                        dq[b, i, h, d] += ds * k[b, j, g, d] * scale
                        dk[b, j, g, d] += ds * q[b, i, h, d] * scale
                        fb += 4
    return o, dq, dk, dv, ff, fb


@pytest.mark.parametrize("B,T,H,KV,D,W", [(1, 7, 2, 2, 4, -1), (2, 9, 4, 2, 3, 2), (1, 6, 3, 1, 5, 0),
                                          (1, 8, 2, 1, 2, 20)])
def test_attn_flops_loop_counted(B, T, H, KV, D, W):
    q, k, v, do = rand(B, T, H, D), rand(B, T, KV, D), rand(B, T, KV, D), rand(B, T, H, D)
    o, dq, dk, dv, ff, fb = _counted_attention(q, k, v, do, W)
    ro, _ = oracle.attn_fwd(q, k, v, W)
    rdq, rdk, rdv = oracle.attn_bwd(q, k, v, do, W)
    for a, r in ((o, ro), (dq, rdq), (dk, rdk), (dv, rdv)):
        np.testing.assert_allclose(a, r, atol=1e-12)
    assert oracle.attn_flops(B, T, H, D, W) == (ff, fb)


def _decode_bytes_brute(lens, H, KV, D, W, eb):
    """Walks each sequence's cache slots and adds the bytes decode must move for
    every visible key: a cached key's K and V rows are read from the cache; the
    new key (slot s) comes from k_new/v_new and is written into the cache; q is
    read and o written once per sequence."""
    row, qrow = KV * D * eb, H * D * eb
    total = 0
    for s in lens:
        total += 2 * qrow
        for j in range(s + 1):
            if W >= 0 and s - j > W:
                continue
            total += 2 * row if j < s else 4 * row
    return total


def test_decode_bytes_brute_force_and_golden():
    # hand-worked: lengths 3, 0, 10 at window 2, H=2, KV=1, D=4, bf16: visible
    # cached rows 2 + 0 + 2 (64 B of K and V), new keys 3 x (16 B read + 16 B
    # written), q and o 3 x 32 B
    assert oracle.decode_bytes([3, 0, 10], 2, 1, 4, 2, 2) == 64 + 96 + 96 == 256
    r = np.random.default_rng(7)
    for _ in range(40):
        B = int(r.integers(1, 6))
        lens = [int(x) for x in r.integers(0, 300, size=B)]
        H, KV, D = 2 * int(r.integers(1, 4)), 2, int(r.choice([4, 8, 128]))
        W = int(r.choice([-1, 0, 1, 17, 128, 299, 1000]))
        eb = int(r.choice([2, 4]))
        assert oracle.decode_bytes(lens, H, KV, D, W, eb) == _decode_bytes_brute(lens, H, KV, D, W, eb)


def test_window_schedule_golden():
    g = json.load(open(os.path.join(GOLDEN, "window_schedule.json")))
    for c in g["cases"]:
        got = oracle.window_sizes(c["pattern"], c["n_layer"], c["short"])
        assert [list(t) for t in got] == c["expect"], c


# ----------------------------------------------------------------- backward

def _loss(q, k, v, do, W):
    return float(np.sum(oracle.attn_fwd(q, k, v, W)[0] * do))


@pytest.mark.parametrize("H,KV,W", [(2, 2, -1), (4, 2, 3), (3, 1, 0)])
def test_bwd_matches_finite_differences(H, KV, W):
    T, D, h = 7, 4, 1e-6
    q, k, v, do = rand(1, T, H, D), rand(1, T, KV, D), rand(1, T, KV, D), rand(1, T, H, D)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, W)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, W)
            x[idx] = old - h
            lm = _loss(q, k, v, do, W)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, atol=2e-8, rtol=1e-6)


@pytest.mark.parametrize("T,H,KV,D,W", [(40, 4, 2, 16, -1), (40, 6, 2, 16, 9), (17, 2, 2, 8, 0)])
def test_bwd_matches_torch_autograd(T, H, KV, D, W):
    q, k, v, do = rand(2, T, H, D), rand(2, T, KV, D), rand(2, T, KV, D), rand(2, T, H, D)
    qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    i, j = torch.arange(T)[:, None], torch.arange(T)[None, :]
    mask = (j <= i) & ((i - j <= W) if W >= 0 else torch.ones(T, T, dtype=torch.bool))
    o = F.scaled_dot_product_attention(qt.permute(0, 2, 1, 3), kt.permute(0, 2, 1, 3), vt.permute(0, 2, 1, 3),
                                       attn_mask=mask, enable_gqa=H != KV).permute(0, 2, 1, 3)
    (o * torch.from_numpy(do)).sum().backward()
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, W)
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-11)


def test_bwd_invariants_and_closed_forms():
    T, H, KV, D = 30, 4, 2, 8
    q, k, v, do = rand(1, T, H, D), rand(1, T, KV, D), rand(1, T, KV, D), rand(1, T, H, D)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 6)
    # shifting every key by a constant vector leaves O unchanged: sum_j dK_j = 0
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-12)
    # rows of P sum to one: sum_j dV_j = sum over the group's heads of sum_i dO_i
    np.testing.assert_allclose(dv.sum(axis=1), do.reshape(1, T, KV, 2, D).sum(axis=(1, 3)), atol=1e-12)
    # W = 0: dQ = dK = 0 and dV_i = sum over the group of dO_i
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, 0)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv, do.reshape(1, T, KV, 2, D).sum(axis=3), atol=1e-14)


# ----------------------------------------------------------------- decode

@pytest.mark.parametrize("W", [-1, 0, 3, 50])
def test_decode_equals_sdpa_last_row(W):
    B, H, KV, D, Tm = 3, 4, 2, 16, 40
    lens = np.array([0, 17, 38])
    q, kn, vn = rand(B, 1, H, D), rand(B, 1, KV, D), rand(B, 1, KV, D)
    kc, vc = rand(B, Tm, KV, D), rand(B, Tm, KV, D)
    for b in range(B):
        kc[b, lens[b]:] = np.nan
        vc[b, lens[b]:] = np.nan
    o, lse, kc2, vc2 = oracle.decode(q, kn, vn, kc, vc, lens, W)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    for b in range(B):
        s = lens[b]
        # slot s written, everything else untouched (bitwise)
        np.testing.assert_array_equal(kc2[b, s], kn[b, 0])
        np.testing.assert_array_equal(vc2[b, s], vn[b, 0])
        keep = np.ones(Tm, bool)
        keep[s] = False
        np.testing.assert_array_equal(np.isnan(kc2[b, keep]), np.isnan(kc[b, keep]))
        np.testing.assert_array_equal(np.nan_to_num(kc2[b, keep]), np.nan_to_num(kc[b, keep]))
        # the decode row equals the last row of torch SDPA over the full prefix
        kf = np.concatenate([kc[b, :s], kn[b]], axis=0)[None]
        vf = np.concatenate([vc[b, :s], vn[b]], axis=0)[None]
        qf = np.zeros((1, s + 1, H, D))
        qf[0, s] = q[b, 0]
        ref = sdpa_ref(qf, kf, vf, W)[0, s]
        np.testing.assert_allclose(o[b, 0], ref, atol=1e-12)
    if W == 0:
        np.testing.assert_allclose(o[:, 0], np.repeat(vn[:, 0], H // KV, axis=1), atol=1e-15)


# ----------------------------------------------------------------- QK-norm + RoPE backward

def _qkr_loss(q, k, dyq, dyk, off, base, eps, gain):
    yq, yk = oracle.qknorm_rope(q, k, off, base, eps, gain)
    return float(np.sum(yq * dyq) + np.sum(yk * dyk))


def _fd_grad(x, loss, h=1e-6):
    num = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        old = x[idx]
        x[idx] = old + h
        lp = loss()
        x[idx] = old - h
        lm = loss()
        x[idx] = old
        num[idx] = (lp - lm) / (2 * h)
    return num


@pytest.mark.parametrize("D,gain,eps", [(8, 1.0, 1e-6), (16, math.sqrt(1.2), 1e-2)])
def test_qknorm_rope_bwd_matches_finite_differences(D, gain, eps):
    """Central differences of the forward (not the backward's formulas) pin the gradient."""
    B, T, H, KV, base = 2, 3, 2, 1, 10000.0
    q, k = rand(B, T, H, D), rand(B, T, KV, D)
    dyq, dyk = rand(B, T, H, D), rand(B, T, KV, D)
    off = np.array([5, 1000])
    gq, gk = oracle.qknorm_rope_bwd(q, k, dyq, dyk, off, base, eps, gain)
    loss = lambda: _qkr_loss(q, k, dyq, dyk, off, base, eps, gain)  # noqa: E731
    np.testing.assert_allclose(gq, _fd_grad(q, loss), atol=1e-8, rtol=1e-6)
    np.testing.assert_allclose(gk, _fd_grad(k, loss), atol=1e-8, rtol=1e-6)


def test_qknorm_rope_bwd_matches_torch_autograd():
    """torch autograd through torch's rms_norm and a complex-multiplication RoPE."""
    B, T, H, D, base, eps, gain = 2, 5, 3, 16, 100000.0, 1e-6, 1.3
    x, dy = rand(B, T, H, D), rand(B, T, H, D)
    off = np.array([0, 77])
    xt = torch.from_numpy(x.copy()).requires_grad_(True)
    n = gain * F.rms_norm(xt, (D,), eps=eps)
    pos = torch.from_numpy(off[:, None] + np.arange(T)[None, :]).double()
    j = torch.arange(D // 2, dtype=torch.float64)
    ang = pos[..., None, None] * base ** (-2.0 * j / D)
    z = torch.complex(n[..., : D // 2], n[..., D // 2:]) * torch.exp(1j * ang)
    y = torch.cat([z.real, z.imag], dim=-1)
    (y * torch.from_numpy(dy)).sum().backward()
    gq, _ = oracle.qknorm_rope_bwd(x, x[:, :, :1], dy, dy[:, :, :1], off, base, eps, gain)
    np.testing.assert_allclose(gq, xt.grad.numpy(), atol=1e-12, rtol=1e-10)


def test_qknorm_rope_bwd_invariants():
    B, T, H, D = 1, 4, 2, 32
    x, dy = rand(B, T, H, D), rand(B, T, H, D)
    pos = np.arange(T, dtype=np.float64)[None, :] + 3.0
    # RoPE's backward undoes its rotation
    np.testing.assert_allclose(oracle.rope_inverse(oracle.apply_rope(x, pos, 10000.0), pos, 10000.0), x,
                               atol=1e-13)
    # with eps = 0 the norm is invariant to scaling x, so the gradient is orthogonal to x
    g = oracle.rms_norm_bwd(x, dy, eps=0.0, gain=1.0)
    np.testing.assert_allclose(np.sum(g * x, axis=-1), 0.0, atol=1e-12)
    # and scaling x by c scales the gradient by 1/c
    np.testing.assert_allclose(oracle.rms_norm_bwd(3.0 * x, dy, eps=0.0), g / 3.0, atol=1e-13)


def test_qknorm_rope_bwd_planted_mistakes():
    """A backward rotating by +theta, or one without the norm's projection term,
    fails the finite-difference pin."""
    import oracle.attention as A
    B, T, H, D, base, eps = 1, 3, 1, 8, 10000.0, 1e-6
    x, dy = rand(B, T, H, D), rand(B, T, H, D)
    off = np.array([40])
    pos = off[:, None] + np.arange(T, dtype=np.float64)[None, :]
    num = _fd_grad(x, lambda: _qkr_loss(x, x[:, :, :1] * 0 + 1, dy, dy[:, :, :1] * 0, off, base, eps, 1.0))
    good = A.rms_norm_bwd(x, A.rope_inverse(dy, pos, base), eps)
    np.testing.assert_allclose(good, num, atol=1e-8, rtol=1e-6)
    wrong_sign = A.rms_norm_bwd(x, A.apply_rope(dy, pos, base), eps)
    assert not np.allclose(wrong_sign, num, atol=1e-6)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    no_projection = A.rope_inverse(dy, pos, base) / r
    assert not np.allclose(no_projection, num, atol=1e-6)


# ----------------------------------------------------------------- chunked prefill

@pytest.mark.parametrize("W", [-1, 0, 3, 9])
def test_prefill_equals_rows_of_full_forward(W):
    """Prefill of a chunk after s cached tokens = rows s.. of the forward over the
    whole sequence (the forward itself pinned to torch SDPA above)."""
    B, H, KV, D, Tn, T_max = 3, 4, 2, 8, 5, 24
    lens = [0, 7, 19]
    full_q, full_k, full_v = rand(B, T_max, H, D), rand(B, T_max, KV, D), rand(B, T_max, KV, D)
    q = np.stack([full_q[b, lens[b]:lens[b] + Tn] for b in range(B)])
    kn = np.stack([full_k[b, lens[b]:lens[b] + Tn] for b in range(B)])
    vn = np.stack([full_v[b, lens[b]:lens[b] + Tn] for b in range(B)])
    kc = np.full((B, T_max, KV, D), np.nan)
    vc = np.full((B, T_max, KV, D), np.nan)
    for b in range(B):
        kc[b, :lens[b]] = full_k[b, :lens[b]]
        vc[b, :lens[b]] = full_v[b, :lens[b]]
    o, lse, kc2, vc2 = oracle.prefill(q, kn, vn, kc, vc, np.array(lens), W)
    for b in range(B):
        T = lens[b] + Tn
        ref = sdpa_ref(full_q[b:b + 1, :T], full_k[b:b + 1, :T], full_v[b:b + 1, :T], W)[0, lens[b]:]
        np.testing.assert_allclose(o[b], ref, atol=1e-12)
        _, rl = oracle.attn_fwd(full_q[b:b + 1, :T], full_k[b:b + 1, :T], full_v[b:b + 1, :T], W)
        np.testing.assert_allclose(lse[b], rl[0][:, lens[b]:], atol=1e-12)
        np.testing.assert_array_equal(kc2[b, lens[b]:lens[b] + Tn], kn[b])
        assert np.all(np.isnan(kc2[b, lens[b] + Tn:]))


def test_prefill_of_one_token_is_decode():
    B, H, KV, D, T_max = 2, 4, 1, 8, 12
    q, kn, vn = rand(B, 1, H, D), rand(B, 1, KV, D), rand(B, 1, KV, D)
    kc, vc = rand(B, T_max, KV, D), rand(B, T_max, KV, D)
    lens = np.array([3, 11])
    for W in (-1, 2):
        o1, l1, k1, v1 = oracle.prefill(q, kn, vn, kc, vc, lens, W)
        o2, l2, k2, v2 = oracle.decode(q, kn, vn, kc, vc, lens, W)
        np.testing.assert_allclose(o1, o2, atol=1e-14)
        np.testing.assert_allclose(l1[:, :, 0], l2, atol=1e-14)
        np.testing.assert_array_equal(k1, k2)


def test_cache_replicate_then_decode_equals_decode_on_the_prefilled_cache():
    """Decoding from every replicated row reproduces decoding from the batch-1
    cache it was copied from (the point of prefilling once and cloning), and the
    rows past the prompt keep their old contents."""
    KV, D, T_src, T_max, N, H = 2, 8, 9, 14, 3, 4
    s = 6
    k_src, v_src = rand(1, T_src, KV, D), rand(1, T_src, KV, D)
    k_dst = np.full((N, T_max, KV, D), 7.25)
    v_dst = np.full((N, T_max, KV, D), -3.5)
    kd, vd, lens = oracle.cache_replicate(k_src, v_src, s, k_dst, v_dst)
    assert lens.dtype == np.int32 and list(lens) == [s] * N
    assert np.all(kd[:, s:] == 7.25) and np.all(vd[:, s:] == -3.5)
    # a batch-1 decode cache of the source's own size holds the prompt rows at [0, s)
    for n in range(N):
        q, kn, vn = rand(1, 1, H, D), rand(1, 1, KV, D), rand(1, 1, KV, D)
        for W in (-1, 3):
            o_rep, lse_rep, _, _ = oracle.decode(q, kn, vn, kd[n:n + 1], vd[n:n + 1], [s], W)
            o_src, lse_src, _, _ = oracle.decode(q, kn, vn, k_src, v_src, [s], W)
            assert np.array_equal(o_rep, o_src) and np.array_equal(lse_rep, lse_src)


def test_cache_replicate_lengths_at_the_edges():
    KV, D, T_src, T_max, N = 1, 4, 5, 8, 2
    k_src, v_src = rand(1, T_src, KV, D), rand(1, T_src, KV, D)
    k_dst, v_dst = rand(N, T_max, KV, D), rand(N, T_max, KV, D)
    kd, vd, lens = oracle.cache_replicate(k_src, v_src, 0, k_dst, v_dst)   # empty prompt: nothing copied
    assert list(lens) == [0, 0] and np.array_equal(kd, k_dst) and np.array_equal(vd, v_dst)
    kd, vd, lens = oracle.cache_replicate(k_src, v_src, T_src, k_dst, v_dst)   # whole source
    assert list(lens) == [T_src] * N
    assert all(np.array_equal(kd[n, :T_src], k_src[0]) for n in range(N))
    assert np.array_equal(kd[:, T_src:], k_dst[:, T_src:])
    for bad in (-1, T_src + 1):   # invalid source length: untouched, lengths -1
        kd, vd, lens = oracle.cache_replicate(k_src, v_src, bad, k_dst, v_dst)
        assert list(lens) == [-1, -1] and np.array_equal(kd, k_dst) and np.array_equal(vd, v_dst)


# ----------------------------------------------------------------- planted mistakes

def test_planted_mistakes_are_caught(monkeypatch):
    """Each mutant of the oracle must fail at least one pin above."""
    import oracle.attention as A

    T, H, KV, D = 9, 4, 2, 8
    q, k, v, do = rand(1, T, H, D), rand(1, T, KV, D), rand(1, T, KV, D), rand(1, T, H, D)

    def fwd_pin(f):
        o, _ = f(q, k, v, 3)
        return np.allclose(o, sdpa_ref(q, k, v, 3), atol=1e-10)

    # 1. exclusive window (i - j < W) instead of inclusive
    def mask_exclusive(T_, W):
        i, j = np.arange(T_)[:, None], np.arange(T_)[None, :]
        return (j <= i) & ((i - j < W) if W >= 0 else True)
    monkeypatch.setattr(A, "visible_mask", mask_exclusive)
    assert not fwd_pin(A.attn_fwd)
    monkeypatch.undo()

    # 2. wrong GQA mapping (kv head h % KV instead of h // G)
    def fwd_bad_gqa(q_, k_, v_, W):
        kk = np.stack([k_[:, :, h % KV] for h in range(H)], axis=2)
        vv = np.stack([v_[:, :, h % KV] for h in range(H)], axis=2)
        return A.attn_fwd(q_, kk, vv, W)
    assert not fwd_pin(fwd_bad_gqa)

    # 3. backward with the softmax-Jacobian term dropped: finite differences catch it
    def bwd_dropped(q_, k_, v_, do_, W):
        Bq, Tq, Hq, Dq = q_.shape
        scale = 1 / np.sqrt(Dq)
        vis = A.visible_mask(Tq, W)
        dq = np.zeros_like(q_)
        for h in range(Hq):
            kh = h // (Hq // k_.shape[2])
            s = np.where(vis, scale * q_[0, :, h] @ k_[0, :, kh].T, -np.inf)
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            dp = do_[0, :, h] @ v_[0, :, kh].T
            dq[0, :, h] = scale * (p * dp) @ k_[0, :, kh]
        return dq
    dq_ref = oracle.attn_bwd(q, k, v, do, 3)[0]
    assert not np.allclose(bwd_dropped(q, k, v, do, 3), dq_ref, atol=1e-6)

    # 4. RoPE rotating by -theta fails the hand-worked golden values
    g = json.load(open(os.path.join(GOLDEN, "rope_hand.json")))
    c = g["cases"][1]
    x = np.array(c["x"]).reshape(1, 1, 1, 4)
    bad = A.apply_rope(x, np.array([[-float(c["pos"])]]), g["base"]).reshape(-1)
    assert not np.allclose(bad, c["expect"], atol=1e-12)

    # 5. interleaved RoPE pairing fails the complex-multiplication pin
    def rope_interleaved(x_, pos, base):
        Dd = x_.shape[-1]
        th = A.rope_angles(pos, Dd, base)[:, :, None, :]
        a, b = x_[..., 0::2], x_[..., 1::2]
        out = np.empty_like(x_)
        out[..., 0::2] = a * np.cos(th) - b * np.sin(th)
        out[..., 1::2] = a * np.sin(th) + b * np.cos(th)
        return out
    xx = rand(1, 3, 1, 8)
    pos = np.array([[1.0, 2.0, 3.0]])
    w = np.array([10000.0 ** (-(2.0 * j) / 8) for j in range(4)])
    z = (xx[..., :4] + 1j * xx[..., 4:]) * np.exp(1j * pos[:, :, None, None] * w)
    ref = np.concatenate([z.real, z.imag], axis=-1)
    assert np.allclose(A.apply_rope(xx, pos, 10000.0), ref, atol=1e-12)
    assert not np.allclose(rope_interleaved(xx, pos, 10000.0), ref, atol=1e-6)

    # 6. decode byte count with the window taken as exclusive fails the brute force
    def decode_bytes_exclusive(lens, H_, KV_, D_, W, eb=2):
        row = KV_ * D_ * eb
        n = sum(s - (0 if W < 0 else max(0, s - W + 1)) for s in lens)
        return n * 2 * row + len(lens) * 4 * row + len(lens) * 2 * H_ * D_ * eb
    assert decode_bytes_exclusive([3, 0, 10], 2, 1, 4, 2) != _decode_bytes_brute([3, 0, 10], 2, 1, 4, 2, 2)

    # 7. FLOPs counted over the dense T x T square (no window) fail the loop count
    qq, kk, vv, dd = rand(1, 6, 2, 3), rand(1, 6, 1, 3), rand(1, 6, 1, 3), rand(1, 6, 2, 3)
    counted = _counted_attention(qq, kk, vv, dd, 1)[4:]
    assert (4 * 3 * 36 * 2, 8 * 3 * 36 * 2) != counted == oracle.attn_flops(1, 6, 2, 3, 1)


# ----------------------------------------------------------------- backward given the forward's output

@pytest.mark.parametrize("W", [-1, 3])
def test_bwd_given_output_closed_forms(W):
    """attn_bwd(..., o=O): with the exact O it is the exact gradient; dV never
    depends on o; and replacing O by O + E moves each row's Delta by
    sum_d dO E, which moves dQ_i by -scale (Delta'_i - Delta_i) sum_j P_ij k_j
    and dK_j by -scale sum_i P_ij (Delta'_i - Delta_i) q_i (closed forms of the
    Jacobian term, computed here from torch's SDPA probabilities)."""
    B, T, H, KV, D = 1, 11, 4, 2, 8
    q, k, v, do = rand(B, T, H, D), rand(B, T, KV, D), rand(B, T, KV, D), rand(B, T, H, D)
    o, _ = oracle.attn_fwd(q, k, v, W)
    exact = oracle.attn_bwd(q, k, v, do, W)
    given = oracle.attn_bwd(q, k, v, do, W, o=o)
    for a, b in zip(exact, given):
        np.testing.assert_allclose(a, b, atol=1e-12)
    E = 1e-3 * rand(B, T, H, D)
    dq2, dk2, dv2 = oracle.attn_bwd(q, k, v, do, W, o=o + E)
    np.testing.assert_allclose(dv2, exact[2], atol=1e-13)
    scale = 1 / math.sqrt(D)
    i = torch.arange(T)[:, None]
    j = torch.arange(T)[None, :]
    mask = (j <= i) & ((i - j <= W) if W >= 0 else torch.ones(T, T, dtype=torch.bool))
    G = H // KV
    want_dq = exact[0].copy()
    want_dk = exact[1].copy()
    for h in range(H):
        kh = h // G
        s = torch.from_numpy(scale * q[0, :, h] @ k[0, :, kh].T).masked_fill(~mask, float("-inf"))
        p = torch.softmax(s, dim=-1).numpy()
        dd = (do[0, :, h] * E[0, :, h]).sum(-1)                  # Delta' - Delta per row
        want_dq[0, :, h] -= scale * dd[:, None] * (p @ k[0, :, kh])
        want_dk[0, :, kh] -= scale * (p * dd[:, None]).T @ q[0, :, h]
    np.testing.assert_allclose(dq2, want_dq, atol=1e-12)
    np.testing.assert_allclose(dk2, want_dk, atol=1e-12)
