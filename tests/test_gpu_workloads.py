"""Parity at the five workload shapes, in the launch configuration the bench
times.  The tiny fp32 case is compared in full; the large cases are compared on
six sampled (sequence, kv-group) slices each (the first, the last and four seeded
interior ones), every row and column of each sampled slice, which is what the
oracle can afford (dense T x T per head in fp64); every output is also checked
for non-finite values over the whole tensor.

For the d12/d20 layers the whole chain runs on both sides from the same seeded
raw inputs: QK-norm + RoPE, then forward and backward at the short (S) and
long (L) window.  The GQA case takes its inputs as already normalised.  The
decode case compares every sequence at both windows."""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_qknorm_amd as nc
from parity_util import check, check_fp8_o, check_lse, f64, group_slice, stored
from workloads import D12, D20, DECODE, GQA, HD64, TINY, config_inputs, decode_inputs, fp8_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.mark.parametrize("gain", [1.0, math.sqrt(1.2)])
def test_tiny_fp32_full_chain(gain):
    cfg = TINY
    say(f"{cfg.name} gain={gain}")
    q, k, v, do = config_inputs(cfg)
    qn, kn = oracle.qknorm_rope(f64(q), f64(k), None, cfg.rope_base, 1e-6, gain)
    ro, rlse = oracle.attn_fwd(qn, kn, f64(v), -1)
    rdq, rdk, rdv = oracle.attn_bwd(qn, kn, f64(v), f64(do), -1, o=stored(ro, "f32"))
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    nc.qknorm_rope_(qd, kd, None, rope_base=cfg.rope_base, eps=1e-6, qk_gain=gain)
    o, lse = nc.fwd(qd, kd, vd)
    dq, dk, dv = nc.bwd(qd, kd, vd, o, lse, dod)
    torch.cuda.synchronize()
    check(qd, qn, "f32", "q'")
    check(kd, kn, "f32", "k'")
    check(o, ro, "f32", "o")
    check_lse(lse, rlse, "f32", "lse")
    check(dq, rdq, "f32", "dq")
    check(dk, rdk, "f32", "dk")
    check(dv, rdv, "f32", "dv")


def _samples(cfg, n_interior=4):
    """(sequence, kv group) slices compared with the oracle: the first, the last
    and n_interior seeded interior ones (distinct)."""
    rng = np.random.default_rng(1000 + cfg.seed)
    out = [(0, 0), (cfg.B - 1, cfg.KV - 1)]
    while len(out) < 2 + n_interior:
        s = (int(rng.integers(0, cfg.B)), int(rng.integers(0, cfg.KV)))
        if s not in out:
            out.append(s)
    return out


_GPU_RESULTS = {}


def _gpu_layer(cfg, W):
    """QK-norm + RoPE (unless the inputs are taken as post-norm), forward and
    backward of the whole workload at window W on the GPU, in the launch
    configuration the bench times; cached per (workload, W).  Every output is
    checked for non-finite values over the whole tensor before it is kept."""
    key = (cfg.name, W)
    if key in _GPU_RESULTS:
        return _GPU_RESULTS[key]
    _GPU_RESULTS.clear()
    say(f"{cfg.name}: W={W} generating inputs")
    q, k, v, do = config_inputs(cfg)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    rstd = None
    if not cfg.pre_normed:
        _, _, rstd = nc.qknorm_rope_rstd_(qd, kd, None, rope_base=cfg.rope_base, eps=1e-6, qk_gain=1.0)
    say(f"{cfg.name}: W={W} fwd/bwd on the GPU")
    o, lse = nc.fwd(qd, kd, vd, window=(W, 0))
    dq, dk, dv = nc.bwd(qd, kd, vd, o, lse, dod, window=(W, 0))
    outs = [("q'", qd), ("k'", kd), ("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)]
    if rstd is not None:
        # the fused backward: gradients of the raw q, k through QK-norm + RoPE,
        # from the post-norm rows and their 1/r
        dqr, dkr, _ = nc.bwd_qknorm_rope(qd, kd, vd, o, lse, dod, rstd, None, rope_base=cfg.rope_base, qk_gain=1.0,
                                         window=(W, 0))
        outs += [("dq_raw", dqr), ("dk_raw", dkr)]
    torch.cuda.synchronize()
    for name, t in outs:
        assert bool(torch.isfinite(t).all()), f"{cfg.name} W={W}: non-finite values in {name}"
    keys = {"q'": "q", "k'": "k"}
    res = dict(inputs=(q, k, v, do), **{keys.get(n, n): t.cpu() for n, t in outs})
    del qd, kd, vd, dod, o, lse, dq, dk, dv, outs, rstd
    torch.cuda.empty_cache()
    _GPU_RESULTS[key] = res
    return res


LAYER_CASES = [(cfg, W) for cfg in (D12, D20, GQA, HD64) for W in sorted(set(cfg.windows))]


@pytest.mark.parametrize("cfg,W", LAYER_CASES, ids=[f"{c.name}-W{W}" for c, W in LAYER_CASES])
def test_workload_layers(cfg, W):
    r = _gpu_layer(cfg, W)
    q, k, v, do = r["inputs"]
    G = cfg.H // cfg.KV
    for b, g in _samples(cfg):
        say(f"{cfg.name}: W={W} oracle on slice b={b} kv-group={g}")
        sq, sk, sv, sdo = group_slice(q, k, v, do, b, g, G)
        hs = slice(g * G, (g + 1) * G)
        if cfg.pre_normed:
            xq, xk = f64(sq), f64(sk)
        else:
            xq, xk = oracle.qknorm_rope(f64(sq), f64(sk), None, cfg.rope_base, 1e-6, 1.0)
            check(r["q"][b:b + 1, :, hs], xq, "bf16", "q'")
            check(r["k"][b:b + 1, :, g:g + 1], xk, "bf16", "k'")
            # the attention reads q', k' as stored (bf16)
            xq, xk = stored(xq, "bf16"), stored(xk, "bf16")
        ro, rlse = oracle.attn_fwd(xq, xk, f64(sv), W)
        # the backward is handed the forward's output as stored (bf16)
        rdq, rdk, rdv = oracle.attn_bwd(xq, xk, f64(sv), f64(sdo), W, o=stored(ro, "bf16"))
        check(r["o"][b:b + 1, :, hs], ro, "bf16", f"o W={W} b={b} g={g}")
        check_lse(r["lse"][b:b + 1, hs], rlse, "bf16", f"lse W={W} b={b} g={g}")
        check(r["dq"][b:b + 1, :, hs], rdq, "bf16", f"dq W={W} b={b} g={g}")
        check(r["dk"][b:b + 1, :, g:g + 1], rdk, "bf16", f"dk W={W} b={b} g={g}")
        check(r["dv"][b:b + 1, :, g:g + 1], rdv, "bf16", f"dv W={W} b={b} g={g}")
        if not cfg.pre_normed:
            # the fused backward, through the norm to the raw inputs of the slice
            rdq_raw, rdk_raw = oracle.qknorm_rope_bwd(f64(sq), f64(sk), rdq, rdk, None, cfg.rope_base, 1e-6, 1.0)
            check(r["dq_raw"][b:b + 1, :, hs], rdq_raw, "bf16", f"dq_raw W={W} b={b} g={g}")
            check(r["dk_raw"][b:b + 1, :, g:g + 1], rdk_raw, "bf16", f"dk_raw W={W} b={b} g={g}")


@pytest.mark.parametrize("W", sorted(set(GQA.windows)))
def test_workload_fp8_forward(W):
    """The fp8 forward at the grouped-query layer's full size (its inputs drawn as
    the bf16 layer's and stored as e4m3 with per-tensor descales), on the six
    sampled (sequence, kv-group) slices, against the oracle's forward on the
    values the fp8 tensors stand for."""
    cfg = GQA
    say(f"{cfg.name} fp8: W={W} generating inputs")
    (q8, k8, v8), (dq, dk, dv) = fp8_inputs(cfg.B, cfg.T, cfg.H, cfg.KV, cfg.D, seed=cfg.seed)
    say(f"{cfg.name} fp8: W={W} forward on the GPU")
    o, lse = nc.fwd_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), dq, dk, dv, window=(W, 0))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    o, lse = o.cpu(), lse.cpu()
    G = cfg.H // cfg.KV
    for b, g in _samples(cfg):
        say(f"{cfg.name} fp8: W={W} oracle on slice b={b} kv-group={g}")
        hs = slice(g * G, (g + 1) * G)
        sq = q8[b:b + 1, :, hs].to(torch.float64).numpy() * dq
        sk = k8[b:b + 1, :, g:g + 1].to(torch.float64).numpy() * dk
        sv = v8[b:b + 1, :, g:g + 1].to(torch.float64).numpy() * dv
        ro, rlse = oracle.attn_fwd(sq, sk, sv, W)
        ra, _ = oracle.attn_fwd(sq, sk, np.abs(sv), W)
        check_fp8_o(o[b:b + 1, :, hs], ro, ra, sv, W, f"o W={W} b={b} g={g}")
        check_lse(lse[b:b + 1, hs], rlse, "bf16", f"lse W={W} b={b} g={g}")


@pytest.mark.parametrize("W", list(DECODE.windows))
def test_engine_decode(W):
    c = DECODE
    say(f"{c.name}: W={W}")
    q, kn, vn, kc, vc, lens = decode_inputs(c.B, c.H, c.KV, c.D, c.min_len, c.max_len, c.T_max, seed=c.seed,
                                            poison=True)
    # one oracle call per sequence on the cache prefix it can read (slots <= s)
    ro = np.empty((c.B, 1, c.H, c.D))
    rlse = np.empty((c.B, c.H))
    for b in range(c.B):
        s = int(lens[b])
        o_b, l_b, _, _ = oracle.decode(f64(q[b:b + 1]), f64(kn[b:b + 1]), f64(vn[b:b + 1]),
                                       f64(kc[b:b + 1, :s + 1]), f64(vc[b:b + 1, :s + 1]), [s], W)
        ro[b], rlse[b] = o_b[0], l_b[0]
    qd, knd, vnd, kcd, vcd, ld = (t.to(DEV) for t in (q, kn, vn, kc, vc, lens))
    o, lse = nc.decode(qd, knd, vnd, kcd, vcd, ld, window=W, return_lse=True)
    torch.cuda.synchronize()
    check(o, ro, "bf16", "o")
    check_lse(lse, rlse, "bf16", "lse")
    kca = kcd.cpu()
    idx = torch.arange(c.B)
    assert torch.equal(kca[idx, lens.long()], kn[:, 0])
