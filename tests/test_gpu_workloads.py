"""Parity at the five workload shapes, in the launch configuration the bench
times.  The tiny fp32 case is compared in full; the large cases are compared on
sampled (sequence, kv-group) slices, every row and column of each sampled slice,
which is what the oracle can afford (dense T x T per head in fp64).

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
from parity_util import check, check_lse, f64, group_slice, lse_tol_after_bf16_inputs
from workloads import D12, D20, DECODE, GQA, TINY, config_inputs, decode_inputs

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
    rdq, rdk, rdv = oracle.attn_bwd(qn, kn, f64(v), f64(do), -1)
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


def _samples(cfg):
    return [(0, 0), (cfg.B - 1, cfg.KV - 1)]


@pytest.mark.parametrize("cfg", [D12, D20, GQA], ids=lambda c: c.name)
def test_workload_layers(cfg):
    say(f"{cfg.name}: generating inputs")
    q, k, v, do = config_inputs(cfg)
    G = cfg.H // cfg.KV
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    if not cfg.pre_normed:
        nc.qknorm_rope_(qd, kd, None, rope_base=cfg.rope_base, eps=1e-6, qk_gain=1.0)
    torch.cuda.synchronize()
    for W in sorted(set(cfg.windows)):
        say(f"{cfg.name}: W={W} fwd/bwd on the GPU")
        o, lse = nc.fwd(qd, kd, vd, window=(W, 0))
        dq, dk, dv = nc.bwd(qd, kd, vd, o, lse, dod, window=(W, 0))
        torch.cuda.synchronize()
        for b, g in _samples(cfg):
            say(f"{cfg.name}: W={W} oracle on slice b={b} kv-group={g}")
            sq, sk, sv, sdo = group_slice(q, k, v, do, b, g, G)
            if cfg.pre_normed:
                xq, xk = f64(sq), f64(sk)
            else:
                xq, xk = oracle.qknorm_rope(f64(sq), f64(sk), None, cfg.rope_base, 1e-6, 1.0)
                check(qd[b:b + 1, :, g * G:(g + 1) * G], xq, "bf16", "q'")
                check(kd[b:b + 1, :, g:g + 1], xk, "bf16", "k'")
            ro, rlse = oracle.attn_fwd(xq, xk, f64(sv), W)
            rdq, rdk, rdv = oracle.attn_bwd(xq, xk, f64(sv), f64(sdo), W)
            hs = slice(g * G, (g + 1) * G)
            check(o[b:b + 1, :, hs], ro, "bf16", f"o W={W}")
            check_lse(lse[b:b + 1, hs], rlse, "bf16", f"lse W={W}",
                      tol=None if cfg.pre_normed else lse_tol_after_bf16_inputs(cfg.D))
            check(dq[b:b + 1, :, hs], rdq, "bf16", f"dq W={W}")
            check(dk[b:b + 1, :, g:g + 1], rdk, "bf16", f"dk W={W}")
            check(dv[b:b + 1, :, g:g + 1], rdv, "bf16", f"dv W={W}")
        del o, lse, dq, dk, dv


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
