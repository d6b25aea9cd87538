"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gqa|d12|d20] [--no-cpu-baseline]

One step = the training-side hot path of one attention workload over its four
SSSL layers, per layer the attention forward and backward (plus QK-norm + RoPE
of q and k first, for the workloads whose recipe starts from raw q, k).  The
default workload, the largest of the five, is the grouped-query layer (B=16,
T=4096, n_head=12, n_kv_head=4, head_dim=128, bf16, windows 2048, 2048, 2048,
full causal; q, k, v taken as already normalised and rotated).  Inputs are
seeded synthetic N(0, 1) tensors already resident in HBM, one distinct set per
layer.  The d12 and d20 layers are timed per layer type under "configs"; the
engine decode (64 sequences, cache lengths U[256, 8192], 10 heads, head_dim 128)
at the full-causal and 1024 windows under "decode".

Prints ONE JSON line.  ``value`` = unmasked attention FLOPs of a step (fwd 4*D
and bwd 8*D per visible (query, key) pair and head) / wall time of the step.
``roofline`` is for the kernel with the largest share of the step, timed with
HIP events on the stream it runs on inside the timed region (step s brackets that
kernel of layer s mod 4; the per-kernel figures under "detail" come from an
untimed pass with events around every kernel, since each event is a GPU packet
of its own between kernels); ``traffic`` comes from the committed rocprofv3
counter summary in profiles/ when it was taken on the current kernel source for
this workload, else null.  ``cpu_baseline`` times the CPU oracle on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA (twice the bf16 rate)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "attn fwd+bwd TFLOP/s (unmasked FLOPs) & % bf16 MFMA peak; decode GB/s"


def visible_pairs(T, W):
    """Visible (query, key) pairs of one head: sum_i min(i + 1, W + 1)."""
    if W < 0 or W >= T - 1:
        return T * (T + 1) // 2
    return (W + 1) * (W + 2) // 2 + (T - W - 1) * (W + 1)


def decode_algorithmic_bytes(lens, H, KV, D, W, elem_bytes=2):
    """Bytes one decode call must move: the visible cached K and V rows of every
    sequence (the newest key comes from k_new/v_new), k_new and v_new read and
    written into the cache, q read and o written."""
    row = KV * D * elem_bytes
    n_cached = sum(s - (0 if W < 0 else max(0, s - W)) for s in lens)
    return n_cached * 2 * row + len(lens) * 4 * row + len(lens) * 2 * H * D * elem_bytes


def kernel_source_hash(name):
    p = os.path.join(ROOT, "transformer_attention_qknorm_amd", "csrc", name)
    h = hashlib.sha256()
    for f in sorted([p, os.path.join(os.path.dirname(p), "attn_tiles.hpp"),
                     os.path.join(os.path.dirname(p), "device_common.hpp")]):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {"fwd": "attn_fwd_bf16.hip", "bwd_dkdv": "attn_bwd_bf16.hip", "bwd_dq": "attn_bwd_bf16.hip",
                  "bwd_delta": "attn_bwd_bf16.hip", "qknorm_rope": "qknorm_rope.hip",
                  "decode_split": "attn_decode.hip", "decode_combine": "attn_decode.hip"}


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed counter
    summary (profiles/traffic.json), if it was taken on the kernel's current
    source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d["workloads"][workload]["kernels"][kernel]
        if e.get("source_hash") != kernel_source_hash(KERNEL_SOURCES[kernel]):
            return None
        return e["bytes_per_launch"]
    except (KeyError, ValueError, TypeError):
        return None


def cpu_baseline(cfg, budget_s=12.0):
    """Time the CPU oracle (fwd + bwd of one (b, head) slice at a time, the short
    and the long window alternately) on the same seeded inputs until ~budget_s
    has passed."""
    import numpy as np
    import oracle
    from workloads import config_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    q, k, v, do = config_inputs(cfg)
    G = cfg.H // cfg.KV
    f = lambda t: t.double().numpy()
    flops, t_used, slices = 0, 0.0, []
    i = 0
    while t_used < budget_s and i < 8 * cfg.B * cfg.H:
        W = cfg.windows[0] if i % 2 == 0 else -1
        b, h = (i // 2) % cfg.B, (i // 2) % cfg.H
        g = h // G
        sq, sk, sv, sdo = (f(x[b:b + 1, :, j:j + 1]) for x, j in ((q, h), (k, g), (v, g), (do, h)))
        t0 = time.perf_counter()
        oracle.attn_fwd(sq, sk, sv, W)
        oracle.attn_bwd(sq, sk, sv, sdo, W)
        t_used += time.perf_counter() - t0
        flops += 12 * cfg.D * visible_pairs(cfg.T, W)
        slices.append((b, h, W))
        i += 1
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(slices)} (b, head) slices of the {cfg.name} workload (T={cfg.T}, D={cfg.D}; "
                      f"{len(set(slices))} distinct (b, head, window)), alternating window {cfg.windows[0]} and "
                      f"full causal, fwd+bwd in float64 numpy; {t_used:.1f} s of CPU work"}


class ClockSampler:
    """Samples the GPU's current graphics clock (MHz) through amdsmi on a
    background thread, every `period` seconds, while a `with` block runs (the
    mean of the per-XCD clocks of the GPU metrics table where the amdgpu driver
    reports them, else the graphics clock).  amdgpu refreshes that table about once a
    second, so a block must run well over a second to show the clock under load.
    When no sample could be taken, summary() says why."""

    def __init__(self, period=0.02):
        import threading
        self.period, self.samples, self.error = period, [], None
        self._stop = threading.Event()
        self._thread = None
        self._read = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if len(handles) != 1:
                raise RuntimeError(f"{len(handles)} GPUs visible to amdsmi, expected one")
            h = handles[0]

            def read():
                try:
                    m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                    xs = [x for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float)) and x > 0]
                    if xs:
                        return sum(xs) / len(xs)
                except Exception:  # pragma: no cover - depends on the amdgpu version
                    pass
                return float(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.SYS)["clk"])
            read()
            self._read = read
        except Exception as e:  # pragma: no cover - depends on the machine
            self.error = f"{type(e).__name__}: {e}"

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception as e:  # pragma: no cover
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        if self._read is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        return False

    def summary(self, skip_s=1.0):
        """Median, min and max of the samples after the first `skip_s` seconds."""
        xs = sorted(self.samples[int(skip_s / self.period):])
        if not xs:
            return {"error": self.error or "no samples"}
        return {"median_mhz": round(xs[len(xs) // 2]), "min_mhz": round(xs[0]), "max_mhz": round(xs[-1]),
                "samples": len(xs)}


def event_us(torch, stream, fn, iters, warm=3):
    """Average microseconds per call of fn over `iters` calls bracketed by HIP events."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / iters


def time_config(nc, torch, cfg, dev, stream, iters=10):
    """Forward and backward of each layer type (short window, full causal) of a
    workload, timed with HIP events over `iters` calls each: the per-layer-type
    TFLOP/s and the SSSL-weighted total.  Reported under "configs"; not part of
    the step above."""
    from workloads import config_inputs
    q, k, v, do = (x.to(dev) for x in config_inputs(cfg))
    o = torch.empty_like(q)
    lse = torch.empty(cfg.B, cfg.H, cfg.T, dtype=torch.float32, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    layers = {}
    for W in sorted(set(cfg.windows), reverse=True):
        ws = nc.bwd_workspace(q, k, (W, 0))
        for _ in range(2):
            nc.fwd(q, k, v, window=(W, 0), out=(o, lse))
            nc.bwd(q, k, v, o, lse, do, window=(W, 0), out=grads, workspace=ws)
        torch.cuda.synchronize()
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(iters)]
        for a, b, c in evs:
            a.record(stream)
            nc.fwd(q, k, v, window=(W, 0), out=(o, lse))
            b.record(stream)
            nc.bwd(q, k, v, o, lse, do, window=(W, 0), out=grads, workspace=ws)
            c.record(stream)
        torch.cuda.synchronize()
        tf = sum(a.elapsed_time(b) for a, b, _ in evs) / iters * 1e-3
        tb = sum(b.elapsed_time(c) for _, b, c in evs) / iters * 1e-3
        pairs = visible_pairs(cfg.T, W) * cfg.B * cfg.H
        ff, fb = 4 * cfg.D * pairs, 8 * cfg.D * pairs
        layers["L" if W < 0 else "S"] = {
            "window": W, "fwd_us": round(tf * 1e6, 1), "bwd_us": round(tb * 1e6, 1),
            "fwd_tflops": round(ff / tf / 1e12, 1), "bwd_tflops": round(fb / tb / 1e12, 1),
            "fwd_bwd_tflops": round((ff + fb) / (tf + tb) / 1e12, 1),
            "frac_bf16_peak": round((ff + fb) / (tf + tb) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "workspace_bytes": int(ws.numel()), "_f": ff + fb, "_t": tf + tb}
        del ws
    n = {key: sum(1 for W in cfg.windows if (W < 0) == (key == "L")) for key in layers}
    tot_f = sum(n[key] * layers[key].pop("_f") for key in layers)
    tot_t = sum(n[key] * layers[key].pop("_t") for key in layers)
    del q, k, v, do, o, lse, grads
    torch.cuda.empty_cache()
    return {"workload": cfg.name, "layers": layers, "sssl_fwd_bwd_tflops": round(tot_f / tot_t / 1e12, 1),
            "sssl_frac_bf16_peak": round(tot_f / tot_t / 1e12 / PEAK_BF16_TFLOPS, 4), "timed_calls": iters}


def fp8_detail(nc, torch, cfg, dev, stream, iters=10):
    """The fp8 forward on a workload's shape (inputs drawn as its bf16 ones and
    stored as e4m3 with per-tensor descales), per window of its layer pattern,
    beside the bf16 forward on the same shape: TFLOP/s (the same algorithmic
    4 D flops per visible pair) and the fraction of the fp8 MFMA peak."""
    from workloads import config_inputs, fp8_inputs
    (q8, k8, v8), (dq, dk, dv) = fp8_inputs(cfg.B, cfg.T, cfg.H, cfg.KV, cfg.D, seed=cfg.seed)
    q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
    q0, k0, v0, _ = config_inputs(cfg)
    q, k, v = q0.to(dev), k0.to(dev), v0.to(dev)
    del q0, k0, v0
    o = torch.empty(cfg.B, cfg.T, cfg.H, cfg.D, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(cfg.B, cfg.H, cfg.T, dtype=torch.float32, device=dev)
    out = {"workload": cfg.name, "descales": [round(x, 8) for x in (dq, dk, dv)]}
    for W in sorted(set(cfg.windows)):
        fl = 4 * cfg.D * visible_pairs(cfg.T, W) * cfg.B * cfg.H
        t8 = event_us(torch, stream, lambda: nc.fwd_fp8(q8, k8, v8, dq, dk, dv, window=(W, 0), out=(o, lse)), iters)
        tb = event_us(torch, stream, lambda: nc.fwd(q, k, v, window=(W, 0), out=(o, lse)), iters)
        out["full" if W < 0 else f"w{W}"] = {
            "fp8_us": round(t8, 2), "fp8_tflops": round(fl / (t8 * 1e-6) / 1e12, 1),
            "frac_fp8_peak": round(fl / (t8 * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "bf16_us": round(tb, 2), "bf16_tflops": round(fl / (tb * 1e-6) / 1e12, 1)}
    del q8, k8, v8, q, k, v, o, lse
    torch.cuda.empty_cache()
    return out


def qknorm_detail(nc, torch, cfg, dev, stream):
    """QK-norm + RoPE of a workload's q, k (GB/s), its backward, the logit-gain
    variant, the forward with QK-norm + RoPE fused into it and the backward with
    the norm's backward fused into it, each against the two calls it replaces,
    per window of the layer pattern."""
    from workloads import config_inputs
    q0, k0, v0, do0 = config_inputs(cfg)
    q, k, v = q0.to(dev), k0.to(dev), v0.to(dev)
    del q0, k0, v0
    B, T, H, KV, D = cfg.B, cfg.T, cfg.H, cfg.KV, cfg.D
    base = cfg.rope_base
    qk_bytes = B * T * (H + KV) * D * 2 * 2
    out = {}
    us = event_us(torch, stream, lambda: nc.qknorm_rope_(q, k, None, rope_base=base, eps=1e-6), 20)
    out["qknorm_rope"] = {"us": round(us, 2), "GBps": round(qk_bytes / (us * 1e-6) / 1e9, 1),
                          "frac_hbm": round(qk_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                          "algorithmic_bytes": qk_bytes}
    us = event_us(torch, stream, lambda: nc.qknorm_rope_(q, k, None, rope_base=base, eps=1e-6,
                                                         qk_gain=math.sqrt(1.2)), 20)
    out["qknorm_rope_gain_sqrt1p2"] = {"us": round(us, 2), "GBps": round(qk_bytes / (us * 1e-6) / 1e9, 1),
                                       "qk_gain": round(math.sqrt(1.2), 6)}
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    us = event_us(torch, stream, lambda: nc.qknorm_rope_bwd_(dq, dk, q, k, None, rope_base=base, eps=1e-6), 20)
    nb = 3 * (qk_bytes // 2)
    out["qknorm_rope_bwd"] = {"us": round(us, 2), "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                              "frac_hbm": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4), "algorithmic_bytes": nb}
    o = torch.empty_like(q)
    lse = torch.empty(B, H, T, dtype=torch.float32, device=dev)
    fused = {}
    for W in sorted(set(cfg.windows)):
        def two_calls():
            nc.qknorm_rope_(q, k, None, rope_base=base, eps=1e-6)
            nc.fwd(q, k, v, window=(W, 0), out=(o, lse))

        def one_call():
            nc.fwd_qknorm_rope_(q, k, v, None, rope_base=base, eps=1e-6, window=(W, 0), out=(o, lse))
        t2 = event_us(torch, stream, two_calls, 20)
        t1 = event_us(torch, stream, one_call, 20)
        fl = 4 * D * visible_pairs(T, W) * B * H
        fused["full" if W < 0 else f"w{W}"] = {"two_calls_us": round(t2, 2), "fused_us": round(t1, 2),
                                               "fused_fwd_TFLOPs": round(fl / (t1 * 1e-6) / 1e12, 1)}
    out["fwd_qknorm_rope"] = fused
    # the backward with QK-norm + RoPE's backward folded into the dQ and dK/dV
    # epilogues, against the attention backward followed by the norm's backward
    do = do0.to(dev)
    del do0
    qn, kn = q.clone(), k.clone()
    _, _, rstd = nc.qknorm_rope_rstd_(qn, kn, None, rope_base=base, eps=1e-6)
    ws = nc.bwd_workspace(q, k, (-1, 0))
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fb = {}
    for W in sorted(set(cfg.windows)):
        nc.fwd(qn, kn, v, window=(W, 0), out=(o, lse))

        def two_calls_bwd():
            nc.bwd(qn, kn, v, o, lse, do, window=(W, 0), out=(gq, gk, gv), workspace=ws)
            nc.qknorm_rope_bwd_(gq, gk, q, k, None, rope_base=base, eps=1e-6)

        def one_call_bwd():
            nc.bwd_qknorm_rope(qn, kn, v, o, lse, do, rstd, None, rope_base=base, window=(W, 0),
                               out=(gq, gk, gv), workspace=ws)
        t2 = event_us(torch, stream, two_calls_bwd, 20)
        t1 = event_us(torch, stream, one_call_bwd, 20)
        fl = 8 * D * visible_pairs(T, W) * B * H
        fb["full" if W < 0 else f"w{W}"] = {"two_calls_us": round(t2, 2), "fused_us": round(t1, 2),
                                            "fused_bwd_TFLOPs": round(fl / (t1 * 1e-6) / 1e12, 1)}
    out["bwd_qknorm_rope"] = fb
    # fwd+bwd including QK-norm + RoPE and its backward, over the layer pattern:
    # the separate calls, and the fused forward + fused backward
    tot_f = tot_sep = tot_fused = 0.0
    for W in cfg.windows:
        key = "full" if W < 0 else f"w{W}"
        tot_f += 12 * D * visible_pairs(T, W) * B * H
        tot_sep += (fused[key]["two_calls_us"] + fb[key]["two_calls_us"]) * 1e-6
        tot_fused += (fused[key]["fused_us"] + fb[key]["fused_us"]) * 1e-6
    out["fwd_bwd_incl_qknorm_rope"] = {
        "layers": list(cfg.windows), "separate_calls_tflops": round(tot_f / tot_sep / 1e12, 1),
        "fused_calls_tflops": round(tot_f / tot_fused / 1e12, 1),
        "note": "algorithmic attention FLOPs of the layers / time of QK-norm + RoPE, fwd, bwd and the norm's bwd"}
    del q, k, v, dq, dk, o, lse, do, qn, kn, ws, gq, gk, gv, rstd
    torch.cuda.empty_cache()
    return out


def run_step_bench(nc, torch, cfg, dev, stream, args):
    """The timed training step of `cfg` (see the module docstring).  Returns
    (ms_per_step, value, roofline, detail, layers, workspace, launch)."""
    from workloads import config_inputs
    B, T, H, KV, D = cfg.B, cfg.T, cfg.H, cfg.KV, cfg.D
    q0, k0, v0, do0 = config_inputs(cfg)
    layers = []
    for W in cfg.windows:
        L = dict(W=W, q=q0.to(dev), k=k0.to(dev), v=v0.to(dev), do=do0.to(dev))
        L["o"] = torch.empty_like(L["q"])
        L["lse"] = torch.empty(B, H, T, dtype=torch.float32, device=dev)
        L["dq"], L["dk"], L["dv"] = torch.empty_like(L["q"]), torch.empty_like(L["k"]), torch.empty_like(L["v"])
        layers.append(L)
    del q0, k0, v0, do0
    # one workspace for every layer, sized for the window that needs the most
    lib = nc.lib()
    W_ws = max(set(cfg.windows), key=lambda W: lib.ncattn_bwd_workspace_bytes(B, T, H, KV, D, W, nc.BF16))
    ws = nc.bwd_workspace(layers[0]["q"], layers[0]["k"], (W_ws, 0))
    with_qk = not cfg.pre_normed
    names = (["qknorm_rope"] if with_qk else []) + ["fwd", "bwd_delta", "bwd_dkdv", "bwd_dq"]

    def kernels(L):
        out = []
        if with_qk:
            out.append(lambda: nc.qknorm_rope_(L["q"], L["k"], None, rope_base=cfg.rope_base, eps=1e-6))
        out.append(lambda: nc.fwd(L["q"], L["k"], L["v"], window=(L["W"], 0), out=(L["o"], L["lse"])))
        for st in ("preprocess", "dkdv", "dq"):
            out.append(lambda st=st: nc.bwd(L["q"], L["k"], L["v"], L["o"], L["lse"], L["do"], window=(L["W"], 0),
                                            out=(L["dq"], L["dk"], L["dv"]), workspace=ws, stage=st))
        return out
    launch = [kernels(L) for L in layers]

    def step(ev=None):
        # ev: {(layer, i): Event}; event i of a layer is recorded before kernel i of
        # `names` (i = len(names): after the last), only where ev has an entry
        for li in range(len(layers)):
            for i, fn in enumerate(launch[li]):
                e = None if ev is None else ev.get((li, i))
                if e is not None:
                    e.record(stream)
                fn()
            e = None if ev is None else ev.get((li, len(names)))
            if e is not None:
                e.record(stream)

    nl = len(layers)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Per-kernel breakdown (the "detail" figures): an untimed pass with an event
    # before and after every kernel.  Each event is a packet of its own between
    # kernels (a few us of GPU time), so the timed region below records events
    # around the dominant kernel only.
    prof_steps = max(1, args.profile_steps)
    pev = [{(li, i): torch.cuda.Event(enable_timing=True) for li in range(nl) for i in range(len(names) + 1)}
           for _ in range(prof_steps)]
    for s in range(prof_steps):
        step(pev[s])
    torch.cuda.synchronize()
    dur = {n: [0.0] * nl for n in names}  # ms per launch, per layer
    for s in range(prof_steps):
        for li in range(nl):
            for i, n in enumerate(names):
                dur[n][li] += pev[s][(li, i)].elapsed_time(pev[s][(li, i + 1)]) / prof_steps
    totals = {n: sum(dur[n]) for n in names}
    dominant = max(totals, key=totals.get)
    kd = names.index(dominant)

    # Timed region: step s brackets the dominant kernel of layer s mod 4 with HIP
    # events (every layer when there are fewer steps than layers), so the launches
    # of every layer type are sampled equally.
    def timed_events(s):
        lis = range(nl) if args.steps < nl else (s % nl,)
        return {(li, i): torch.cuda.Event(enable_timing=True) for li in lis for i in (kd, kd + 1)}
    events = [timed_events(s) for s in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    samples = [[] for _ in range(nl)]  # dominant-kernel durations (ms), per layer
    for ev in events:
        for li in range(nl):
            if (li, kd) in ev:
                samples[li].append(ev[(li, kd)].elapsed_time(ev[(li, kd + 1)]))
    dom_ms = [sum(x) / len(x) for x in samples]  # average launch per layer, over the timed region

    pairs = [visible_pairs(T, L["W"]) * B * H for L in layers]
    f_fwd = [4 * D * p for p in pairs]
    f_bwd = [8 * D * p for p in pairs]
    flops_step = sum(f_fwd) + sum(f_bwd)
    value = flops_step / (ms_per_step * 1e-3) / 1e12
    attn_names = [n for n in names if n != "qknorm_rope"]
    t_attn = sum(totals[n] for n in attn_names)
    # algorithmic work attributed per kernel: fwd 4D/pair; dkdv computes dV, dP, dK
    # (6D/pair); dq computes dQ (2D/pair); the S/dP recomputations are not counted
    share = {"fwd": 4, "bwd_dkdv": 6, "bwd_dq": 2}
    if dominant in share:
        work = sum(share[dominant] * D * p for p in pairs)
        achieved = work / (sum(dom_ms) * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "kernel": dominant,
                "work_per_unit": f"{share[dominant]}*D flops per visible (query, key) pair and head",
                "units_per_launch": sum(pairs) // nl}
    else:
        nbytes = (B * T * (H + KV) * D * 2 * 2) if dominant == "qknorm_rope" else (B * T * H * D * 2 * 2 + B * H * T * 4)
        achieved = nbytes * len(layers) / (sum(dom_ms) * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "kernel": dominant}
    roof["traffic"] = measured_traffic(dominant, cfg.name)
    roof["avg_launch_us"] = round(sum(dom_ms) * 1e3 / nl, 2)
    roof["launches_timed"] = sum(len(x) for x in samples)

    per_layer = []
    for li, L in enumerate(layers):
        tf = dur["fwd"][li]
        tb = dur["bwd_delta"][li] + dur["bwd_dkdv"][li] + dur["bwd_dq"][li]
        e = {"window": L["W"], "fwd_us": round(tf * 1e3, 1), "bwd_us": round(tb * 1e3, 1),
             "fwd_tflops": round(f_fwd[li] / (tf * 1e-3) / 1e12, 1),
             "bwd_tflops": round(f_bwd[li] / (tb * 1e-3) / 1e12, 1),
             "dkdv_us": round(dur["bwd_dkdv"][li] * 1e3, 1), "dq_us": round(dur["bwd_dq"][li] * 1e3, 1),
             "delta_us": round(dur["bwd_delta"][li] * 1e3, 1)}
        if with_qk:
            e["qknorm_rope_us"] = round(dur["qknorm_rope"][li] * 1e3, 1)
        per_layer.append(e)
    detail = {
        "fwd_bwd_tflops_kernels_only": round(flops_step / (t_attn * 1e-3) / 1e12, 1),
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "kernel_ms_per_step": {n: round(totals[n], 4) for n in names},
        "kernel_share_of_step": {n: round(totals[n] / sum(totals.values()), 4) for n in names},
        "layers": per_layer,
        "algorithmic_gflop_per_step": round(flops_step / 1e9, 2),
        "bwd_workspace_bytes": int(ws.numel()),
        "per_kernel_from": f"untimed pass of {prof_steps} steps with events around every kernel",
    }
    names_idx = {n: i for i, n in enumerate(names)}
    dom_launch = launch[-1][names_idx[dominant]]
    return ms_per_step, value, roof, detail, layers, ws, dom_launch, dominant


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa", choices=["gqa", "d12", "d20"],
                    help="workload of the timed step (default: the grouped-query layer, the largest)")
    ap.add_argument("--profile-steps", type=int, default=5,
                    help="untimed steps with an event around every kernel, for the per-kernel breakdown")
    ap.add_argument("--decode-iters", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the 2 s graphics-clock measurement under the dominant kernel")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-layer-type fwd/bwd timings of the other workloads and the QK-norm + RoPE "
                         "figures (standalone, backward, gain variant, fused forward)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB device-to-device 3 times: a kernel of "
                         "known traffic for calibrating rocprofv3's FETCH_SIZE/WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only (the attention path needs no collective); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_attention_qknorm_amd as nc
    from workloads import D12, D20, DECODE, GQA, HD64, decode_inputs

    nc.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    cfg = {"gqa": GQA, "d12": D12, "d20": D20}[args.workload]
    ms_per_step, value, roof, detail, layers, ws, dom_launch, dominant = run_step_bench(nc, torch, cfg, dev, stream,
                                                                                        args)

    # Graphics clock while the dominant kernel runs back to back for 2 s (full
    # causal layer), after the timed region: amdsmi's table lags about a second.
    if not args.no_clock:
        clock = ClockSampler()
        with clock:
            t_end = time.perf_counter() + 2.0
            while time.perf_counter() < t_end:
                for _ in range(5):
                    dom_launch()
                torch.cuda.synchronize()
        detail["gpu_clock_mhz"] = dict(clock.summary(skip_s=1.2), under=f"{dominant} back to back, full-causal layer",
                                       source="amdsmi, every 20 ms, samples of the last 0.8 s")
    del layers, ws, dom_launch
    torch.cuda.empty_cache()

    if not args.no_configs:
        detail["qknorm_rope"] = {c.name: qknorm_detail(nc, torch, c, dev, stream) for c in (D12, D20, GQA)}

    prefill = None
    if not args.no_decode:
        from workloads import PREFILL, prefill_inputs
        c = PREFILL
        qp, knp, vnp, kcp, vcp, lensp = (x.to(dev) for x in prefill_inputs(
            c.B, c.Tn, c.H, c.KV, c.D, c.min_len, c.max_len, c.T_max, seed=c.seed, poison=False))
        op = torch.empty_like(qp)
        lens_h = lensp.cpu().tolist()
        prefill = {}
        for W in c.windows:
            us = event_us(torch, stream, lambda: nc.prefill(qp, knp, vnp, kcp, vcp, lensp, window=W, out=op), 10)
            pairs = sum(min(s_ + i + 1, W + 1) if W >= 0 else s_ + i + 1 for s_ in lens_h for i in range(c.Tn))
            tf = 4 * c.D * pairs * c.H / (us * 1e-6) / 1e12
            prefill["L" if W < 0 else "S"] = {"window": W, "us": round(us, 2), "tflops": round(tf, 1),
                                              "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                              "workload": c.name}
        del qp, knp, vnp, kcp, vcp

    replicate = None
    if not args.no_decode:
        # prefill once, clone for the samples: a 2048-token batch-1 prompt cache
        # copied into the 64 rows of the engine decode cache
        from workloads import replicate_inputs
        c, s_len = DECODE, 2048
        ksr, vsr, kdr, vdr, slr = (x.to(dev) for x in replicate_inputs(c.B, s_len, c.T_max, c.KV, c.D, s_len, seed=9))
        dlr = torch.empty(c.B, dtype=torch.int32, device=dev)
        us = event_us(torch, stream, lambda: nc.cache_replicate(ksr, vsr, slr, kdr, vdr, dlr), 10)
        part = 2 * s_len * c.KV * c.D * 2            # K and V of the prompt
        nbytes = part * (1 + c.B)                    # read once, written to every row
        gbps = nbytes / (us * 1e-6) / 1e9
        replicate = {"rows": c.B, "prompt_len": s_len, "us": round(us, 2), "GBps": round(gbps, 1),
                     "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4), "algorithmic_bytes": nbytes}
        del ksr, vsr, kdr, vdr

    decode = None
    if not args.no_decode:
        c = DECODE
        qd, knd, vnd, kcd, vcd, lens = (x.to(dev) for x in decode_inputs(c.B, c.H, c.KV, c.D, c.min_len, c.max_len,
                                                                           c.T_max, seed=c.seed, poison=False))
        sets = [(kcd, vcd)] + [(kcd.clone(), vcd.clone()) for _ in range(3)]  # rotate past the 256 MB MALL
        od = torch.empty_like(qd)
        decode = {}
        lens_h = lens.cpu().tolist()
        for W in c.windows:
            wsd = nc.decode_workspace(qd, kcd, W)
            for i in range(3):
                kc, vc = sets[i % 4]
                nc.decode(qd, knd, vnd, kc, vc, lens, window=W, out=od, workspace=wsd)
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.decode_iters)]
            for i in range(args.decode_iters):
                kc, vc = sets[i % 4]
                evs[i][0].record(stream)
                nc.decode(qd, knd, vnd, kc, vc, lens, window=W, out=od, workspace=wsd)
                evs[i][1].record(stream)
            torch.cuda.synchronize()
            us = sum(a.elapsed_time(b) for a, b in evs) * 1e3 / len(evs)
            nbytes = decode_algorithmic_bytes(lens_h, c.H, c.KV, c.D, W)
            gbps = nbytes / (us * 1e-6) / 1e9
            tr = [measured_traffic(kn, f"{c.name} W={W}") for kn in ("decode_split", "decode_combine")]
            decode["L" if W < 0 else "S"] = {"window": W, "us": round(us, 2), "GBps": round(gbps, 1),
                                             "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
                                             "algorithmic_bytes": nbytes,
                                             "traffic": None if None in tr else sum(tr)}
        del sets

    configs = None
    if not args.no_configs:
        configs = {c.name: time_config(nc, torch, c, dev, stream) for c in (GQA, D12, D20) if c is not cfg}
        # the head_dim-64 kernels on a layer of GPT-2's head size (not one of the
        # workloads above: reported as detail)
        detail["head_dim_64"] = time_config(nc, torch, HD64, dev, stream)
        # the fp8 forward on the grouped-query layer's shape (reported as detail:
        # the step above is bf16)
        detail["fp8_fwd"] = fp8_detail(nc, torch, GQA, dev, stream)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "global_batch": cfg.B, "seq_len": cfg.T, "n_head": cfg.H,
                   "n_kv_head": cfg.KV, "head_dim": cfg.D, "windows": list(cfg.windows),
                   "qknorm_rope_in_step": not cfg.pre_normed, "parallelism": "single GPU"},
        "roofline": roof,
        "decode": decode,
        "prefill": prefill,
        "cache_replicate": replicate,
        "configs": configs,
        "detail": detail,
    }
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
