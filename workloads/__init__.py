"""Seeded synthetic workloads shared by the tests, the bench and smoke().

This module only draws random numbers and describes shapes: it holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can be fed from it
without sharing any of the method's code.

Recipe: ``numpy.random.default_rng(seed)`` (PCG64) draws float32 N(0, 1) arrays in
a fixed order (q, k, v, dO for attention; L_b, caches, q, k_new, v_new for
decode).  Values are rounded once to the I/O dtype with torch (round to nearest
even for bf16); the *same* rounded values go to the GPU and, upcast to float64,
to the oracle.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

try:  # torch is only needed to round to bf16 and hand tensors to the device
    import torch
except ImportError:  # pragma: no cover
    torch = None


@dataclass(frozen=True)
class AttnConfig:
    name: str
    B: int
    T: int
    H: int
    KV: int
    D: int
    dtype: str                 # "bf16" | "f32"
    short_window: int          # window of the 'S' layers
    pattern: str = "SSSL"
    n_layer: int = 4
    windows: tuple = ()        # per-layer window_left, written out (-1 = full causal)
    rope_base: float = 100000.0
    pre_normed: bool = False   # True: q, k are used as drawn (already post-norm/RoPE)
    seed: int = 0


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    H: int
    KV: int
    D: int
    min_len: int
    max_len: int
    T_max: int
    windows: tuple = (-1, 1024)
    seed: int = 5
    dtype: str = "bf16"


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    Tn: int          # tokens of the chunk appended to every sequence
    H: int
    KV: int
    D: int
    min_len: int     # cached tokens before the chunk, U[min_len, max_len]
    max_len: int
    T_max: int
    windows: tuple = (-1, 1024)
    seed: int = 6
    dtype: str = "bf16"


# The five workloads: a tiny fp32 case, two nanochat-shaped layers (d12: model
# dim 768, 6 heads; d20: 1280, 10 heads; head_dim 128, T = 2048, SSSL windows),
# a grouped-query case at T = 4096 and an engine decode batch.
TINY = AttnConfig("tiny_b1_t64_h2_d64_f32", B=1, T=64, H=2, KV=2, D=64, dtype="f32",
                  short_window=-1, pattern="L", n_layer=1, windows=(-1,), rope_base=10000.0, seed=1)
D12 = AttnConfig("d12_b8_t2048_h6_d128_bf16", B=8, T=2048, H=6, KV=6, D=128, dtype="bf16",
                 short_window=1024, windows=(1024, 1024, 1024, -1), seed=2)
D20 = AttnConfig("d20_b32_t2048_h10_d128_bf16", B=32, T=2048, H=10, KV=10, D=128, dtype="bf16",
                 short_window=1024, windows=(1024, 1024, 1024, -1), seed=3)
GQA = AttnConfig("gqa_b16_t4096_h12_kv4_d128_bf16", B=16, T=4096, H=12, KV=4, D=128, dtype="bf16",
                 short_window=2048, windows=(2048, 2048, 2048, -1),
                 pre_normed=True, seed=4)
# head_dim 64 (GPT-2's n_embd / n_head = 768 / 12, "nanoGPT Administrator & Developer
# Guide", sections 3 and 6) at the d12 layer's token count per batch: a measurement
# and parity case for the head_dim-64 kernels, inputs taken as post-norm.
HD64 = AttnConfig("hd64_b16_t2048_h12_d64_bf16", B=16, T=2048, H=12, KV=12, D=64, dtype="bf16",
                  short_window=1024, windows=(1024, 1024, 1024, -1), pre_normed=True, seed=7)
DECODE = DecodeConfig("decode_b64_h10_d128_bf16", B=64, H=10, KV=10, D=128,
                      min_len=256, max_len=8192, T_max=8320)

# Chunked prefill (the engine path beyond single-token decode): 16 sequences with
# 0..3584 cached tokens each receive a 512-token chunk.
PREFILL = PrefillConfig("prefill_b16_tn512_h10_d128_bf16", B=16, Tn=512, H=10, KV=10, D=128,
                        min_len=0, max_len=3584, T_max=4096)

ATTN_CONFIGS = {c.name: c for c in (TINY, D12, D20, GQA)}


def _to_dtype(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def attn_inputs(B, T, H, KV, D, dtype="bf16", seed=0):
    """q [B][T][H][D], k, v [B][T][KV][D], dO [B][T][H][D] as CPU torch tensors
    of the I/O dtype, drawn in that order from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, D), dtype=np.float32)
    k = rng.standard_normal((B, T, KV, D), dtype=np.float32)
    v = rng.standard_normal((B, T, KV, D), dtype=np.float32)
    do = rng.standard_normal((B, T, H, D), dtype=np.float32)
    return tuple(_to_dtype(x, dtype) for x in (q, k, v, do))


def fp8_inputs(B, T, H, KV, D, seed=0):
    """q [B][T][H][D], k, v [B][T][KV][D] drawn as attn_inputs draws them (fp32
    N(0, 1), in that order) and stored as OCP e4m3 (torch.float8_e4m3fn, round to
    nearest) with one descale per tensor, amax / 448, so that each tensor's largest
    magnitude lands on e4m3's largest finite value.  Returns ((q8, k8, v8),
    (q_descale, k_descale, v_descale)): CPU tensors and Python floats; x8 times its
    descale is the value the test's reference sees."""
    rng = np.random.default_rng(seed)
    xs = (rng.standard_normal((B, T, H, D), dtype=np.float32),
          rng.standard_normal((B, T, KV, D), dtype=np.float32),
          rng.standard_normal((B, T, KV, D), dtype=np.float32))
    out, scales = [], []
    for x in xs:
        descale = float(np.abs(x).max()) / 448.0
        out.append((torch.from_numpy(x) / descale).to(torch.float8_e4m3fn))
        scales.append(descale)
    return tuple(out), tuple(scales)


def config_inputs(cfg: AttnConfig):
    return attn_inputs(cfg.B, cfg.T, cfg.H, cfg.KV, cfg.D, cfg.dtype, cfg.seed)


def decode_inputs(B, H, KV, D, min_len, max_len, T_max, seed=5, poison=True, dtype="bf16"):
    """Engine decode batch: lengths L_b ~ U[min_len, max_len] (inclusive), caches
    [B][T_max][KV][D] with slots < L_b ~ N(0, 1) and slots >= L_b NaN (poison) or
    N(0, 1), then q [B][1][H][D], k_new, v_new [B][1][KV][D]; cache_seqlens = L_b.
    Returns CPU torch tensors (caches/q/new in the I/O dtype, lengths int32)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(min_len, max_len + 1, size=B).astype(np.int32)
    assert int(lens.max()) < T_max
    kc = rng.standard_normal((B, T_max, KV, D), dtype=np.float32)
    vc = rng.standard_normal((B, T_max, KV, D), dtype=np.float32)
    if poison:
        slot = np.arange(T_max)[None, :]
        dead = slot >= lens[:, None]
        kc[dead] = np.nan
        vc[dead] = np.nan
    q = rng.standard_normal((B, 1, H, D), dtype=np.float32)
    kn = rng.standard_normal((B, 1, KV, D), dtype=np.float32)
    vn = rng.standard_normal((B, 1, KV, D), dtype=np.float32)
    out = [_to_dtype(x, dtype) for x in (q, kn, vn, kc, vc)]
    return (*out, torch.from_numpy(lens))


def replicate_inputs(N, T_src, T_max, KV, D, prompt_len, seed=9, dtype="bf16"):
    """Batch-1 prefill cache k_src, v_src [1][T_src][KV][D] ~ N(0, 1) with rows
    >= prompt_len NaN (they must not be copied), destination caches k_dst, v_dst
    [N][T_max][KV][D] ~ N(0, 1) (their rows >= prompt_len must survive), and the
    source length as int32 [1].  CPU torch tensors of the I/O dtype."""
    rng = np.random.default_rng(seed)
    ks = rng.standard_normal((1, T_src, KV, D), dtype=np.float32)
    vs = rng.standard_normal((1, T_src, KV, D), dtype=np.float32)
    if 0 <= prompt_len <= T_src:
        ks[:, prompt_len:] = np.nan
        vs[:, prompt_len:] = np.nan
    kd = rng.standard_normal((N, T_max, KV, D), dtype=np.float32)
    vd = rng.standard_normal((N, T_max, KV, D), dtype=np.float32)
    out = [_to_dtype(x, dtype) for x in (ks, vs, kd, vd)]
    return (*out, torch.tensor([prompt_len], dtype=torch.int32))


def prefill_inputs(B, Tn, H, KV, D, min_len, max_len, T_max, seed=6, poison=True, dtype="bf16"):
    """Prefill batch: lengths L_b ~ U[min_len, max_len] (inclusive), caches
    [B][T_max][KV][D] with slots < L_b ~ N(0, 1) and slots >= L_b NaN (poison) or
    N(0, 1), then q [B][Tn][H][D], k_new, v_new [B][Tn][KV][D]; cache_seqlens =
    L_b.  Returns CPU torch tensors (lengths int32)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(min_len, max_len + 1, size=B).astype(np.int32)
    assert int(lens.max()) + Tn <= T_max
    kc = rng.standard_normal((B, T_max, KV, D), dtype=np.float32)
    vc = rng.standard_normal((B, T_max, KV, D), dtype=np.float32)
    if poison:
        dead = np.arange(T_max)[None, :] >= lens[:, None]
        kc[dead] = np.nan
        vc[dead] = np.nan
    q = rng.standard_normal((B, Tn, H, D), dtype=np.float32)
    kn = rng.standard_normal((B, Tn, KV, D), dtype=np.float32)
    vn = rng.standard_normal((B, Tn, KV, D), dtype=np.float32)
    out = [_to_dtype(x, dtype) for x in (q, kn, vn, kc, vc)]
    return (*out, torch.from_numpy(lens))


def f64(t):
    """CPU float64 numpy view of a (possibly bf16, possibly device) tensor."""
    return t.detach().to("cpu", torch.float64).numpy()
