"""CPU-side checks of the C-ABI library: it loads, exports every function that
include/ncattn.h declares, and rejects bad arguments on the host with the right
status code before anything is launched (so these run without a GPU)."""

import ctypes
import json
import os
import re

import pytest

import transformer_attention_qknorm_amd as nc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ncattn.h")

EINVAL, EUNSUP, EWS = -1, -2, -3
P = 4096          # a fake, 16-byte-aligned, non-NULL "device pointer": never dereferenced
MIS = 4096 + 8    # misaligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nc.LIB_PATH):
        from transformer_attention_qknorm_amd._build import build
        build()
    return nc.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ncattn_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert {"ncattn_qknorm_rope", "ncattn_qknorm_rope_bwd", "ncattn_fwd", "ncattn_bwd", "ncattn_decode"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"libncattn.so does not export {n}"
    # and the shared object's dynamic symbol table agrees
    import subprocess
    syms = subprocess.run(["nm", "-D", "--defined-only", nc.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", syms), n


def test_version_and_empty_error(L):
    assert L.ncattn_version().decode().startswith("ncattn")
    assert isinstance(L.ncattn_last_error(), bytes)


def test_qknorm_rope_bwd_validation(L):
    f = L.ncattn_qknorm_rope_bwd
    args = dict(dq=P, dk=P + 16, q=P + 32, k=P + 48)
    def call(dq=P, dk=P + 16, q=P + 32, k=P + 48, D=128, base=1e5, eps=1e-6, gain=1.0, dt=0, pos=None):
        return f(dq, dk, q, k, 1, 4, 2, 2, D, pos, base, eps, gain, dt, None)
    assert call(dq=None) == EINVAL
    assert call(k=None) == EINVAL
    assert call(dq=P + 32) == EINVAL          # dq aliases q
    assert call(dk=P + 48) == EINVAL          # dk aliases k
    assert call(dk=P) == EINVAL               # dq == dk
    assert call(q=MIS) == EINVAL
    assert call(D=96) == EUNSUP
    assert call(base=1.0) == EINVAL
    assert call(eps=-1.0) == EINVAL
    assert call(pos=P + 2) == EINVAL
    assert call(dt=5) == EINVAL
    assert "ncattn_qknorm_rope_bwd" in L.ncattn_last_error().decode()


def fwd(L, q=P, k=P, v=P, o=P + 16, lse=P + 32, B=1, T=64, H=2, KV=2, D=128, wl=-1, wr=0, scale=0.0, dt=0):
    return L.ncattn_fwd(q, k, v, o, lse, B, T, H, KV, D, wl, wr, scale, dt, None)


def test_fwd_validation(L):
    assert fwd(L, q=None) == EINVAL
    assert "q is NULL" in L.ncattn_last_error().decode()
    assert fwd(L, k=MIS) == EINVAL
    assert "aligned" in L.ncattn_last_error().decode()
    assert fwd(L, B=0) == EINVAL
    assert fwd(L, T=-3) == EINVAL
    assert fwd(L, H=6, KV=4) == EINVAL
    assert fwd(L, wl=-2) == EINVAL
    assert fwd(L, wr=1) == EINVAL
    assert fwd(L, dt=7) == EINVAL
    assert fwd(L, D=96) == EUNSUP          # bf16 MFMA path is head_dim 64 or 128
    assert fwd(L, D=256) == EUNSUP
    assert fwd(L, D=96, dt=1) == EUNSUP
    assert fwd(L, o=P) == EINVAL            # o aliases q
    assert fwd(L, scale=float("nan")) == EINVAL


def test_fwd_qknorm_rope_validation(L):
    f = L.ncattn_fwd_qknorm_rope
    def call(q=P, k=P + 16, v=P + 32, o=P + 48, lse=P + 64, rstd=None, B=1, T=4, H=2, KV=2, D=128, pos=None,
             base=1e5, eps=1e-6, gain=1.0, wl=-1, wr=0, scale=0.0, dt=0):
        return f(q, k, v, o, lse, rstd, B, T, H, KV, D, pos, base, eps, gain, wl, wr, scale, dt, None)
    assert call(q=None) == EINVAL
    assert call(lse=MIS) == EINVAL
    assert call(rstd=P + 2) == EINVAL         # rstd misaligned
    assert call(k=P) == EINVAL                # q and k must be distinct
    assert call(o=P + 16) == EINVAL           # o aliases k
    assert call(v=P) == EINVAL                # v aliases q
    assert call(H=6, KV=4) == EINVAL
    assert call(base=0.5) == EINVAL
    assert call(eps=-1.0) == EINVAL
    assert call(pos=P + 2) == EINVAL          # pos_offset misaligned
    assert call(wl=-2) == EINVAL
    assert call(wr=1) == EINVAL
    assert call(D=96) == EUNSUP               # head_dim 64 or 128
    assert call(D=96, dt=1) == EUNSUP
    assert call(scale=float("inf")) == EINVAL


def test_qknorm_rope_rstd_validation(L):
    f = L.ncattn_qknorm_rope_rstd
    assert f(P, P + 16, None, 1, 4, 2, 2, 128, None, 1e5, 1e-6, 1.0, 0, None) == EINVAL   # rstd NULL
    assert f(P, P + 16, P + 34, 1, 4, 2, 2, 128, None, 1e5, 1e-6, 1.0, 0, None) == EINVAL  # rstd misaligned
    assert f(None, P + 16, P + 32, 1, 4, 2, 2, 128, None, 1e5, 1e-6, 1.0, 0, None) == EINVAL
    assert f(P, P + 16, P + 32, 1, 4, 2, 2, 96, None, 1e5, 1e-6, 1.0, 0, None) == EUNSUP
    assert f(P, P + 16, P + 32, 1, 4, 2, 2, 128, None, 0.5, 1e-6, 1.0, 0, None) == EINVAL
    assert "ncattn_qknorm_rope_rstd" in L.ncattn_last_error().decode()


def test_bwd_qknorm_rope_validation(L):
    f = L.ncattn_bwd_qknorm_rope
    need = L.ncattn_bwd_workspace_bytes(1, 8, 2, 2, 128, -1, 0)

    def call(rstd=P + 160, dq=P + 96, base=1e5, D=128, wl=-1, ws=P + 192, wsb=None):
        return f(P, P + 16, P + 32, P + 48, P + 64, P + 80, rstd, None, base, 1.0, dq, P + 112, P + 128, 1, 8, 2, 2,
                 D, wl, 0, 0.0, 0, ws, need if wsb is None else wsb, None)
    assert call(rstd=None) == EINVAL
    assert call(rstd=P + 162) == EINVAL
    assert call(dq=P + 160) == EINVAL          # dq aliases rstd
    assert call(dq=P) == EINVAL                # dq aliases q
    assert call(base=1.0) == EINVAL
    assert call(D=96) == EUNSUP
    assert call(wl=-2) == EINVAL
    assert call(wsb=need - 1) == EWS


def test_qknorm_rope_validation(L):
    f = L.ncattn_qknorm_rope
    assert f(None, P, 1, 4, 2, 2, 128, None, 1e5, 1e-6, 1.0, 0, None) == EINVAL
    assert f(P, P + 16, 1, 4, 2, 2, 96, None, 1e5, 1e-6, 1.0, 0, None) == EUNSUP
    assert f(P, P + 16, 1, 4, 2, 2, 128, None, 0.5, 1e-6, 1.0, 0, None) == EINVAL
    assert f(P, P + 16, 1, 4, 2, 2, 128, None, 1e5, -1.0, 1.0, 0, None) == EINVAL
    assert f(P, P + 16, 1, 4, 2, 2, 128, P + 2, 1e5, 1e-6, 1.0, 0, None) == EINVAL  # pos_offset misaligned
    assert f(P, P + 16, 1, 4, 3, 2, 128, None, 1e5, 1e-6, 1.0, 0, None) == EINVAL


def test_bwd_validation_and_workspace(L):
    # the per-row D (fp32, padded to 256 B); bf16 adds LSE * log2(e) of the same
    # size.  Nothing grows with T^2: the dQ stage recomputes dS instead of reading
    # it from the workspace.
    def rows(B, T, H):
        return (B * H * T * 4 + 255) // 256 * 256
    assert L.ncattn_bwd_workspace_bytes(2, 100, 4, 2, 128, -1, 1) == rows(2, 100, 4) == 3328
    # shapes the calls refuse get 0, never a wrapped size
    big = 2 ** 31 - 1
    assert L.ncattn_bwd_workspace_bytes(big, big, big, 1, 128, -1, 0) == 0
    assert L.ncattn_bwd_workspace_bytes(2, 100, 6, 4, 128, -1, 0) == 0        # n_head % n_kv_head
    assert L.ncattn_decode_workspace_bytes(big, big, big, 1, 128, -1) == 0
    for B, T, H, W in [(2, 100, 4, -1), (2, 100, 4, 98), (1, 2048, 1, -1), (1, 2048, 1, 1024), (1, 2048, 1, 0),
                       (3, 777, 2, 256), (16, 4096, 12, 2048), (16, 4096, 12, -1), (1, 32768, 10, -1)]:
        assert L.ncattn_bwd_workspace_bytes(B, T, H, H, 128, W, 0) == 2 * rows(B, T, H), (B, T, H, W)
    # a window reaching every key (W >= T - 1, up to INT_MAX) is full causal, sized as such
    full = L.ncattn_bwd_workspace_bytes(2, 100, 4, 2, 128, -1, 0)
    for W in (99, 100, 5000, 2 ** 31 - 64, 2 ** 31 - 1):
        assert L.ncattn_bwd_workspace_bytes(2, 100, 4, 2, 128, W, 0) == full, W
    assert L.ncattn_bwd_workspace_bytes(1, 2048, 1, 1, 128, -2, 0) == 0
    need = L.ncattn_bwd_workspace_bytes(2, 100, 4, 2, 128, -1, 0)
    args = [P, P + 16, P + 32, P + 48, P + 64, P + 80, P + 96, P + 112, P + 128, 2, 100, 4, 2, 128, -1, 0, 0.0, 0]
    assert L.ncattn_bwd(*args, None, 0, None) == EWS
    assert L.ncattn_bwd(*args, P + 256, need - 1, None) == EWS
    bad = list(args)
    bad[6] = P  # dq aliases q
    assert L.ncattn_bwd(*bad, P + 256, need, None) == EINVAL
    bad = list(args)
    bad[7] = bad[8]  # dk == dv
    assert L.ncattn_bwd(*bad, P + 256, need, None) == EINVAL
    bad = list(args)
    bad[14] = -5
    assert L.ncattn_bwd(*bad, P + 256, need, None) == EINVAL


def test_decode_validation_and_workspace(L):
    n_full = L.ncattn_decode_workspace_bytes(64, 8320, 10, 10, 128, -1)
    n_win = L.ncattn_decode_workspace_bytes(64, 8320, 10, 10, 128, 1024)
    assert n_full > n_win > 0
    assert L.ncattn_decode_workspace_bytes(0, 8320, 10, 10, 128, -1) == 0
    # a window reaching every cached key is full causal, up to INT_MAX
    for W in (8319, 8320, 2 ** 31 - 2, 2 ** 31 - 1):
        assert L.ncattn_decode_workspace_bytes(64, 8320, 10, 10, 128, W) == n_full, W
    base = [P, P + 16, P + 32, P + 48, P + 64, P + 80, P + 96, None, 4, 512, 2, 2, 128, -1, 0.0]
    ws = L.ncattn_decode_workspace_bytes(4, 512, 2, 2, 128, -1)
    assert L.ncattn_decode(*base, 1, P + 256, ws, None) == EUNSUP       # fp32 decode
    assert L.ncattn_decode(*base, 0, None, 0, None) == EWS
    bad = list(base)
    bad[5] = P + 82                                                    # seqlens misaligned
    assert L.ncattn_decode(*bad, 0, P + 256, ws, None) == EINVAL
    bad = list(base)
    bad[4] = bad[3]                                                    # k_cache == v_cache
    assert L.ncattn_decode(*bad, 0, P + 256, ws, None) == EINVAL
    bad = list(base)
    bad[12] = 96
    assert L.ncattn_decode(*bad, 0, P + 256, ws, None) == EUNSUP       # head_dim 64 or 128
    bad[12] = 32
    assert L.ncattn_decode(*bad, 0, P + 256, ws, None) == EUNSUP


def test_decode_noalloc_validation(L):
    # the same checks as ncattn_decode, and shapes beyond the scratch are refused
    # on the host, before any device call
    args = [P, P + 16, P + 32, P + 48, P + 64, P + 80, P + 96, None, 4, 512, 2, 2, 128, -1, 0.0]
    assert L.ncattn_decode_noalloc(*args, 1, None) == EUNSUP             # fp32 decode
    bad = list(args)
    bad[4] = bad[3]                                                    # k_cache == v_cache
    assert L.ncattn_decode_noalloc(*bad, 0, None) == EINVAL
    bad = list(args)
    bad[0] = None
    assert L.ncattn_decode_noalloc(*bad, 0, None) == EINVAL
    big = list(args)
    big[8:13] = [64, 16384, 16, 16, 128]                               # 68 MB of partials
    assert L.ncattn_decode_workspace_bytes(64, 16384, 16, 16, 128, -1) > 32 << 20
    assert L.ncattn_decode_noalloc(*big, 0, None) == EWS
    assert b"scratch" in L.ncattn_last_error()
    # the engine-decode batch (64 sequences, T_max 8320, 10 heads) fits the scratch
    assert L.ncattn_decode_workspace_bytes(64, 8320, 10, 10, 128, -1) <= 32 << 20


def test_prefill_validation(L):
    f = L.ncattn_prefill
    def call(q=P, kn=P + 16, vn=P + 32, kc=P + 48, vc=P + 64, lens=P + 80, o=P + 96, lse=None, Tn=8, T_max=64,
             D=128, W=-1, dt=0):
        return f(q, kn, vn, kc, vc, lens, o, lse, 2, Tn, T_max, 2, 2, D, W, 0.0, dt, None)
    assert call(q=None) == EINVAL
    assert call(lens=None) == EINVAL
    assert call(lens=P + 82) == EINVAL
    assert call(lse=P + 2) == EINVAL
    assert call(Tn=0) == EINVAL
    assert call(Tn=65) == EINVAL
    assert call(W=-3) == EINVAL
    assert call(kc=P + 64) == EINVAL          # k_cache == v_cache
    assert call(o=P) == EINVAL                # o aliases q
    assert call(dt=1) == EUNSUP
    assert call(D=96) == EUNSUP


def test_window_sizes_binding_golden():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "window_schedule.json")))
    for c in g["cases"]:
        assert [list(t) for t in nc.window_sizes(c["pattern"], c["n_layer"], c["short"])] == c["expect"]
    with pytest.raises(ValueError):
        nc.window_sizes("SXL", 4, 128)


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    x = torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nc.fwd(x, x, x)


def test_cache_replicate_validation(L):
    f = L.ncattn_cache_replicate
    def call(ks=P, vs=P + 16, sl=P + 32, kd=P + 48, vd=P + 64, dl=P + 80, N=4, T_src=16, T_max=32, KV=2, D=128, dt=0):
        return f(ks, vs, sl, kd, vd, dl, N, T_src, T_max, KV, D, dt, None)
    assert call(ks=None) == EINVAL
    assert call(dl=None) == EINVAL
    assert call(sl=P + 34) == EINVAL          # misaligned length pointer
    assert call(N=0) == EINVAL
    assert call(T_src=0) == EINVAL
    assert call(T_max=15) == EINVAL           # T_src > T_max
    assert call(KV=1, D=4) == EINVAL          # a row of 8 bytes is not a multiple of 16
    assert call(kd=P + 8) == EINVAL           # misaligned cache pointer
    assert call(vd=P + 48) == EINVAL          # k_dst == v_dst
    assert call(kd=P) == EINVAL               # destination aliases a source
    assert call(dt=7) == EINVAL
