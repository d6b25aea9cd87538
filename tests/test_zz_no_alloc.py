"""The allocation-free decode entry point (ncattn_decode_noalloc, called through
the C ABI with ctypes) gives the same results as ncattn_decode with a workspace:
bit for bit, and within the parity bar of each other, on two calls in a row, the
second on a smaller batch and cache (the per-device scratch keeps the first
call's contents, which the second must not depend on).  It also rejects a shape
whose partials exceed the scratch, and allocates nothing."""

import ctypes
import sys

import pytest
import torch

import transformer_attention_qknorm_amd as nc
from parity_util import check, check_lse, f64
from workloads import decode_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _call_noalloc(q, kn, vn, kc, vc, lens, o, lse, W):
    B, _, H, D = q.shape
    T_max, KV = kc.shape[1], kc.shape[2]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return nc.lib().ncattn_decode_noalloc(_p(q), _p(kn), _p(vn), _p(kc), _p(vc), _p(lens), _p(o), _p(lse), B, T_max,
                                          H, KV, D, W, 0.0, nc.BF16, stream)


def _case(B, H, KV, T_max, lo, hi, W, seed, check_free=True):
    say(f"no-alloc decode B={B} H={H} KV={KV} T_max={T_max} W={W}")
    q, kn, vn, kc, vc, lens = (t.to(DEV) for t in decode_inputs(B, H, KV, 128, lo, hi, T_max, seed=seed, poison=True))
    kc2, vc2 = kc.clone(), vc.clone()
    o_ref, lse_ref = nc.decode(q, kn, vn, kc, vc, lens, window=W, return_lse=True)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    rc = _call_noalloc(q, kn, vn, kc2, vc2, lens, o, lse, W)
    torch.cuda.synchronize()
    assert rc == 0, nc.lib().ncattn_last_error().decode()
    if check_free:  # the first call on a device may let the runtime finish loading the module
        assert torch.cuda.mem_get_info()[0] == free0, "the no-alloc call changed the free device memory"
    check(o, f64(o_ref), "bf16", "o vs ncattn_decode")
    check_lse(lse, f64(lse_ref), "bf16", "lse vs ncattn_decode")
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), "not bit-identical to ncattn_decode"
    for a, b in ((kc2, kc), (vc2, vc)):  # the same cache slots written, NaN poison elsewhere untouched
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_noalloc_decode_matches_decode_twice_then_smaller():
    # the engine-decode shape at full causal (partials 21.6 MB of the 32 MiB), then
    # a smaller batch at a window, in the same process: the second call reuses the
    # scratch the first one filled
    _case(64, 10, 10, 8320, 256, 8192, -1, seed=5, check_free=False)
    _case(64, 10, 10, 8320, 256, 8192, -1, seed=6)
    _case(5, 8, 2, 700, 1, 690, 100, seed=7)


def test_noalloc_decode_rejects_shapes_beyond_the_scratch():
    B, H, KV, T_max = 64, 16, 16, 16384  # partials: 64 * 16 * 128 * 520 B = 68 MB > 32 MiB
    need = nc.lib().ncattn_decode_workspace_bytes(B, T_max, H, KV, 128, -1)
    assert need > nc.DECODE_SCRATCH_BYTES
    q = torch.zeros(B, 1, H, 128, dtype=torch.bfloat16, device=DEV)
    kn = torch.zeros(B, 1, KV, 128, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(B, 2, KV, 128, dtype=torch.bfloat16, device=DEV)  # never read: rejected on the host
    lens = torch.zeros(B, dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    # T_max is what sizes the partials; the cache tensors are not touched
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = nc.lib().ncattn_decode_noalloc(_p(q), _p(kn), _p(kn.clone()), _p(kc), _p(kc.clone()), _p(lens), _p(o), None,
                                        B, T_max, H, KV, 128, -1, 0.0, nc.BF16, stream)
    assert rc == -3 and b"scratch" in nc.lib().ncattn_last_error()
