"""The bench's work accounting agrees with the oracle's pinned pair count, and its
traffic lookup only reports figures that match the kernel source (CPU only)."""

import os
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 300, 2048, 4096])
@pytest.mark.parametrize("W", [-1, 0, 1, 63, 64, 1024, 2047, 5000])
def test_visible_pairs_matches_oracle(T, W):
    assert bench.visible_pairs(T, W) == oracle.n_visible_pairs(T, W)


def test_decode_bytes_match_the_oracle():
    import numpy as np
    r = np.random.default_rng(3)
    for W in (-1, 0, 1, 100, 1024, 9000):
        lens = [int(x) for x in r.integers(0, 8193, size=64)]
        assert bench.decode_algorithmic_bytes(lens, 10, 10, 128, W) == oracle.decode_bytes(lens, 10, 10, 128, W)


def test_traffic_lookup_requires_matching_source():
    assert bench.measured_traffic("no_such_kernel", "no_such_workload") is None
    h = bench.kernel_source_hash("attn_bwd_bf16.hip")
    assert h == bench.kernel_source_hash("attn_bwd_bf16.hip") and len(h) == 16
    tr = bench.measured_traffic("bwd_dkdv", "gqa_b16_t4096_h12_kv4_d128_bf16")
    assert tr is None or (isinstance(tr, int) and tr > 0)


def test_bench_refuses_more_than_one_gpu():
    """Nothing here uses a second GPU: --gpus N > 1 (or a multi-rank launch)
    exits with a message before touching any device."""
    import subprocess
    for extra_env, argv in (({}, ["--gpus", "2"]), ({"WORLD_SIZE": "8"}, [])):
        env = dict(os.environ, **extra_env)
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                           env=env, timeout=120)
        assert r.returncode == 2 and "one GPU only" in r.stderr, (r.returncode, r.stderr)
