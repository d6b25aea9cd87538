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


def test_traffic_lookup_requires_matching_source():
    assert bench.measured_traffic("no_such_kernel") is None
    h = bench.kernel_source_hash("attn_bwd_bf16.hip")
    assert h == bench.kernel_source_hash("attn_bwd_bf16.hip") and len(h) == 16
    tr = bench.measured_traffic("bwd_dkdv")
    assert tr is None or (isinstance(tr, int) and tr > 0)
