"""CPU fp64 oracle for the QK-norm + RoPE + causal sliding-window GQA attention path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, links or runs
it, and it imports nothing from the product path.

Every function here is the plain definition of what the path computes, written
out in numpy float64 without blocking, fusion or reordering, so that it can be
checked against the pages by eye.  See ``oracle/attention.py`` for the functions
and the passages each one follows.

Parity status (which functions are pinned to something other than themselves is
listed in ``oracle/attention.py``'s header): every function is pinned; the RoPE
pairing/sign convention is a reading of the pages (they do not fix it), so parity
*against the pages' own project* for that convention is unpinned, while parity of
the kernels against this oracle is pinned.
"""

from .attention import (  # noqa: F401
    rms_norm,
    rms_rstd,
    rope_angles,
    apply_rope,
    qknorm_rope,
    rope_inverse,
    rms_norm_bwd,
    qknorm_rope_bwd,
    visible_mask,
    n_visible_pairs,
    attn_fwd,
    attn_bwd,
    decode,
    prefill,
    cache_replicate,
    window_sizes,
    attn_flops,
    decode_bytes,
)
