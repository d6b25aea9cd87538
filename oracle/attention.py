"""Plain CPU float64 oracle: QK-norm, RoPE, causal sliding-window GQA attention
(forward, backward) and single-token decode against a KV cache.

TEST INFRASTRUCTURE ONLY -- imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.  It imports nothing from
the HIP path and shares no code with it.

Every function is the textbook definition, in numpy float64, with no blocking,
online softmax, fusion or reordering.  Sources (page title, section):

* "nanochat Admin & Developer Guide", section 3 "The GPT Model (Internals)":
  rotary embeddings with base 100000, QK-norm (weightless RMSNorm on queries and
  keys) followed by a logit gain of 1.2 split between q and k, grouped-query
  attention (n_kv_head <= n_head), and per-layer sliding windows from a pattern
  string tiled over the layers with the last layer always full, handed to the
  attention call as (left, right) tuples.
* same page, section 6 "Attention: FA3 with SDPA Fallback": the fallback covers
  full-context, single-token decode over the window and chunked windowed
  inference, and does GQA the way SDPA's enable_gqa does (query head h reads
  kv head h // (n_head / n_kv_head)).
* same page, section 7 "The Inference Engine & Tool Use", "KV cache": cache
  laid out (B, T, H, D) per layer, per-sequence int32 cache_seqlens, the new
  token written into the cache in place.
* "nanoGPT Administrator & Developer Guide", section 8 "Developer Internals",
  model.py CausalSelfAttention: scores q.k^T scaled by 1/sqrt(d_k), a lower
  triangular mask, softmax, then times V.
* "nanochat (Python)" feature catalog, entry AI / Model & kernels / Backward
  pass: the backward is autograd of the forward, i.e. its exact gradient.

Readings where the pages are silent:
* RMSNorm eps is an argument (default 1e-6); the norm is per head over head_dim.
* The 1.2 gain is read as a total logit gain, g = sqrt(1.2) on each of q and k;
  ``gain`` is an argument and the workloads use g = 1 (plain weightless RMSNorm).
* RoPE pairs element j with element j + D/2 ("half split"), rotates by +theta,
  theta = pos * base**(-2j/D), pos = pos_offset[b] + t.
* RMSNorm then RoPE (the two commute exactly: RoPE preserves the RMS).
* The window is inclusive: key j is visible to query i iff j <= i and
  (W < 0 or i - j <= W), the (left, right) = (W, 0) convention.
* LSE is the natural-log logsumexp of the scaled, visible scores, laid out
  [B][H][T]; no dropout, no score soft-cap, no document mask.

Parity: all functions are pinned by tests that do not call back into them for
the expected value (torch's float64 SDPA and autograd, finite differences,
closed forms, brute-force counts, complex-multiplication RoPE, golden fixtures);
see tests/test_oracle_*.py.  The RoPE pairing/sign is a reading, not fixed by the
pages, so its agreement with the pages' own project is "parity unpinned".
"""

from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# QK-norm and RoPE  ("nanochat Admin & Developer Guide", section 3)
# --------------------------------------------------------------------------

def rms_norm(x, eps=1e-6, gain=1.0):
    """Weightless RMSNorm over the last axis: g * x / sqrt(mean(x^2) + eps).

    Section 3 of the nanochat Admin & Developer Guide: RMSNorm has no learnable
    parameters; queries and keys are RMS-normalised per head.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return gain * x / np.sqrt(ms + eps)


def rms_rstd(x, eps=1e-6):
    """1 / sqrt(mean(x^2) + eps) of each row (last axis), the reciprocal RMS that
    weightless RMSNorm divides by (section 3 of the nanochat Admin & Developer
    Guide); the per-row statistic the QK-norm forward can store for its backward.
    Returns shape x.shape[:-1]."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)


def rope_angles(pos, head_dim, base):
    """theta[p, j] = pos[p] * base ** (-2 j / head_dim), j < head_dim / 2 (float64)."""
    pos = np.asarray(pos, dtype=np.float64)
    j = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * j / head_dim)
    return pos[..., None] * inv_freq


def apply_rope(x, pos, base):
    """Rotate pairs (x_j, x_{j+D/2}) of every row by +theta(pos, j).

    ``x`` is [B][T][heads][D]; ``pos`` is [B][T] (absolute position of each token).
    Section 3 of the nanochat Admin & Developer Guide: rotary positional
    embeddings, no learned positions.  Pairing and sign are the reading stated in
    the module header.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    theta = rope_angles(pos, D, base)[:, :, None, :]          # [B][T][1][D/2]
    c, s = np.cos(theta), np.sin(theta)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def qknorm_rope(q, k, pos_offset=None, base=100000.0, eps=1e-6, gain=1.0):
    """QK-norm then RoPE on q [B][T][H][D] and k [B][T][KV][D]; v is untouched.

    Position of token t of sequence b is pos_offset[b] + t (0-based; the decode
    case passes pos_offset = cache_seqlens, one token per sequence).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, T = q.shape[0], q.shape[1]
    off = np.zeros(B) if pos_offset is None else np.asarray(pos_offset, dtype=np.float64)
    pos = off[:, None] + np.arange(T, dtype=np.float64)[None, :]
    qn = apply_rope(rms_norm(q, eps, gain), pos, base)
    kn = apply_rope(rms_norm(k, eps, gain), pos, base)
    return qn, kn


def rope_inverse(y, pos, base):
    """The transpose of apply_rope's rotation (its inverse): every pair
    (y_j, y_{j+D/2}) rotated by -theta(pos, j).  This is how a gradient flows
    back through RoPE."""
    y = np.asarray(y, dtype=np.float64)
    D = y.shape[-1]
    half = D // 2
    theta = rope_angles(pos, D, base)[:, :, None, :]
    c, s = np.cos(theta), np.sin(theta)
    a, b = y[..., :half], y[..., half:]
    return np.concatenate([a * c + b * s, -a * s + b * c], axis=-1)


def rms_norm_bwd(x, dn, eps=1e-6, gain=1.0):
    """Gradient of rms_norm at x, given dn = dL/dn for n = g x / r with
    r = sqrt(mean(x^2) + eps):  dL/dx = (g / r) (dn - x sum(dn x) / (D r^2)),
    the derivative of n_i with respect to x_k being g (delta_ik / r - x_i x_k / (D r^3))."""
    x = np.asarray(x, dtype=np.float64)
    dn = np.asarray(dn, dtype=np.float64)
    D = x.shape[-1]
    r2 = np.mean(x * x, axis=-1, keepdims=True) + eps
    r = np.sqrt(r2)
    dot = np.sum(dn * x, axis=-1, keepdims=True)
    return gain / r * (dn - x * dot / (D * r2))


def qknorm_rope_bwd(q, k, dq_out, dk_out, pos_offset=None, base=100000.0, eps=1e-6, gain=1.0):
    """Gradient of qknorm_rope with respect to its inputs q and k, given the
    gradients dq_out, dk_out of its outputs: back through RoPE (rope_inverse),
    then through the RMSNorm (rms_norm_bwd), the chain rule in the forward's
    reverse order ("nanochat (Python)" catalog, Backward pass: autograd of the
    forward; the forward is section 3 of the nanochat Admin & Developer Guide)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, T = q.shape[0], q.shape[1]
    off = np.zeros(B) if pos_offset is None else np.asarray(pos_offset, dtype=np.float64)
    pos = off[:, None] + np.arange(T, dtype=np.float64)[None, :]
    dq = rms_norm_bwd(q, rope_inverse(dq_out, pos, base), eps, gain)
    dk = rms_norm_bwd(k, rope_inverse(dk_out, pos, base), eps, gain)
    return dq, dk


# --------------------------------------------------------------------------
# Attention forward / backward
# ("nanoGPT Administrator & Developer Guide" section 8 CausalSelfAttention;
#  "nanochat Admin & Developer Guide" sections 3 and 6)
# --------------------------------------------------------------------------

def visible_mask(T, window_left):
    """vis[i, j] = (j <= i) and (W < 0 or i - j <= W): causal, inclusive window."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    vis = j <= i
    if window_left >= 0:
        vis = vis & (i - j <= window_left)
    return vis


def n_visible_pairs(T, window_left):
    """Number of visible (query, key) pairs in one head: sum_i min(i + 1, W + 1)."""
    i = np.arange(T, dtype=np.int64)
    cnt = i + 1
    if window_left >= 0:
        cnt = np.minimum(cnt, window_left + 1)
    return int(cnt.sum())


def _scale(head_dim, softmax_scale):
    return 1.0 / np.sqrt(head_dim) if (softmax_scale is None or softmax_scale <= 0) else float(softmax_scale)


def attn_fwd(q, k, v, window_left=-1, softmax_scale=None):
    """O = softmax(scale * Q K^T + mask) V and LSE per query row.

    q [B][T][H][D], k/v [B][T][KV][D] -> o [B][T][H][D], lse [B][H][T] (natural log).
    Query head h reads kv head h // (H / KV).  Built per (b, h) as a dense T x T
    score matrix with the visibility mask and a textbook softmax.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, D = q.shape
    KV = k.shape[2]
    G = H // KV
    scale = _scale(D, softmax_scale)
    vis = visible_mask(T, window_left)
    o = np.empty((B, T, H, D))
    lse = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            kh = h // G
            s = scale * (q[b, :, h, :] @ k[b, :, kh, :].T)
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            p = e / z
            o[b, :, h, :] = p @ v[b, :, kh, :]
            lse[b, h, :] = (m + np.log(z))[:, 0]
    return o, lse


def attn_bwd(q, k, v, dout, window_left=-1, softmax_scale=None, o=None):
    """Exact gradient of sum(O * dO) with respect to q, k and v.

    Chain rule through the forward above: dV = P^T dO, dP = dO V^T,
    dS = P * (dP - Delta), dQ = scale dS K, dK = scale dS^T Q.  dK and dV of a
    kv head are summed over the query heads of its group.  Returns dq
    [B][T][H][D], dk/dv [B][T][KV][D].

    Delta is the softmax-Jacobian term.  With o=None it is sum_j P dP per row
    (the exact gradient).  A backward that is handed the forward's output, as
    the attention backward of the FA3 interface is ("nanochat Admin & Developer
    Guide", section 6: the flash_attn calls match the Flash Attention 3 API, whose
    backward takes the forward's out and softmax_lse), forms it as
    Delta_i = sum_d dO_i o_i from that output instead; ``o`` [B][T][H][D] is that
    given output (the two agree when o is the exact O).  dV does not depend on
    Delta.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    if o is not None:
        o = np.asarray(o, dtype=np.float64)
    B, T, H, D = q.shape
    KV = k.shape[2]
    G = H // KV
    scale = _scale(D, softmax_scale)
    vis = visible_mask(T, window_left)
    dq = np.zeros((B, T, H, D))
    dk = np.zeros((B, T, KV, D))
    dv = np.zeros((B, T, KV, D))
    for b in range(B):
        for h in range(H):
            kh = h // G
            s = scale * (q[b, :, h, :] @ k[b, :, kh, :].T)
            s = np.where(vis, s, -np.inf)
            e = np.exp(s - s.max(axis=1, keepdims=True))
            p = e / e.sum(axis=1, keepdims=True)
            do = dout[b, :, h, :]
            dv[b, :, kh, :] += p.T @ do
            dp = do @ v[b, :, kh, :].T
            if o is None:
                delta = (p * dp).sum(axis=1, keepdims=True)
            else:
                delta = (do * o[b, :, h, :]).sum(axis=1, keepdims=True)
            ds = p * (dp - delta)
            dq[b, :, h, :] = scale * (ds @ k[b, :, kh, :])
            dk[b, :, kh, :] += scale * (ds.T @ q[b, :, h, :])
    return dq, dk, dv


# --------------------------------------------------------------------------
# Decode against a KV cache ("nanochat Admin & Developer Guide", sections 6, 7)
# --------------------------------------------------------------------------

def decode(q, k_new, v_new, k_cache, v_cache, cache_seqlens, window_left=-1, softmax_scale=None):
    """Single-token decode.

    For each sequence b with s = cache_seqlens[b]: write k_new/v_new into cache
    slot s, then attend query q[b] (position s) over keys [max(0, s - W), s]
    (all of [0, s] when W < 0).  q [B][1][H][D], k_new/v_new [B][1][KV][D],
    caches [B][T_max][KV][D].  Returns (o [B][1][H][D], lse [B][H],
    k_cache', v_cache') where the caches are updated copies.
    """
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    B, _, H, D = q.shape
    KV = k_new.shape[2]
    G = H // KV
    scale = _scale(D, softmax_scale)
    o = np.empty((B, 1, H, D))
    lse = np.empty((B, H))
    for b in range(B):
        s_b = int(cache_seqlens[b])
        kc[b, s_b] = k_new[b, 0]
        vc[b, s_b] = v_new[b, 0]
        lo = 0 if window_left < 0 else max(0, s_b - window_left)
        for h in range(H):
            kh = h // G
            keys = kc[b, lo:s_b + 1, kh, :]
            vals = vc[b, lo:s_b + 1, kh, :]
            sc = scale * (keys @ q[b, 0, h, :])
            m = sc.max()
            e = np.exp(sc - m)
            z = e.sum()
            o[b, 0, h, :] = (e / z) @ vals
            lse[b, h] = m + np.log(z)
    return o, lse, kc, vc


def prefill(q, k_new, v_new, k_cache, v_cache, cache_seqlens, window_left=-1, softmax_scale=None):
    """Chunked prefill against the KV cache (multi-token decode).

    For each sequence b with s = cache_seqlens[b]: write the chunk's keys and
    values k_new[b, i], v_new[b, i] into cache slots s + i, then attend query
    q[b, i] (position s + i) over keys [max(0, s + i - W), s + i] of the updated
    cache ("nanochat Admin & Developer Guide", section 6: chunked inference
    against the cache through the fallback path; section 7: the cache updated in
    place at each sequence's position).  q [B][Tn][H][D], k_new/v_new
    [B][Tn][KV][D], caches [B][T_max][KV][D].  Returns (o [B][Tn][H][D],
    lse [B][H][Tn], k_cache', v_cache') with the caches as updated copies.
    """
    q = np.asarray(q, dtype=np.float64)
    k_new = np.asarray(k_new, dtype=np.float64)
    v_new = np.asarray(v_new, dtype=np.float64)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    B, Tn, H, D = q.shape
    KV = k_new.shape[2]
    G = H // KV
    scale = _scale(D, softmax_scale)
    o = np.empty((B, Tn, H, D))
    lse = np.empty((B, H, Tn))
    for b in range(B):
        s_b = int(cache_seqlens[b])
        kc[b, s_b:s_b + Tn] = k_new[b]
        vc[b, s_b:s_b + Tn] = v_new[b]
        for i in range(Tn):
            p = s_b + i
            lo = 0 if window_left < 0 else max(0, p - window_left)
            for h in range(H):
                kh = h // G
                sc = scale * (kc[b, lo:p + 1, kh, :] @ q[b, i, h, :])
                m = sc.max()
                e = np.exp(sc - m)
                z = e.sum()
                o[b, i, h, :] = (e / z) @ vc[b, lo:p + 1, kh, :]
                lse[b, h, i] = m + np.log(z)
    return o, lse, kc, vc


def cache_replicate(k_src, v_src, src_seqlen, k_dst, v_dst):
    """Replication of a batch-1 prefill cache into a batch-N decode cache.

    With s = src_seqlen: rows [0, s) of the single source sequence are copied
    into rows [0, s) of every destination sequence, and every destination length
    becomes s ("nanochat Admin & Developer Guide", section 7, "KV cache": the
    prompt is prefilled once at batch 1, then its cache is copied into each row
    of the cache the samples decode from).  k_src, v_src [1][T_src][KV][D],
    k_dst, v_dst [N][T_max][KV][D]; destination rows t >= s keep their contents.
    A length outside [0, T_src] (an invalid source) copies nothing and marks
    every destination length -1.  The copy keeps the arrays' own dtype: it moves
    values, it computes none.  Returns (k_dst', v_dst', dst_seqlens int32 [N]).
    """
    kd = np.array(k_dst, copy=True)
    vd = np.array(v_dst, copy=True)
    N = kd.shape[0]
    T_src = np.shape(k_src)[1]
    s = int(src_seqlen)
    if not 0 <= s <= T_src:
        return kd, vd, np.full(N, -1, dtype=np.int32)
    for n in range(N):
        kd[n, :s] = k_src[0, :s]
        vd[n, :s] = v_src[0, :s]
    return kd, vd, np.full(N, s, dtype=np.int32)


# --------------------------------------------------------------------------
# Window schedule and work accounting
# --------------------------------------------------------------------------

def window_sizes(pattern, n_layer, short_window, long_window=-1):
    """Per-layer (left, right) windows: ``pattern`` tiled over the layers,
    'S' -> short_window, 'L' -> long_window (-1 = unbounded), final layer 'L'.

    "nanochat Admin & Developer Guide", section 3, "Sliding-window attention".
    """
    pattern = pattern.upper()
    if not pattern or any(c not in "SL" for c in pattern):
        raise ValueError("window pattern must be a non-empty string of 'S' and 'L'")
    out = []
    for layer in range(n_layer):
        c = pattern[layer % len(pattern)]
        if layer == n_layer - 1:
            c = "L"
        out.append((short_window if c == "S" else long_window, 0))
    return out


def attn_flops(B, T, H, D, window_left):
    """Algorithmic (unmasked) FLOPs of one layer: (fwd, bwd) = (4 D, 8 D) per
    visible pair per head, the 12*H*Q per (query, key) convention of the MFU
    formula in "nanoGPT Administrator & Developer Guide" section 6, with T
    replaced by the visible keys as nanochat's estimate_flops does for windows
    ("nanochat Admin & Developer Guide", section 3)."""
    pairs = n_visible_pairs(T, window_left) * B * H
    return 4 * D * pairs, 8 * D * pairs


def decode_bytes(cache_seqlens, H, KV, D, window_left=-1, elem_bytes=2):
    """Minimum HBM bytes of one decode call: read the visible cached K and V rows
    (the newest key comes from k_new/v_new), read q, k_new, v_new, write o and the
    new cache slot."""
    n_cached = 0
    for s in np.asarray(cache_seqlens, dtype=np.int64):
        lo = 0 if window_left < 0 else max(0, int(s) - window_left)
        n_cached += int(s) - lo
    B = len(cache_seqlens)
    row = KV * D * elem_bytes
    return (n_cached * 2 * row            # visible cached K and V
            + B * 2 * row                 # k_new, v_new read
            + B * 2 * row                 # cache slot written
            + B * 2 * H * D * elem_bytes) # q read, o written
