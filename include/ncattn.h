/*
 * ncattn -- QK-norm + RoPE + causal sliding-window grouped-query attention
 * (forward, backward, single-token decode) for AMD Instinct MI355X (gfx950).
 *
 * What is computed (page titles and sections of the sources):
 *   - "nanochat Admin & Developer Guide", section 3 "The GPT Model (Internals)":
 *     rotary embeddings (base 100000 there), QK-norm = weightless RMSNorm of q and
 *     k (optionally followed by a logit gain), grouped-query attention
 *     (n_kv_head <= n_head), per-layer sliding windows given as (left, right).
 *   - same page, section 6 "Attention: FA3 with SDPA Fallback": full-context
 *     training attention, single-token decode over the window, GQA.
 *   - same page, section 7 "The Inference Engine & Tool Use", "KV cache": the
 *     cache is (B, T, H, D) per layer with per-sequence int32 cache_seqlens and
 *     the new token is written into it in place.
 *   - "nanoGPT Administrator & Developer Guide", section 8, model.py
 *     CausalSelfAttention: softmax(q k^T / sqrt(d_k) + causal mask) v.
 *   - "nanochat (Python)" catalog, AI / Model & kernels / Backward pass: the
 *     backward is the exact gradient (autograd) of that forward.
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller; tensors are
 *     contiguous and row-major in the layouts given per argument, and 16-byte
 *     aligned.  bf16 is IEEE bfloat16 (stored as uint16), f32 is IEEE float.
 *   - Calls enqueue kernels on `stream` (a hipStream_t; NULL = the default
 *     stream) and return without synchronising.  The library never allocates
 *     device memory: scratch space is passed in as `workspace`.
 *   - Key j is visible to query i iff j <= i and (window_left < 0 or
 *     i - j <= window_left): the inclusive (left, right) = (W, 0) convention.
 *     window_right must be 0.
 *   - softmax_scale <= 0 selects 1 / sqrt(head_dim).
 *   - Query head h reads kv head h / (n_head / n_kv_head).
 *   - Return value: NCATTN_OK, or a negative ncattn_status_t.  Arguments are
 *     validated on the host before anything is launched; on error nothing is
 *     enqueued and ncattn_last_error() (thread-local) describes the problem.
 *     No C++ exception crosses this interface.
 *   - Outputs must not alias inputs, except where a call says it works in place.
 *   - Apart from the thread-local error string and the per-device scratch of
 *     ncattn_decode_noalloc (below) the library keeps no mutable global state;
 *     calls on different streams may run concurrently, except that
 *     ncattn_decode_noalloc calls on one device must not overlap.
 *
 * Supported: dtype NCATTN_BF16 (fp32 accumulation, bf16 MFMA contractions) with
 * head_dim 64 or 128 (nanochat's --head-dim 128, "nanochat User Guide", section
 * 13; GPT-2's n_embd / n_head = 768 / 12 = 64, "nanoGPT Administrator & Developer
 * Guide", sections 3 and 6); dtype NCATTN_F32 (fp32 throughout) with head_dim 64 or 128.  Decode and
 * prefill are bf16 only.  Anything else returns NCATTN_EUNSUPPORTED.
 */
#ifndef NCATTN_H
#define NCATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { NCATTN_BF16 = 0, NCATTN_F32 = 1 } ncattn_dtype_t;

typedef enum {
  NCATTN_OK = 0,
  NCATTN_EINVAL = -1,       /* bad argument (NULL, non-positive size, misaligned, ...) */
  NCATTN_EUNSUPPORTED = -2, /* valid but not implemented (head_dim, dtype combination) */
  NCATTN_EWORKSPACE = -3,   /* workspace missing or smaller than *_workspace_bytes()   */
  NCATTN_EHIP = -4          /* the HIP runtime reported an error at launch             */
} ncattn_status_t;

/*
 * QK-norm + RoPE, in place ("nanochat Admin & Developer Guide", section 3).
 * For every row x (one head of one token) of q [B][T][n_head][head_dim] and of
 * k [B][T][n_kv_head][head_dim]:
 *     x <- qk_gain * x / sqrt(mean_d(x_d^2) + eps)
 *     (x_j, x_{j+D/2}) <- (x_j cos a - x_{j+D/2} sin a, x_j sin a + x_{j+D/2} cos a),
 *     a = pos * rope_base^(-2j/D), pos = pos_offset[b] + t   (j < D/2)
 * pos_offset: device int32 [B], or NULL for 0 (decode passes cache_seqlens).
 * Arithmetic is fp32 with the angle reduced in fp64; storage stays in `dtype`.
 * v is not touched.  q and k are read and written in place.
 */
int ncattn_qknorm_rope(void *q, void *k, int B, int T, int n_head, int n_kv_head, int head_dim,
                       const int32_t *pos_offset, float rope_base, float eps, float qk_gain,
                       int dtype, void *stream);

/*
 * ncattn_qknorm_rope that also stores each row's 1/r = 1/sqrt(mean_d(x_d^2) + eps)
 * in fp32 (the statistic a backward needs besides the outputs, so that the raw
 * q and k need not be kept; "nanochat Admin & Developer Guide", section 3).
 *   rstd [B][T][n_head + n_kv_head] fp32, written: q rows at [b][t][h], k rows at
 *   [b][t][n_head + kv head]; 4-byte aligned, not NULL.
 *   Everything else as ncattn_qknorm_rope (same q, k results, bit for bit).
 */
int ncattn_qknorm_rope_rstd(void *q, void *k, float *rstd, int B, int T, int n_head, int n_kv_head,
                            int head_dim, const int32_t *pos_offset, float rope_base, float eps, float qk_gain,
                            int dtype, void *stream);

/*
 * Backward of ncattn_qknorm_rope ("nanochat (Python)" catalog, Backward pass:
 * autograd of the forward; the forward is section 3 of the nanochat Admin &
 * Developer Guide).  With n = g x / r, r = sqrt(mean_d(x_d^2) + eps), y = R(pos) n:
 *     dn = R(pos)^T dy                 (each pair rotated by -a)
 *     dx = (g / r) (dn - x sum_d(dn_d x_d) / (D r^2))
 *   dq [B][T][n_head][head_dim], dk [B][T][n_kv_head][head_dim]: on entry the
 *     gradients dy of the forward's outputs, on return the gradients dx of its
 *     inputs (in place, dtype).
 *   q, k: the forward's inputs (before normalisation), read only; they must not
 *     overlap dq / dk.
 *   Other arguments, arithmetic, validation and status codes as ncattn_qknorm_rope.
 */
int ncattn_qknorm_rope_bwd(void *dq, void *dk, const void *q, const void *k, int B, int T, int n_head,
                           int n_kv_head, int head_dim, const int32_t *pos_offset, float rope_base,
                           float eps, float qk_gain, int dtype, void *stream);

/*
 * Attention forward ("nanoGPT Administrator & Developer Guide" section 8;
 * "nanochat Admin & Developer Guide" sections 3 and 6).
 *   q [B][T][n_head][D], k, v [B][T][n_kv_head][D]          (dtype)
 *   o [B][T][n_head][D]                                      (dtype, written)
 *   lse [B][n_head][T] fp32, natural-log logsumexp of the scaled visible
 *   scores of each query row (written; every row has at least its own key).
 * Tiles of keys outside every row's window are skipped.
 */
int ncattn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int T, int n_head, int n_kv_head, int head_dim,
               int window_left, int window_right, float softmax_scale, int dtype, void *stream);

/*
 * Attention forward with fp8 inputs ("nanochat Admin & Developer Guide", section
 * 6, Attention: FA3 with SDPA fallback, which runs attention in bf16 or fp8).
 *   q [B][T][n_head][128], k, v [B][T][n_kv_head][128]: OCP e4m3 bytes (FP8 E4M3FN:
 *     1 sign, 4 exponent bits with bias 7, 3 fraction bits, no infinities, 0x7f /
 *     0xff NaN); the value an element stands for is its byte's value times the
 *     tensor's descale (q_descale, k_descale, v_descale: finite, > 0).
 *   o [B][T][n_head][128] bf16 (written); lse [B][n_head][T] fp32 as ncattn_fwd's.
 *   Computes ncattn_fwd's function of those values (window and softmax_scale as
 *   there).  P enters the P V contraction rounded to e4m3 (as 2^8 P against an
 *   exponent reference within 0.8, base 2, of the running row maximum, so below
 *   e4m3's 448), so o carries a relative error of up to 2^-4 per probability:
 *   |o_id - o_exact,id| <= 2^-4 sum_j P_ij |v_jd| + n 2^-18 max_j |v_jd| + the
 *   bf16 rounding of o, n the row's visible keys.
 * head_dim must be 128 (NCATTN_EUNSUPPORTED otherwise); pointers 16-byte
 * aligned; o must not alias an input (NCATTN_EINVAL).
 */
int ncattn_fwd_fp8(const void *q, const void *k, const void *v, float q_descale, float k_descale, float v_descale,
                   void *o, float *lse, int B, int T, int n_head, int n_kv_head, int head_dim, int window_left,
                   int window_right, float softmax_scale, void *stream);

/*
 * QK-norm + RoPE fused into the attention forward ("nanochat Admin & Developer
 * Guide", section 3: q and k are RMS-normalised and rotated before attention;
 * sections 3 and 6 for the attention).  Exactly ncattn_qknorm_rope(q, k, ...)
 * followed by ncattn_fwd(q, k, v, ...) with the same arguments: q and k are
 * normalised and rotated IN PLACE (the backward needs them), then o and lse are
 * computed from them.  For bf16 the query rows are normalised and rotated in the
 * forward's prologue (each row once, by the workgroup that attends from it) and k
 * by a separate pass, which saves the separate read and write of q; for fp32 the
 * two calls run one after the other.
 *   q [B][T][n_head][D], k [B][T][n_kv_head][D]: raw on entry, normalised and
 *   rotated on return; v, o, lse as ncattn_fwd; rstd NULL, or each row's 1/r as
 *   ncattn_qknorm_rope_rstd writes it; pos_offset, rope_base, eps and qk_gain as
 *   ncattn_qknorm_rope; window and scale as ncattn_fwd.  o and v must not alias
 *   q, k or each other.  Validation and status codes as the two calls.
 */
int ncattn_fwd_qknorm_rope(void *q, void *k, const void *v, void *o, float *lse, float *rstd, int B, int T,
                           int n_head, int n_kv_head, int head_dim, const int32_t *pos_offset, float rope_base,
                           float eps, float qk_gain, int window_left, int window_right, float softmax_scale,
                           int dtype, void *stream);

/*
 * Bytes of workspace ncattn_bwd needs for this shape: the per-row fp32
 * D_i = sum_d dO_i O_i (for bf16 stored negated, next to a second row array of
 * LSE_i log2 e), i.e. 4 (fp32) or 8 (bf16) bytes per (b, head, query row), each
 * array padded to 256 bytes.  Linear in T for every window.  0 for invalid sizes.
 */
size_t ncattn_bwd_workspace_bytes(int B, int T, int n_head, int n_kv_head, int head_dim, int window_left,
                                  int dtype);

/*
 * Attention backward: the exact gradient of sum(O * dO) ("nanochat (Python)"
 * catalog, Backward pass = autograd of the forward).
 *   inputs q, k, v, o (as from ncattn_fwd), lse [B][n_head][T] fp32 from
 *   ncattn_fwd, dout [B][T][n_head][D]; outputs dq [B][T][n_head][D],
 *   dk, dv [B][T][n_kv_head][D] (dtype; fp32 accumulation).  dk and dv of a kv
 *   head are summed over the query heads of its group.  Deterministic: no
 *   atomics, the same inputs give the same bits.  Delta_i = sum_d dO_i o_i is
 *   formed from the o passed in (the forward's output, as stored), as an FA3-style
 *   backward does.  For bf16 the probabilities P and dS = P (dP - Delta) enter the
 *   dV, dK and dQ products as bf16 hi + lo pairs (fp32 precision), so only the final
 *   rounding of dq, dk, dv to bf16 is lost.
 *   workspace: device memory of at least ncattn_bwd_workspace_bytes(...) bytes,
 *   overwritten.
 */
int ncattn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
               const void *dout, void *dq, void *dk, void *dv,
               int B, int T, int n_head, int n_kv_head, int head_dim,
               int window_left, int window_right, float softmax_scale, int dtype,
               void *workspace, size_t workspace_bytes, void *stream);

/*
 * The three stages of ncattn_bwd, callable one at a time with the same
 * arguments and checks: ncattn_bwd_preprocess writes D_i = sum_d dO_i O_i (and,
 * for bf16, LSE_i log2 e) into the workspace, ncattn_bwd_dkdv then writes dk and
 * dv, ncattn_bwd_dq writes dq; the last two only read the workspace and may run
 * in either order.  Enqueuing the three in this order on one stream, with one
 * workspace, is exactly ncattn_bwd.  Useful for timing each stage.
 */
int ncattn_bwd_preprocess(const void *q, const void *k, const void *v, const void *o, const float *lse,
                          const void *dout, void *dq, void *dk, void *dv,
                          int B, int T, int n_head, int n_kv_head, int head_dim,
                          int window_left, int window_right, float softmax_scale, int dtype,
                          void *workspace, size_t workspace_bytes, void *stream);
int ncattn_bwd_dkdv(const void *q, const void *k, const void *v, const void *o, const float *lse,
                    const void *dout, void *dq, void *dk, void *dv,
                    int B, int T, int n_head, int n_kv_head, int head_dim,
                    int window_left, int window_right, float softmax_scale, int dtype,
                    void *workspace, size_t workspace_bytes, void *stream);
int ncattn_bwd_dq(const void *q, const void *k, const void *v, const void *o, const float *lse,
                  const void *dout, void *dq, void *dk, void *dv,
                  int B, int T, int n_head, int n_kv_head, int head_dim,
                  int window_left, int window_right, float softmax_scale, int dtype,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * The backward of QK-norm + RoPE followed by attention, in one call: the
 * attention backward of ncattn_bwd whose dq and dk are carried back through
 * QK-norm + RoPE ("nanochat Admin & Developer Guide", section 3: weightless
 * RMSNorm of q and k, then rotary embedding; "nanochat (Python)" catalog,
 * Backward pass: the chain rule through that forward) before they are stored.
 * With y = R(pos) g x / r the forward's output row:
 *     dx = (g / r) R(pos)^T (dy - y sum_d(dy_d y_d) / (g^2 D))
 * which is ncattn_qknorm_rope_bwd's dx written with y and 1/r in place of x.
 *   q, k: the post-norm rows the forward attended with (ncattn_qknorm_rope_rstd's
 *   or ncattn_fwd_qknorm_rope's output); rstd: their 1/r as those calls store it
 *   ([B][T][n_head + n_kv_head] fp32); pos_offset, rope_base, qk_gain as given to
 *   the forward; the rest as ncattn_bwd.  The raw q and k are not needed.
 *   Outputs: dq = d/dq_raw, dk = d/dk_raw (dtype), dv as ncattn_bwd.  For bf16
 *   the norm's backward is applied to the fp32 gradients in the dQ and dK/dV
 *   kernels' epilogues, before the one rounding to bf16, and dq, dk of the
 *   post-norm rows are never written to memory; for fp32 (head_dim 64 or 128)
 *   ncattn_bwd runs, then the norm's backward in place.  dq, dk, dv must not
 *   alias any input.  workspace: ncattn_bwd_workspace_bytes(...) bytes.
 */
int ncattn_bwd_qknorm_rope(const void *q, const void *k, const void *v, const void *o, const float *lse,
                           const void *dout, const float *rstd, const int32_t *pos_offset, float rope_base,
                           float qk_gain, void *dq, void *dk, void *dv, int B, int T, int n_head, int n_kv_head,
                           int head_dim, int window_left, int window_right, float softmax_scale, int dtype,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace ncattn_decode needs (split-KV partial results). */
size_t ncattn_decode_workspace_bytes(int B, int T_max, int n_head, int n_kv_head, int head_dim,
                                     int window_left);

/*
 * Single-token decode against a KV cache ("nanochat Admin & Developer Guide",
 * sections 6 and 7).  For every sequence b with s = cache_seqlens[b]:
 *   1. k_new[b], v_new[b] are written into cache slot s (in place);
 *   2. o[b] = softmax(scale * q[b] . K[j]) V[j] over j in [max(0, s - W), s]
 *      (all of [0, s] when window_left < 0), key s being the new one.
 *   q [B][1][n_head][D], k_new, v_new [B][1][n_kv_head][D],
 *   k_cache, v_cache [B][T_max][n_kv_head][D] (bf16), cache_seqlens device
 *   int32 [B] (NOT advanced: the caller owns the position),
 *   o [B][1][n_head][D] bf16, lse [B][n_head] fp32 or NULL.
 *   Precondition 0 <= cache_seqlens[b] < T_max (not checkable on the host
 *   without a sync): a row that breaks it is skipped, its cache is left
 *   untouched and o[b] (and lse[b]) are set to NaN.
 *   workspace: at least ncattn_decode_workspace_bytes(...) bytes, overwritten.
 */
int ncattn_decode(const void *q, const void *k_new, const void *v_new,
                  void *k_cache, void *v_cache, const int32_t *cache_seqlens,
                  void *o, float *lse,
                  int B, int T_max, int n_head, int n_kv_head, int head_dim,
                  int window_left, float softmax_scale, int dtype,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * ncattn_decode without a workspace argument, for callers that cannot allocate
 * device memory: code recorded under HIP graph capture, serving loops that must
 * not call the allocator, harnesses that forbid allocation.  The split-KV partials
 * go to a file-scope device array of NCATTN_DECODE_SCRATCH_BYTES bytes, of which
 * every device the library runs on holds one copy until the process ends (its
 * address is looked up once per device, on the first call with that device
 * current).  The call allocates nothing and needs no zeroed memory.
 *   Arguments, semantics, validation and status codes as ncattn_decode (minus
 *   the workspace); the current device must be the one `stream` belongs to.
 *   A shape whose partials need more than NCATTN_DECODE_SCRATCH_BYTES
 *   (ncattn_decode_workspace_bytes() > the limit: about B * n_head *
 *   ceil(min(T_max, window_left + 1) / 128) * (head_dim + 2) * 4 bytes) returns
 *   NCATTN_EWORKSPACE and enqueues nothing.
 *   Every call on one device shares that device's array: two calls that overlap
 *   in time on one device (different streams, or threads) race and give wrong
 *   results; calls in order on one stream are safe.
 */
#define NCATTN_DECODE_SCRATCH_BYTES (32u << 20)
int ncattn_decode_noalloc(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                          const int32_t *cache_seqlens, void *o, float *lse, int B, int T_max, int n_head,
                          int n_kv_head, int head_dim, int window_left, float softmax_scale, int dtype,
                          void *stream);

/*
 * Chunked prefill against a KV cache (multi-token decode; "nanochat Admin &
 * Developer Guide", section 6: chunked inference against the cache; section 7:
 * the cache updated in place).  For every sequence b with s = cache_seqlens[b]:
 *   1. k_new[b, i], v_new[b, i] are written into cache rows s + i (in place);
 *   2. o[b, i] = softmax(scale * q[b, i] . K[j]) V[j] over
 *      j in [max(0, s + i - W), s + i] (all of [0, s + i] when window_left < 0).
 *   q [B][Tn][n_head][D], k_new, v_new [B][Tn][n_kv_head][D],
 *   k_cache, v_cache [B][T_max][n_kv_head][D] (bf16), cache_seqlens device
 *   int32 [B] (NOT advanced: the caller owns the position),
 *   o [B][Tn][n_head][D] bf16, lse [B][n_head][Tn] fp32 or NULL.
 *   Precondition 0 <= cache_seqlens[b] <= T_max - Tn (not checkable on the host
 *   without a sync): a sequence that breaks it is skipped, its cache is left
 *   untouched and its rows of o (and lse) are NaN.
 *   Supported: bf16, head_dim 64 or 128; no workspace.
 */
int ncattn_prefill(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                   const int32_t *cache_seqlens, void *o, float *lse, int B, int Tn, int T_max,
                   int n_head, int n_kv_head, int head_dim, int window_left, float softmax_scale,
                   int dtype, void *stream);

/*
 * Replication of a batch-1 prefill cache into a batch-N decode cache ("nanochat
 * Admin & Developer Guide", section 7, KV cache and generation flow: the prompt is
 * prefilled once at batch 1 and its cache copied into every row of the cache the
 * samples then decode from).  With s = src_seqlen[0] (device int32):
 *   k_dst[n, t] = k_src[0, t] and v_dst[n, t] = v_src[0, t] for n < N, t < s;
 *   dst_seqlens[n] = s for n < N.
 *   k_src, v_src [1][T_src][n_kv_head][D]; k_dst, v_dst [N][T_max][n_kv_head][D],
 *   same dtype (bf16 or fp32), 16-byte aligned, a row of n_kv_head * D elements a
 *   multiple of 16 bytes; dst_seqlens device int32 [N].  Destination rows t >= s
 *   are left untouched.  Requires T_src <= T_max.
 *   Precondition 0 <= s <= T_src (a device value, not checkable on the host
 *   without a sync): otherwise nothing is copied and every dst_seqlens[n] is set
 *   to -1, which ncattn_decode treats as an invalid row (NaN output).
 *   No workspace; the sources are only read.
 */
int ncattn_cache_replicate(const void *k_src, const void *v_src, const int32_t *src_seqlen, void *k_dst,
                           void *v_dst, int32_t *dst_seqlens, int N, int T_src, int T_max, int n_kv_head,
                           int head_dim, int dtype, void *stream);

/* Thread-local description of the last non-OK return on this thread ("" if none). */
const char *ncattn_last_error(void);

/* Library version string. */
const char *ncattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NCATTN_H */
