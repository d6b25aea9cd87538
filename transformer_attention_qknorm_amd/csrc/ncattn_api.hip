// C ABI of ncattn: host-side validation, workspace sizing and dispatch.
// Every argument is checked before anything is enqueued; errors come back as
// status codes with a thread-local message (include/ncattn.h).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <new>

#include "ncattn.h"
#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return NCATTN_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(NCATTN_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The element-count limit of every tensor (see check_heads).
bool too_large(int B, int T, int H, int D) { return (double)B * T * H * D > 4.0e15; }

// Shape checks common to every attention call.
int check_heads(const char *fn, int B, int T, int H, int KV, int D) {
  if (B <= 0 || T <= 0 || H <= 0 || KV <= 0 || D <= 0)
    return fail(NCATTN_EINVAL, "%s: sizes must be positive (B=%d T=%d n_head=%d n_kv_head=%d head_dim=%d)", fn, B,
                T, H, KV, D);
  if (H % KV != 0) return fail(NCATTN_EINVAL, "%s: n_head (%d) must be a multiple of n_kv_head (%d)", fn, H, KV);
  // every index used by the kernels is formed in 64-bit, but per-tensor element
  // counts must still fit the int64 address arithmetic comfortably
  if (too_large(B, T, H, D)) return fail(NCATTN_EINVAL, "%s: tensor too large", fn);
  return NCATTN_OK;
}

int check_dtype(const char *fn, int dtype) {
  if (dtype != NCATTN_BF16 && dtype != NCATTN_F32) return fail(NCATTN_EINVAL, "%s: unknown dtype %d", fn, dtype);
  return NCATTN_OK;
}

int check_attn_support(const char *fn, int dtype, int T, int H, int D) {
  if (dtype == NCATTN_BF16 && D != 64 && D != 128)
    return fail(NCATTN_EUNSUPPORTED, "%s: bf16 attention supports head_dim 64 or 128 (got %d)", fn, D);
  // the bf16 kernels address one (batch, head) slice of q/k/v/dO through 32-bit
  // byte offsets: (T + 64) rows of the token stride must stay below 2^31
  if (dtype == NCATTN_BF16 && ((double)T + 64.0) * H * D * 2.0 >= 2147483648.0)
    return fail(NCATTN_EUNSUPPORTED, "%s: seq_len x n_head too large for the bf16 kernels (T=%d n_head=%d)", fn, T, H);
  if (dtype == NCATTN_F32 && D != 64 && D != 128)
    return fail(NCATTN_EUNSUPPORTED, "%s: fp32 attention supports head_dim 64 or 128 (got %d)", fn, D);
  return NCATTN_OK;
}

int check_window(const char *fn, int wl, int wr) {
  if (wl < -1) return fail(NCATTN_EINVAL, "%s: window_left must be >= -1 (got %d)", fn, wl);
  if (wr != 0) return fail(NCATTN_EINVAL, "%s: window_right must be 0 (causal), got %d", fn, wr);
  return NCATTN_OK;
}

// A window that reaches past the first key of every row is full causal
// attention; window_left >= span - 1 (span = the rows a query can see) is mapped
// to -1 before any sizing or launch, so that no kernel forms i + W or W + 63 with
// a W near INT_MAX.
int effective_window(int wl, int span) { return (wl < 0 || wl >= span - 1) ? -1 : wl; }

#define NC_TRY(expr)            \
  do {                          \
    int _rc = (expr);           \
    if (_rc != NCATTN_OK) return _rc; \
  } while (0)

#define NC_PTR(p, fn)                                                                \
  do {                                                                               \
    if ((p) == nullptr) return fail(NCATTN_EINVAL, "%s: %s is NULL", fn, #p);        \
    if (!aligned16(p)) return fail(NCATTN_EINVAL, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

float resolve_scale(float s, int D) { return s > 0.f ? s : (float)(1.0 / sqrt((double)D)); }

}  // namespace

extern "C" {

const char *ncattn_last_error(void) { return g_err; }

const char *ncattn_version(void) { return "ncattn 0.1.0 (gfx950)"; }

// Checks shared by the QK-norm + RoPE calls; fills inv_freq[j] = base^(-2j/D).
static int check_qknorm(const char *fn, int B, int T, int n_head, int n_kv_head, int head_dim,
                        const int32_t *pos_offset, float rope_base, float eps, float qk_gain, int dtype,
                        double *inv_freq) {
  NC_TRY(check_heads(fn, B, T, n_head, n_kv_head, head_dim));
  NC_TRY(check_dtype(fn, dtype));
  if (head_dim != 64 && head_dim != 128)
    return fail(NCATTN_EUNSUPPORTED, "%s: head_dim must be 64 or 128 (got %d)", fn, head_dim);
  if (pos_offset != nullptr && ((uintptr_t)pos_offset & 3u))
    return fail(NCATTN_EINVAL, "%s: pos_offset is not 4-byte aligned", fn);
  if (!(rope_base > 1.0f) || !isfinite(rope_base)) return fail(NCATTN_EINVAL, "%s: rope_base must be > 1", fn);
  if (!(eps >= 0.0f) || !isfinite(eps)) return fail(NCATTN_EINVAL, "%s: eps must be >= 0", fn);
  if (!isfinite(qk_gain)) return fail(NCATTN_EINVAL, "%s: qk_gain must be finite", fn);
  for (int j = 0; j < head_dim / 2; ++j) inv_freq[j] = pow((double)rope_base, -2.0 * j / head_dim);
  return NCATTN_OK;
}

int ncattn_qknorm_rope(void *q, void *k, int B, int T, int n_head, int n_kv_head, int head_dim,
                       const int32_t *pos_offset, float rope_base, float eps, float qk_gain, int dtype,
                       void *stream) {
  const char *fn = "ncattn_qknorm_rope";
  NC_PTR(q, fn);
  NC_PTR(k, fn);
  double inv_freq[64];
  NC_TRY(check_qknorm(fn, B, T, n_head, n_kv_head, head_dim, pos_offset, rope_base, eps, qk_gain, dtype,
                      inv_freq));
  return hip_status(ncattn::launch_qknorm_rope(q, k, B, T, n_head, n_kv_head, head_dim, pos_offset, inv_freq, eps,
                                               qk_gain, dtype == NCATTN_BF16, (hipStream_t)stream),
                    fn);
}

int ncattn_qknorm_rope_rstd(void *q, void *k, float *rstd, int B, int T, int n_head, int n_kv_head, int head_dim,
                            const int32_t *pos_offset, float rope_base, float eps, float qk_gain, int dtype,
                            void *stream) {
  const char *fn = "ncattn_qknorm_rope_rstd";
  NC_PTR(q, fn);
  NC_PTR(k, fn);
  if (rstd == nullptr) return fail(NCATTN_EINVAL, "%s: rstd is NULL", fn);
  if ((uintptr_t)rstd & 3u) return fail(NCATTN_EINVAL, "%s: rstd is not 4-byte aligned", fn);
  double inv_freq[64];
  NC_TRY(check_qknorm(fn, B, T, n_head, n_kv_head, head_dim, pos_offset, rope_base, eps, qk_gain, dtype,
                      inv_freq));
  return hip_status(ncattn::launch_qknorm_rope(q, k, B, T, n_head, n_kv_head, head_dim, pos_offset, inv_freq, eps,
                                               qk_gain, dtype == NCATTN_BF16, (hipStream_t)stream, rstd,
                                               (long long)n_head + n_kv_head, n_head),
                    fn);
}

int ncattn_qknorm_rope_bwd(void *dq, void *dk, const void *q, const void *k, int B, int T, int n_head,
                           int n_kv_head, int head_dim, const int32_t *pos_offset, float rope_base, float eps,
                           float qk_gain, int dtype, void *stream) {
  const char *fn = "ncattn_qknorm_rope_bwd";
  NC_PTR(dq, fn);
  NC_PTR(dk, fn);
  NC_PTR(q, fn);
  NC_PTR(k, fn);
  double inv_freq[64];
  NC_TRY(check_qknorm(fn, B, T, n_head, n_kv_head, head_dim, pos_offset, rope_base, eps, qk_gain, dtype,
                      inv_freq));
  if (dq == q || dq == k || dk == q || dk == k)
    return fail(NCATTN_EINVAL, "%s: dq / dk must not alias the forward's inputs", fn);
  if (dq == dk) return fail(NCATTN_EINVAL, "%s: dq and dk must differ", fn);
  return hip_status(ncattn::launch_qknorm_rope_bwd(dq, dk, q, k, B, T, n_head, n_kv_head, head_dim, pos_offset,
                                                   inv_freq, eps, qk_gain, dtype == NCATTN_BF16,
                                                   (hipStream_t)stream),
                    fn);
}

int ncattn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int T, int n_head,
               int n_kv_head, int head_dim, int window_left, int window_right, float softmax_scale, int dtype,
               void *stream) {
  const char *fn = "ncattn_fwd";
  NC_PTR(q, fn);
  NC_PTR(k, fn);
  NC_PTR(v, fn);
  NC_PTR(o, fn);
  NC_PTR(lse, fn);
  NC_TRY(check_heads(fn, B, T, n_head, n_kv_head, head_dim));
  NC_TRY(check_dtype(fn, dtype));
  NC_TRY(check_window(fn, window_left, window_right));
  NC_TRY(check_attn_support(fn, dtype, T, n_head, head_dim));
  if (!isfinite(softmax_scale)) return fail(NCATTN_EINVAL, "%s: softmax_scale must be finite", fn);
  if (o == q || o == k || o == v) return fail(NCATTN_EINVAL, "%s: o must not alias an input", fn);
  window_left = effective_window(window_left, T);
  ncattn::AttnShape sh{B, T, n_head, n_kv_head, head_dim, window_left, resolve_scale(softmax_scale, head_dim)};
  hipError_t e = dtype == NCATTN_BF16
                     ? ncattn::launch_fwd_bf16(q, k, v, o, lse, sh, (hipStream_t)stream)
                     : ncattn::launch_fwd_f32((const float *)q, (const float *)k, (const float *)v, (float *)o, lse,
                                              sh, (hipStream_t)stream);
  return hip_status(e, fn);
}

int ncattn_fwd_fp8(const void *q, const void *k, const void *v, float q_descale, float k_descale, float v_descale,
                   void *o, float *lse, int B, int T, int n_head, int n_kv_head, int head_dim, int window_left,
                   int window_right, float softmax_scale, void *stream) {
  const char *fn = "ncattn_fwd_fp8";
  NC_PTR(q, fn);
  NC_PTR(k, fn);
  NC_PTR(v, fn);
  NC_PTR(o, fn);
  NC_PTR(lse, fn);
  NC_TRY(check_heads(fn, B, T, n_head, n_kv_head, head_dim));
  NC_TRY(check_window(fn, window_left, window_right));
  if (head_dim != 128)
    return fail(NCATTN_EUNSUPPORTED, "%s: fp8 attention supports head_dim 128 (got %d)", fn, head_dim);
  // one (batch, head) slice of k / v is addressed through 32-bit byte offsets
  if (((double)T + 64.0) * n_kv_head * head_dim >= 2147483648.0)
    return fail(NCATTN_EUNSUPPORTED, "%s: seq_len x n_kv_head too large (T=%d n_kv_head=%d)", fn, T, n_kv_head);
  if (!isfinite(softmax_scale)) return fail(NCATTN_EINVAL, "%s: softmax_scale must be finite", fn);
  if (!(isfinite(q_descale) && q_descale > 0.f && isfinite(k_descale) && k_descale > 0.f && isfinite(v_descale) &&
        v_descale > 0.f))
    return fail(NCATTN_EINVAL, "%s: descales must be finite and > 0", fn);
  if (o == q || o == k || o == v) return fail(NCATTN_EINVAL, "%s: o must not alias an input", fn);
  window_left = effective_window(window_left, T);
  ncattn::AttnShape sh{B, T, n_head, n_kv_head, head_dim, window_left, resolve_scale(softmax_scale, head_dim)};
  return hip_status(ncattn::launch_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, o, lse, sh, (hipStream_t)stream),
                    fn);
}

int ncattn_fwd_qknorm_rope(void *q, void *k, const void *v, void *o, float *lse, float *rstd, int B, int T,
                           int n_head, int n_kv_head, int head_dim, const int32_t *pos_offset, float rope_base,
                           float eps, float qk_gain, int window_left, int window_right, float softmax_scale,
                           int dtype, void *stream) {
  const char *fn = "ncattn_fwd_qknorm_rope";
  NC_PTR(q, fn);
  NC_PTR(k, fn);
  NC_PTR(v, fn);
  NC_PTR(o, fn);
  NC_PTR(lse, fn);
  if (rstd != nullptr && ((uintptr_t)rstd & 3u)) return fail(NCATTN_EINVAL, "%s: rstd is not 4-byte aligned", fn);
  double inv_freq[64];
  NC_TRY(check_qknorm(fn, B, T, n_head, n_kv_head, head_dim, pos_offset, rope_base, eps, qk_gain, dtype,
                      inv_freq));
  NC_TRY(check_window(fn, window_left, window_right));
  NC_TRY(check_attn_support(fn, dtype, T, n_head, head_dim));
  if (!isfinite(softmax_scale)) return fail(NCATTN_EINVAL, "%s: softmax_scale must be finite", fn);
  if (q == k) return fail(NCATTN_EINVAL, "%s: q and k must be distinct", fn);
  if (o == q || o == k || o == v || v == q || v == k)
    return fail(NCATTN_EINVAL, "%s: o and v must not alias q, k or each other", fn);
  window_left = effective_window(window_left, T);
  ncattn::AttnShape sh{B, T, n_head, n_kv_head, head_dim, window_left, resolve_scale(softmax_scale, head_dim)};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  const long long rstride = (long long)n_head + n_kv_head;
  if (dtype == NCATTN_BF16) {
    // k alone (no query rows), then the forward that normalises q in its prologue
    e = ncattn::launch_qknorm_rope(k, k, B, T, 0, n_kv_head, head_dim, pos_offset, inv_freq, eps, qk_gain, true, s,
                                   rstd, rstride, n_head);
    if (e == hipSuccess)
      e = ncattn::launch_fwd_bf16_qknorm_rope(q, k, v, o, lse, sh, pos_offset, inv_freq, eps, qk_gain, s, rstd,
                                              rstride);
  } else {
    e = ncattn::launch_qknorm_rope(q, k, B, T, n_head, n_kv_head, head_dim, pos_offset, inv_freq, eps, qk_gain,
                                   false, s, rstd, rstride, n_head);
    if (e == hipSuccess)
      e = ncattn::launch_fwd_f32((const float *)q, (const float *)k, (const float *)v, (float *)o, lse, sh, s);
  }
  return hip_status(e, fn);
}

size_t ncattn_bwd_workspace_bytes(int B, int T, int n_head, int n_kv_head, int head_dim, int window_left,
                                  int dtype) {
  // 0 for any shape the backward refuses (never a wrapped size)
  if (B <= 0 || T <= 0 || n_head <= 0 || n_kv_head <= 0 || head_dim <= 0 || window_left < -1) return 0;
  if (n_head % n_kv_head != 0 || too_large(B, T, n_head, head_dim)) return 0;
  return ncattn::bwd_workspace_bytes(B, T, n_head, effective_window(window_left, T), dtype == NCATTN_BF16);
}
}  // extern "C"

namespace {

int bwd_common(const char *fn, int stages, const void *q, const void *k, const void *v, const void *o,
               const float *lse, const void *dout, void *dq, void *dk, void *dv, int B, int T, int n_head,
               int n_kv_head, int head_dim, int window_left, int window_right, float softmax_scale, int dtype,
               void *workspace, size_t workspace_bytes, void *stream) {
  NC_PTR(q, fn);
  NC_PTR(k, fn);
  NC_PTR(v, fn);
  NC_PTR(o, fn);
  NC_PTR(lse, fn);
  NC_PTR(dout, fn);
  NC_PTR(dq, fn);
  NC_PTR(dk, fn);
  NC_PTR(dv, fn);
  NC_TRY(check_heads(fn, B, T, n_head, n_kv_head, head_dim));
  NC_TRY(check_dtype(fn, dtype));
  NC_TRY(check_window(fn, window_left, window_right));
  NC_TRY(check_attn_support(fn, dtype, T, n_head, head_dim));
  if (!isfinite(softmax_scale)) return fail(NCATTN_EINVAL, "%s: softmax_scale must be finite", fn);
  const void *ins[] = {q, k, v, o, lse, dout};
  void *outs[] = {dq, dk, dv};
  for (void *x : outs)
    for (const void *y : ins)
      if (x == y) return fail(NCATTN_EINVAL, "%s: gradients must not alias an input", fn);
  if (dq == dk || dq == dv || dk == dv) return fail(NCATTN_EINVAL, "%s: dq, dk, dv must be distinct", fn);
  size_t need = ncattn_bwd_workspace_bytes(B, T, n_head, n_kv_head, head_dim, window_left, dtype);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(NCATTN_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned16(workspace)) return fail(NCATTN_EINVAL, "%s: workspace is not 16-byte aligned", fn);
  if (stages == 0) return ok();  // validation only (the caller launches)
  window_left = effective_window(window_left, T);
  ncattn::AttnShape sh{B, T, n_head, n_kv_head, head_dim, window_left, resolve_scale(softmax_scale, head_dim)};
  hipError_t e =
      dtype == NCATTN_BF16
          ? ncattn::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, workspace, sh, stages,
                                    (hipStream_t)stream)
          : ncattn::launch_bwd_f32((const float *)q, (const float *)k, (const float *)v, (const float *)o, lse,
                                   (const float *)dout, (float *)dq, (float *)dk, (float *)dv, (float *)workspace, sh,
                                   stages, (hipStream_t)stream);
  return hip_status(e, fn);
}

}  // namespace

extern "C" {

int ncattn_bwd_qknorm_rope(const void *q, const void *k, const void *v, const void *o, const float *lse,
                           const void *dout, const float *rstd, const int32_t *pos_offset, float rope_base,
                           float qk_gain, void *dq, void *dk, void *dv, int B, int T, int n_head, int n_kv_head,
                           int head_dim, int window_left, int window_right, float softmax_scale, int dtype,
                           void *workspace, size_t workspace_bytes, void *stream) {
  const char *fn = "ncattn_bwd_qknorm_rope";
  if (rstd == nullptr) return fail(NCATTN_EINVAL, "%s: rstd is NULL", fn);
  if ((uintptr_t)rstd & 3u) return fail(NCATTN_EINVAL, "%s: rstd is not 4-byte aligned", fn);
  double inv_freq[64];
  NC_TRY(check_qknorm(fn, B, T, n_head, n_kv_head, head_dim, pos_offset, rope_base, 0.f, qk_gain, dtype,
                      inv_freq));
  if ((const void *)rstd == dq || (const void *)rstd == dk || (const void *)rstd == dv)
    return fail(NCATTN_EINVAL, "%s: gradients must not alias rstd", fn);
  // every check of ncattn_bwd, with launching deferred to here
  NC_TRY(bwd_common(fn, 0, q, k, v, o, lse, dout, dq, dk, dv, B, T, n_head, n_kv_head, head_dim, window_left,
                    window_right, softmax_scale, dtype, workspace, workspace_bytes, stream));
  window_left = effective_window(window_left, T);
  ncattn::AttnShape sh{B, T, n_head, n_kv_head, head_dim, window_left, resolve_scale(softmax_scale, head_dim)};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (dtype == NCATTN_BF16) {
    e = ncattn::launch_bwd_bf16_qknorm_rope(q, k, v, o, lse, dout, rstd, dq, dk, dv, workspace, sh, pos_offset,
                                            inv_freq, qk_gain, s);
  } else {
    e = ncattn::launch_bwd_f32((const float *)q, (const float *)k, (const float *)v, (const float *)o, lse,
                               (const float *)dout, (float *)dq, (float *)dk, (float *)dv, (float *)workspace, sh,
                               ncattn::kBwdAll, s);
    if (e == hipSuccess)
      e = ncattn::launch_qknorm_rope_bwd(dq, dk, q, k, B, T, n_head, n_kv_head, head_dim, pos_offset, inv_freq, 0.f,
                                         qk_gain, false, s, rstd, (long long)n_head + n_kv_head, n_head);
  }
  return hip_status(e, fn);
}

#define NC_BWD_ARGS                                                                                          \
  q, k, v, o, lse, dout, dq, dk, dv, B, T, n_head, n_kv_head, head_dim, window_left, window_right, softmax_scale, \
      dtype, workspace, workspace_bytes, stream
#define NC_BWD_PARAMS                                                                                        \
  const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout, void *dq,    \
      void *dk, void *dv, int B, int T, int n_head, int n_kv_head, int head_dim, int window_left,             \
      int window_right, float softmax_scale, int dtype, void *workspace, size_t workspace_bytes, void *stream

int ncattn_bwd(NC_BWD_PARAMS) { return bwd_common("ncattn_bwd", ncattn::kBwdAll, NC_BWD_ARGS); }
int ncattn_bwd_preprocess(NC_BWD_PARAMS) {
  return bwd_common("ncattn_bwd_preprocess", ncattn::kBwdDelta, NC_BWD_ARGS);
}
int ncattn_bwd_dkdv(NC_BWD_PARAMS) { return bwd_common("ncattn_bwd_dkdv", ncattn::kBwdDkDv, NC_BWD_ARGS); }
int ncattn_bwd_dq(NC_BWD_PARAMS) { return bwd_common("ncattn_bwd_dq", ncattn::kBwdDq, NC_BWD_ARGS); }

size_t ncattn_decode_workspace_bytes(int B, int T_max, int n_head, int n_kv_head, int head_dim, int window_left) {
  // 0 for any shape decode refuses (never a wrapped size)
  if (B <= 0 || T_max <= 0 || n_head <= 0 || n_kv_head <= 0 || head_dim <= 0 || window_left < -1) return 0;
  if (n_head % n_kv_head != 0 || too_large(B, T_max, n_head, head_dim)) return 0;
  return ncattn::decode_workspace_bytes(B, T_max, n_head, n_kv_head, head_dim, effective_window(window_left, T_max));
}

}  // extern "C"

namespace {

// Checks shared by the two decode calls; on success window_left holds the
// effective window.
int decode_check(const char *fn, const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                 const int32_t *cache_seqlens, void *o, float *lse, int B, int T_max, int n_head, int n_kv_head,
                 int head_dim, int &window_left, float softmax_scale, int dtype) {
  NC_PTR(q, fn);
  NC_PTR(k_new, fn);
  NC_PTR(v_new, fn);
  NC_PTR(k_cache, fn);
  NC_PTR(v_cache, fn);
  NC_PTR(o, fn);
  if (cache_seqlens == nullptr) return fail(NCATTN_EINVAL, "%s: cache_seqlens is NULL", fn);
  if ((uintptr_t)cache_seqlens & 3u) return fail(NCATTN_EINVAL, "%s: cache_seqlens is not 4-byte aligned", fn);
  if (lse != nullptr && ((uintptr_t)lse & 3u)) return fail(NCATTN_EINVAL, "%s: lse is not 4-byte aligned", fn);
  NC_TRY(check_heads(fn, B, T_max, n_head, n_kv_head, head_dim));
  NC_TRY(check_dtype(fn, dtype));
  if (window_left < -1) return fail(NCATTN_EINVAL, "%s: window_left must be >= -1 (got %d)", fn, window_left);
  if (dtype != NCATTN_BF16) return fail(NCATTN_EUNSUPPORTED, "%s: decode supports bf16 only", fn);
  if (head_dim != 64 && head_dim != 128)
    return fail(NCATTN_EUNSUPPORTED, "%s: decode supports head_dim 64 or 128 (got %d)", fn, head_dim);
  if (!isfinite(softmax_scale)) return fail(NCATTN_EINVAL, "%s: softmax_scale must be finite", fn);
  if (k_cache == v_cache) return fail(NCATTN_EINVAL, "%s: k_cache and v_cache must differ", fn);
  if (o == q || o == k_cache || o == v_cache || o == k_new || o == v_new)
    return fail(NCATTN_EINVAL, "%s: o must not alias an input", fn);
  window_left = effective_window(window_left, T_max);
  return NCATTN_OK;
}

}  // namespace

extern "C" {

int ncattn_decode(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                  const int32_t *cache_seqlens, void *o, float *lse, int B, int T_max, int n_head, int n_kv_head,
                  int head_dim, int window_left, float softmax_scale, int dtype, void *workspace,
                  size_t workspace_bytes, void *stream) {
  const char *fn = "ncattn_decode";
  NC_TRY(decode_check(fn, q, k_new, v_new, k_cache, v_cache, cache_seqlens, o, lse, B, T_max, n_head, n_kv_head,
                      head_dim, window_left, softmax_scale, dtype));
  size_t need = ncattn::decode_workspace_bytes(B, T_max, n_head, n_kv_head, head_dim, window_left);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(NCATTN_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned16(workspace)) return fail(NCATTN_EINVAL, "%s: workspace is not 16-byte aligned", fn);
  hipError_t e = ncattn::launch_decode_bf16(q, k_new, v_new, k_cache, v_cache, cache_seqlens, o, lse, B, T_max,
                                            n_head, n_kv_head, head_dim, window_left,
                                            resolve_scale(softmax_scale, head_dim), workspace, (hipStream_t)stream);
  return hip_status(e, fn);
}

int ncattn_decode_noalloc(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                          const int32_t *cache_seqlens, void *o, float *lse, int B, int T_max, int n_head,
                          int n_kv_head, int head_dim, int window_left, float softmax_scale, int dtype,
                          void *stream) {
  const char *fn = "ncattn_decode_noalloc";
  NC_TRY(decode_check(fn, q, k_new, v_new, k_cache, v_cache, cache_seqlens, o, lse, B, T_max, n_head, n_kv_head,
                      head_dim, window_left, softmax_scale, dtype));
  const size_t need = ncattn::decode_workspace_bytes(B, T_max, n_head, n_kv_head, head_dim, window_left);
  if (need > (size_t)NCATTN_DECODE_SCRATCH_BYTES)
    return fail(NCATTN_EWORKSPACE,
                "%s: this shape needs %zu bytes of split-KV scratch; the library's per-device scratch holds %zu "
                "(use ncattn_decode with a workspace)",
                fn, need, (size_t)NCATTN_DECODE_SCRATCH_BYTES);
  void *scratch = nullptr;
  hipError_t e = ncattn::decode_scratch_ptr(&scratch);
  if (e != hipSuccess) return hip_status(e, fn);
  e = ncattn::launch_decode_bf16(q, k_new, v_new, k_cache, v_cache, cache_seqlens, o, lse, B, T_max, n_head,
                                 n_kv_head, head_dim, window_left, resolve_scale(softmax_scale, head_dim), scratch,
                                 (hipStream_t)stream);
  return hip_status(e, fn);
}

int ncattn_prefill(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                   const int32_t *cache_seqlens, void *o, float *lse, int B, int Tn, int T_max, int n_head,
                   int n_kv_head, int head_dim, int window_left, float softmax_scale, int dtype, void *stream) {
  const char *fn = "ncattn_prefill";
  NC_PTR(q, fn);
  NC_PTR(k_new, fn);
  NC_PTR(v_new, fn);
  NC_PTR(k_cache, fn);
  NC_PTR(v_cache, fn);
  NC_PTR(o, fn);
  if (cache_seqlens == nullptr) return fail(NCATTN_EINVAL, "%s: cache_seqlens is NULL", fn);
  if ((uintptr_t)cache_seqlens & 3u) return fail(NCATTN_EINVAL, "%s: cache_seqlens is not 4-byte aligned", fn);
  if (lse != nullptr && ((uintptr_t)lse & 3u)) return fail(NCATTN_EINVAL, "%s: lse is not 4-byte aligned", fn);
  NC_TRY(check_heads(fn, B, T_max, n_head, n_kv_head, head_dim));
  if (Tn <= 0 || Tn > T_max) return fail(NCATTN_EINVAL, "%s: need 0 < Tn <= T_max (Tn=%d T_max=%d)", fn, Tn, T_max);
  NC_TRY(check_dtype(fn, dtype));
  if (window_left < -1) return fail(NCATTN_EINVAL, "%s: window_left must be >= -1 (got %d)", fn, window_left);
  if (dtype != NCATTN_BF16) return fail(NCATTN_EUNSUPPORTED, "%s: prefill supports bf16 only", fn);
  NC_TRY(check_attn_support(fn, dtype, T_max, n_head, head_dim));
  if (!isfinite(softmax_scale)) return fail(NCATTN_EINVAL, "%s: softmax_scale must be finite", fn);
  if (k_cache == v_cache) return fail(NCATTN_EINVAL, "%s: k_cache and v_cache must differ", fn);
  if (o == q || o == k_cache || o == v_cache || o == k_new || o == v_new)
    return fail(NCATTN_EINVAL, "%s: o must not alias an input", fn);
  window_left = effective_window(window_left, T_max);
  hipError_t e = ncattn::launch_prefill_bf16(q, k_new, v_new, k_cache, v_cache, cache_seqlens, o, lse, B, Tn, T_max,
                                             n_head, n_kv_head, head_dim, window_left,
                                             resolve_scale(softmax_scale, head_dim), (hipStream_t)stream);
  return hip_status(e, fn);
}

int ncattn_cache_replicate(const void *k_src, const void *v_src, const int32_t *src_seqlen, void *k_dst,
                           void *v_dst, int32_t *dst_seqlens, int N, int T_src, int T_max, int n_kv_head,
                           int head_dim, int dtype, void *stream) {
  const char *fn = "ncattn_cache_replicate";
  NC_PTR(k_src, fn);
  NC_PTR(v_src, fn);
  NC_PTR(k_dst, fn);
  NC_PTR(v_dst, fn);
  if (src_seqlen == nullptr || dst_seqlens == nullptr) return fail(NCATTN_EINVAL, "%s: a length pointer is NULL", fn);
  if (((uintptr_t)src_seqlen & 3u) || ((uintptr_t)dst_seqlens & 3u))
    return fail(NCATTN_EINVAL, "%s: length pointers must be 4-byte aligned", fn);
  NC_TRY(check_dtype(fn, dtype));
  if (N < 1 || T_src < 1 || n_kv_head < 1 || head_dim < 1)
    return fail(NCATTN_EINVAL, "%s: need N, T_src, n_kv_head, head_dim >= 1 (N=%d T_src=%d n_kv_head=%d head_dim=%d)",
                fn, N, T_src, n_kv_head, head_dim);
  if (T_max < T_src) return fail(NCATTN_EINVAL, "%s: need T_src <= T_max (T_src=%d T_max=%d)", fn, T_src, T_max);
  const int elem = dtype == NCATTN_BF16 ? 2 : 4;
  // sizes checked in floating point before any integer product is formed
  if ((double)n_kv_head * head_dim * elem / 16.0 > 2147483647.0 ||
      (double)N * T_max * n_kv_head * head_dim * elem / 16.0 > 1152921504606846976.0 /* 2^60 */)
    return fail(NCATTN_EINVAL, "%s: sizes too large", fn);
  const long long row_bytes = (long long)n_kv_head * head_dim * elem;
  if (row_bytes % 16) return fail(NCATTN_EINVAL, "%s: a cache row (n_kv_head * head_dim elements) must be a multiple of 16 bytes", fn);
  if ((((uintptr_t)k_src | (uintptr_t)v_src | (uintptr_t)k_dst | (uintptr_t)v_dst) & 15u))
    return fail(NCATTN_EINVAL, "%s: cache pointers must be 16-byte aligned", fn);
  if (k_dst == v_dst || k_dst == k_src || k_dst == v_src || v_dst == k_src || v_dst == v_src)
    return fail(NCATTN_EINVAL, "%s: the destination caches must be distinct from each other and from the sources", fn);
  hipError_t e = ncattn::launch_cache_replicate(k_src, v_src, src_seqlen, k_dst, v_dst, dst_seqlens, N, T_src, T_max,
                                                (int)(row_bytes / 16), (hipStream_t)stream);
  return hip_status(e, fn);
}

}  // extern "C"
