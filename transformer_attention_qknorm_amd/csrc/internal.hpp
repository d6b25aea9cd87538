// Internal launch functions behind the C ABI (include/ncattn.h).  Each one
// assumes arguments were validated by ncattn_api.hip and only sizes the grid and
// enqueues kernels on the given stream; it returns hipGetLastError() afterwards.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sizing.hpp"

namespace ncattn {

struct AttnShape {
  int B, T, H, KV, D;
  int window;   // window_left, -1 = unbounded
  float scale;  // resolved softmax scale (> 0)
};

// QK-norm + RoPE in place; inv_freq[j] = base^(-2j/D) computed on the host in fp64.
// rstd (optional): each row's 1/sqrt(mean(x^2) + eps) at rstd[token * rstd_stride +
// head] (q rows) and [token * rstd_stride + rstd_k_off + kv head] (k rows).
hipError_t launch_qknorm_rope(void *q, void *k, int B, int T, int H, int KV, int D,
                              const int32_t *pos_offset, const double *inv_freq_host, float eps,
                              float gain, bool bf16, hipStream_t s, float *rstd = nullptr,
                              long long rstd_stride = 0, int rstd_k_off = 0);

// Its backward: dq/dk hold dy on entry and dx on return; q/k are the forward's
// inputs x, or, when rstd is given, its outputs y with the rows' 1/r in rstd
// (layout as launch_qknorm_rope's).
hipError_t launch_qknorm_rope_bwd(void *dq, void *dk, const void *q, const void *k, int B, int T, int H, int KV,
                                  int D, const int32_t *pos_offset, const double *inv_freq_host, float eps,
                                  float gain, bool bf16, hipStream_t s, const float *rstd = nullptr,
                                  long long rstd_stride = 0, int rstd_k_off = 0);

// Backward stages (bit mask): D_i = dO.O, then dK/dV, then dQ.
constexpr int kBwdDelta = 1, kBwdDkDv = 2, kBwdDq = 4, kBwdAll = 7;

// workspace: bwd_workspace_bytes() (sizing.hpp)

// bf16, head_dim 64 or 128, MFMA kernels.
hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                           const AttnShape &sh, hipStream_t s);
// The same forward with QK-norm + RoPE of q done in its prologue: each query row
// is normalised and rotated in registers and written back into q, which the
// attention then uses; k must already be normalised.  inv_freq_host[j] =
// base^(-2j/D) in fp64.
hipError_t launch_fwd_bf16_qknorm_rope(void *q, const void *k, const void *v, void *o, float *lse,
                                       const AttnShape &sh, const int32_t *pos_offset,
                                       const double *inv_freq_host, float eps, float gain, hipStream_t s,
                                       float *rstd = nullptr, long long rstd_stride = 0);
// The same forward for Tq query rows per sequence at positions q_pos0[b] + r
// (q_pos0 device int32 [B], NULL for 0) over key rows [0, q_pos0[b] + Tq) of K/V
// arrays with Tk rows per sequence; lse may be NULL.  Sequences whose offset
// leaves the queries outside [0, Tk) get NaN rows.
hipError_t launch_fwd_bf16_rows(const void *q, const void *k, const void *v, void *o, float *lse,
                                const int32_t *q_pos0, int B, int Tq, int Tk, int H, int KV, int D, int W,
                                float scale, hipStream_t s);
hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                           const float *lse, const void *dout, void *dq, void *dk, void *dv,
                           void *workspace, const AttnShape &sh, int stages, hipStream_t s);
// The full backward whose dq / dk are the gradients of the raw (pre-norm) rows:
// the dQ and dK/dV kernels carry their results back through QK-norm + RoPE
// before storing them, from the post-norm q, k and each row's 1/r (rstd
// [B][T][H + KV], q rows first).
hipError_t launch_bwd_bf16_qknorm_rope(const void *q, const void *k, const void *v, const void *o, const float *lse,
                                       const void *dout, const float *rstd, void *dq, void *dk, void *dv,
                                       void *workspace, const AttnShape &sh, const int32_t *pos_offset,
                                       const double *inv_freq_host, float gain, hipStream_t s);

// fp8 (OCP e4m3) q, k, v with per-tensor descales, bf16 o, head_dim 128.
hipError_t launch_fwd_fp8(const void *q, const void *k, const void *v, float q_descale, float k_descale,
                          float v_descale, void *o, float *lse, const AttnShape &sh, hipStream_t s);

// fp32 reference-precision kernels (head_dim 64 or 128).
hipError_t launch_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                          const AttnShape &sh, hipStream_t s);
hipError_t launch_bwd_f32(const float *q, const float *k, const float *v, const float *o,
                          const float *lse, const float *dout, float *dq, float *dk, float *dv,
                          float *delta, const AttnShape &sh, int stages, hipStream_t s);

// Split-KV decode, bf16, head_dim 64 or 128.
hipError_t launch_decode_bf16(const void *q, const void *k_new, const void *v_new, void *k_cache,
                              void *v_cache, const int32_t *seqlens, void *o, float *lse, int B,
                              int T_max, int H, int KV, int D, int window, float scale,
                              void *workspace, hipStream_t s);

// The address of this device's file-scope decode scratch array (looked up with
// hipGetSymbolAddress on the first call on the current device, then cached per
// device).  The array holds NCATTN_DECODE_SCRATCH_BYTES bytes.
hipError_t decode_scratch_ptr(void **out);

// Chunked prefill, bf16, head_dim 64 or 128: append k_new/v_new [B][Tn][KV][D] at
// cache rows seqlens[b].., then the forward of q [B][Tn][H][D] over the cache.
hipError_t launch_cache_replicate(const void *k_src, const void *v_src, const int32_t *src_seqlen, void *k_dst,
                                  void *v_dst, int32_t *dst_seqlens, int N, int T_src, int T_max, int row_pieces,
                                  hipStream_t s);
hipError_t launch_prefill_bf16(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                               const int32_t *seqlens, void *o, float *lse, int B, int Tn, int T_max, int H,
                               int KV, int D, int window, float scale, hipStream_t s);

}  // namespace ncattn
