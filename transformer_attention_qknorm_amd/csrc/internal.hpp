// Internal launch functions behind the C ABI (include/ncattn.h).  Each one
// assumes arguments were validated by ncattn_api.hip and only sizes the grid and
// enqueues kernels on the given stream; it returns hipGetLastError() afterwards.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ncattn {

struct AttnShape {
  int B, T, H, KV, D;
  int window;   // window_left, -1 = unbounded
  float scale;  // resolved softmax scale (> 0)
};

// QK-norm + RoPE in place; inv_freq[j] = base^(-2j/D) computed on the host in fp64.
hipError_t launch_qknorm_rope(void *q, void *k, int B, int T, int H, int KV, int D,
                              const int32_t *pos_offset, const double *inv_freq_host, float eps,
                              float gain, bool bf16, hipStream_t s);

// Its backward: dq/dk hold dy on entry and dx on return; q/k are the forward's inputs.
hipError_t launch_qknorm_rope_bwd(void *dq, void *dk, const void *q, const void *k, int B, int T, int H, int KV,
                                  int D, const int32_t *pos_offset, const double *inv_freq_host, float eps,
                                  float gain, bool bf16, hipStream_t s);

// Backward stages (bit mask): D_i = dO.O, then dK/dV, then dQ.
constexpr int kBwdDelta = 1, kBwdDkDv = 2, kBwdDq = 4, kBwdAll = 7;

// The bf16 backward hands dS = P (dP - D) from the dK/dV stage to the dQ stage
// through the workspace, as bf16 64 x 64 tiles stored transposed ([key][query],
// row-major), one per (b, head, query tile, key tile) inside the window band:
// query tile qt keeps key tiles kt_lo(qt) .. qt, slot j = kt - kt_lo(qt).
struct DsBand {
  int nqt;  // query tiles of 64 rows
  int nbw;  // key-tile slots per query tile
};
inline DsBand ds_band(int T, int W) {
  const int nt = (T + 63) / 64;
  const int nbw = W < 0 ? nt : (W + 63) / 64 + 1;
  return DsBand{nt, nbw < nt ? nbw : nt};
}
__host__ __device__ inline int ds_kt_lo(int qt, int W) {
  if (W < 0) return 0;
  const int x = 64 * qt - W;
  return x > 0 ? x / 64 : 0;
}
// workspace: D [B][H][T] fp32 (padded to 256 B); bf16 adds LSE * log2(e) (same size) and
// the dS band
size_t bwd_workspace_bytes(int B, int T, int H, int W, bool bf16);

// bf16, head_dim 128, MFMA kernels.
hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                           const AttnShape &sh, hipStream_t s);
// The same forward with QK-norm + RoPE of q done in its prologue: each query row
// is normalised and rotated in registers and written back into q, which the
// attention then uses; k must already be normalised.  inv_freq_host[j] =
// base^(-2j/D) in fp64.
hipError_t launch_fwd_bf16_qknorm_rope(void *q, const void *k, const void *v, void *o, float *lse,
                                       const AttnShape &sh, const int32_t *pos_offset,
                                       const double *inv_freq_host, float eps, float gain, hipStream_t s);
// The same forward for Tq query rows per sequence at positions q_pos0[b] + r
// (q_pos0 device int32 [B], NULL for 0) over key rows [0, q_pos0[b] + Tq) of K/V
// arrays with Tk rows per sequence; lse may be NULL.  Sequences whose offset
// leaves the queries outside [0, Tk) get NaN rows.
hipError_t launch_fwd_bf16_rows(const void *q, const void *k, const void *v, void *o, float *lse,
                                const int32_t *q_pos0, int B, int Tq, int Tk, int H, int KV, int W, float scale,
                                hipStream_t s);
hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o,
                           const float *lse, const void *dout, void *dq, void *dk, void *dv,
                           void *workspace, const AttnShape &sh, int stages, hipStream_t s);

// fp32 reference-precision kernels (head_dim 64 or 128).
hipError_t launch_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                          const AttnShape &sh, hipStream_t s);
hipError_t launch_bwd_f32(const float *q, const float *k, const float *v, const float *o,
                          const float *lse, const float *dout, float *dq, float *dk, float *dv,
                          float *delta, const AttnShape &sh, int stages, hipStream_t s);

// Split-KV decode, bf16, head_dim 128.
size_t decode_workspace_bytes(int B, int T_max, int H, int KV, int D, int window);
hipError_t launch_decode_bf16(const void *q, const void *k_new, const void *v_new, void *k_cache,
                              void *v_cache, const int32_t *seqlens, void *o, float *lse, int B,
                              int T_max, int H, int KV, int D, int window, float scale,
                              void *workspace, hipStream_t s);

// Chunked prefill, bf16, head_dim 128: append k_new/v_new [B][Tn][KV][D] at
// cache rows seqlens[b].., then the forward of q [B][Tn][H][D] over the cache.
hipError_t launch_cache_replicate(const void *k_src, const void *v_src, const int32_t *src_seqlen, void *k_dst,
                                  void *v_dst, int32_t *dst_seqlens, int N, int T_src, int T_max, int row_pieces,
                                  hipStream_t s);
hipError_t launch_prefill_bf16(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                               const int32_t *seqlens, void *o, float *lse, int B, int Tn, int T_max, int H,
                               int KV, int window, float scale, hipStream_t s);

}  // namespace ncattn
