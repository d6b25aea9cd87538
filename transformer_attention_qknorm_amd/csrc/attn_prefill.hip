// Chunked prefill against the KV cache, bf16, head_dim 64 or 128.
//
// For each sequence b with s = seqlens[b], the chunk's keys and values
// k_new[b, i], v_new[b, i] are written into cache rows s + i, then query
// q[b, i] (position s + i) attends over cache rows [max(0, s + i - W), s + i]
// ("nanochat Admin & Developer Guide", section 6: chunked inference against the
// cache; section 7: the cache updated in place at each sequence's position).
// The caller advances seqlens.
//
// Two launches on the caller's stream: a copy of the chunk into the cache (16
// bytes per lane), then the attention forward kernel itself, which takes each
// sequence's query offset from seqlens and bounds its key rows by s + Tn.  A
// sequence with s outside [0, T_max - Tn] is left untouched in the cache and gets
// NaN rows in o and lse (it cannot be checked on the host without a sync).
//
// Also the replication of a batch-1 prefill cache into a batch-N decode cache
// (same guide, section 7: the prompt is prefilled once, then its cache is copied
// into every row the samples decode from).
#include "device_common.hpp"
#include "internal.hpp"

namespace ncattn {

namespace {

template <int D>
__global__ __launch_bounds__(256) void prefill_append_kernel(const uint16_t *__restrict__ k_new,
                                                             const uint16_t *__restrict__ v_new,
                                                             uint16_t *__restrict__ k_cache,
                                                             uint16_t *__restrict__ v_cache,
                                                             const int32_t *__restrict__ seqlens, int B, int Tn,
                                                             int T_max, int KV) {
  // one 16-byte piece of one (b, i, kv head) row per lane; a row is D / 8 pieces
  constexpr int rp = D / 8;
  const long long pieces = (long long)B * Tn * KV * rp;
  for (long long p = (long long)blockIdx.x * blockDim.x + threadIdx.x; p < pieces;
       p += (long long)gridDim.x * blockDim.x) {
    const long long row = p / rp;           // (b, i, kv head) row of the chunk
    const int part = (int)(p % rp);
    const long long bi = row / KV;          // b * Tn + i
    const int kvh = (int)(row % KV);
    const int b = (int)(bi / Tn);
    const int i = (int)(bi % Tn);
    const int s = seqlens[b];
    if (s < 0 || s > T_max - Tn) continue;
    const long long src = row * D + part * 8;
    const long long dst = (((long long)b * T_max + s + i) * KV + kvh) * D + part * 8;
    *(u32x4 *)(k_cache + dst) = *(const u32x4 *)(k_new + src);
    *(u32x4 *)(v_cache + dst) = *(const u32x4 *)(v_new + src);
  }
}

// Copies the first s = *src_seqlen rows of a batch-1 cache into each of the N rows
// of a batch-N cache and sets the N lengths to s; a length outside [0, T_src]
// copies nothing and marks the rows -1.  Each lane reads a 16-byte piece of K and
// of V once and stores it N times.
__global__ __launch_bounds__(256) void cache_replicate_kernel(const u32x4 *__restrict__ k_src,
                                                              const u32x4 *__restrict__ v_src,
                                                              const int32_t *__restrict__ src_seqlen,
                                                              u32x4 *__restrict__ k_dst, u32x4 *__restrict__ v_dst,
                                                              int32_t *__restrict__ dst_seqlens, int N, int T_src,
                                                              int T_max, int row_pieces) {
  const int s = *src_seqlen;
  const bool valid = s >= 0 && s <= T_src;
  if (blockIdx.x == 0)
    for (int n = threadIdx.x; n < N; n += blockDim.x) dst_seqlens[n] = valid ? s : -1;
  if (!valid) return;
  const long long pieces = (long long)s * row_pieces;  // the source prefix is contiguous
  const long long dst_seq = (long long)T_max * row_pieces;
  for (long long p = (long long)blockIdx.x * blockDim.x + threadIdx.x; p < pieces;
       p += (long long)gridDim.x * blockDim.x) {
    const u32x4 kk = k_src[p];
    const u32x4 vv = v_src[p];
    for (int n = 0; n < N; ++n) {
      k_dst[n * dst_seq + p] = kk;
      v_dst[n * dst_seq + p] = vv;
    }
  }
}

}  // namespace

hipError_t launch_cache_replicate(const void *k_src, const void *v_src, const int32_t *src_seqlen, void *k_dst,
                                  void *v_dst, int32_t *dst_seqlens, int N, int T_src, int T_max, int row_pieces,
                                  hipStream_t s) {
  long long blocks = ((long long)T_src * row_pieces + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(cache_replicate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4 *)k_src,
                     (const u32x4 *)v_src, src_seqlen, (u32x4 *)k_dst, (u32x4 *)v_dst, dst_seqlens, N, T_src, T_max,
                     row_pieces);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                               const int32_t *seqlens, void *o, float *lse, int B, int Tn, int T_max, int H,
                               int KV, int D, int window, float scale, hipStream_t s) {
  const long long pieces = (long long)B * Tn * KV * (D / 8);
  long long blocks = (pieces + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (D == 64)
    hipLaunchKernelGGL(prefill_append_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t *)k_new,
                       (const uint16_t *)v_new, (uint16_t *)k_cache, (uint16_t *)v_cache, seqlens, B, Tn, T_max, KV);
  else if (D == 128)
    hipLaunchKernelGGL(prefill_append_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t *)k_new,
                       (const uint16_t *)v_new, (uint16_t *)k_cache, (uint16_t *)v_cache, seqlens, B, Tn, T_max, KV);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_fwd_bf16_rows(q, k_cache, v_cache, o, lse, seqlens, B, Tn, T_max, H, KV, D, window, scale, s);
}

}  // namespace ncattn
