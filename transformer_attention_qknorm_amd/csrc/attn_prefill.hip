// Chunked prefill against the KV cache, bf16, head_dim 128.
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
#include "device_common.hpp"
#include "internal.hpp"

namespace ncattn {

namespace {

__global__ __launch_bounds__(256) void prefill_append_kernel(const uint16_t *__restrict__ k_new,
                                                             const uint16_t *__restrict__ v_new,
                                                             uint16_t *__restrict__ k_cache,
                                                             uint16_t *__restrict__ v_cache,
                                                             const int32_t *__restrict__ seqlens, int B, int Tn,
                                                             int T_max, int KV) {
  // one 16-byte piece of one (b, i, kv head) row per lane; D = 128 is 16 pieces
  const long long pieces = (long long)B * Tn * KV * 16;
  for (long long p = (long long)blockIdx.x * blockDim.x + threadIdx.x; p < pieces;
       p += (long long)gridDim.x * blockDim.x) {
    const long long row = p >> 4;           // (b, i, kv head) row of the chunk
    const int part = (int)(p & 15);
    const long long bi = row / KV;          // b * Tn + i
    const int kvh = (int)(row % KV);
    const int b = (int)(bi / Tn);
    const int i = (int)(bi % Tn);
    const int s = seqlens[b];
    if (s < 0 || s > T_max - Tn) continue;
    const long long src = row * 128 + part * 8;
    const long long dst = (((long long)b * T_max + s + i) * KV + kvh) * 128 + part * 8;
    *(u32x4 *)(k_cache + dst) = *(const u32x4 *)(k_new + src);
    *(u32x4 *)(v_cache + dst) = *(const u32x4 *)(v_new + src);
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                               const int32_t *seqlens, void *o, float *lse, int B, int Tn, int T_max, int H,
                               int KV, int window, float scale, hipStream_t s) {
  const long long pieces = (long long)B * Tn * KV * 16;
  long long blocks = (pieces + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(prefill_append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t *)k_new,
                     (const uint16_t *)v_new, (uint16_t *)k_cache, (uint16_t *)v_cache, seqlens, B, Tn, T_max, KV);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_fwd_bf16_rows(q, k_cache, v_cache, o, lse, seqlens, B, Tn, T_max, H, KV, window, scale, s);
}

}  // namespace ncattn
