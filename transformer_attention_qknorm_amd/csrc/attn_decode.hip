// Single-token decode against a KV cache, bf16, head_dim 64 or 128 (HBM-bound).
//
// "nanochat Admin & Developer Guide", section 6 (the fallback's single-token
// decode attends over the window of the cache) and section 7 "KV cache" (cache
// (B, T, H, D) per layer, per-sequence int32 cache_seqlens, the new token written
// into the cache in place).  For sequence b with s = cache_seqlens[b]:
//   cache[b, s] <- (k_new[b], v_new[b]);
//   o[b, h] = softmax_j(scale q[b, h] . k_j) v_j over j in [max(0, s - W), s].
//
// Split-KV: the visible keys of each (b, kv head) are cut into chunks of 128.
// decode_split: one workgroup per (b, chunk, kv head), the kv heads of a chunk
// on consecutive blocks so that the KV x 2 D contiguous bytes of each cached key
// are read at about the same time; D / 8 lanes per K or V row (16 B each), so
// 256 / (D / 8) groups of lanes (16 for D = 128, 32 for D = 64), each owning
// 8 or 4 keys, and every load instruction covers whole rows (four 256-byte or
// eight 128-byte rows).  All K and V loads of the chunk are issued up front;
// scores are reduced over the row's lanes with DPP, the softmax
// statistics over the groups through LDS, and each query head of the group reuses
// the K/V registers.  The chunk that holds key s takes it from k_new/v_new and
// writes it into the cache; no other chunk touches slot s, and slots past s are
// never read (they may hold anything, NaN included).
// decode_combine: one workgroup per (b, h) merges the chunk partials
// (max, sum, unnormalised output) into o and lse: the maximum over the chunks in
// parallel, then the weighted sums with eight chunks' loads in flight.
#include <mutex>

#include "ncattn.h"
#include "device_common.hpp"
#include "internal.hpp"

namespace ncattn {

namespace {

constexpr int kCH = kDecodeChunk;  // keys per chunk


// Sum over each group of 8 lanes (DPP): xor-1 and xor-2 quad permutes, then the
// half-row mirror, which pairs the two quads of the group.
__device__ __forceinline__ float row8_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ Kn, const uint16_t *__restrict__ Vn,
    uint16_t *__restrict__ Kc, uint16_t *__restrict__ Vc, const int32_t *__restrict__ seqlens,
    float *__restrict__ ws_o, float *__restrict__ ws_m, float *__restrict__ ws_l, int B, int T_max, int H, int KV,
    int W, float c, int C_max) {
  constexpr int kLanes = D / 8;           // lanes per row
  constexpr int kGroups = 256 / kLanes;   // key groups of the workgroup
  constexpr int kPerGroup = kCH / kGroups;
  __shared__ float red[kGroups];
  __shared__ float obuf[kGroups][D + 4];
  const int tid = threadIdx.x;
  const int grp = tid / kLanes;
  const int p16 = tid % kLanes;
  // the KV heads of one (sequence, chunk) are consecutive blocks: they read the
  // same keys' rows (KV x 256 contiguous bytes per key) at about the same time
  const int kvh = (int)(blockIdx.x % KV);
  const int rest = (int)(blockIdx.x / KV);
  const int chunk = rest % C_max;
  const int b = rest / C_max;
  const int G = H / KV;
  const int s = seqlens[b];
  if (s < 0 || s >= T_max) return;
  const int lo = W < 0 ? 0 : max(0, s - W);
  const int j0 = lo + chunk * kCH;
  if (j0 > s) return;

  const long long row_stride = (long long)KV * D;
  const long long cache_base = (long long)b * T_max * row_stride + (long long)kvh * D + p16 * 8;
  const long long new_off = ((long long)b * KV + kvh) * D + p16 * 8;

  u32x4 kreg[kPerGroup], vreg[kPerGroup];
#pragma unroll
  for (int it = 0; it < kPerGroup; ++it) {
    const int j = j0 + grp + kGroups * it;
    if (j < s) {
      kreg[it] = *(const u32x4 *)(Kc + cache_base + (long long)j * row_stride);
      vreg[it] = *(const u32x4 *)(Vc + cache_base + (long long)j * row_stride);
    } else if (j == s) {
      kreg[it] = *(const u32x4 *)(Kn + new_off);
      vreg[it] = *(const u32x4 *)(Vn + new_off);
      *(u32x4 *)(Kc + cache_base + (long long)j * row_stride) = kreg[it];
      *(u32x4 *)(Vc + cache_base + (long long)j * row_stride) = vreg[it];
    } else {
      kreg[it] = u32x4{0u, 0u, 0u, 0u};
      vreg[it] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  for (int g = 0; g < G; ++g) {
    const int h = kvh * G + g;
    float qv[8];
    {
      const u32x4 w = *(const u32x4 *)(Q + ((long long)b * H + h) * D + p16 * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qv[2 * i] = lo_bf16(w[i]);
        qv[2 * i + 1] = hi_bf16(w[i]);
      }
    }
    float sc[kPerGroup];
    float mloc = -INFINITY;
#pragma unroll
    for (int it = 0; it < kPerGroup; ++it) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        part = __builtin_fmaf(qv[2 * i], lo_bf16(kreg[it][i]), part);
        part = __builtin_fmaf(qv[2 * i + 1], hi_bf16(kreg[it][i]), part);
      }
      const float tot = (kLanes == 16 ? row16_sum(part) : row8_sum(part)) * c;  // log2-domain score
      const int j = j0 + grp + kGroups * it;
      sc[it] = j <= s ? tot : -INFINITY;
      mloc = fmaxf(mloc, sc[it]);
    }
    if (p16 == 0) red[grp] = mloc;
    __syncthreads();
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kGroups; ++i) m = fmaxf(m, red[i]);
    __syncthreads();
    float lsum = 0.f;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
    for (int it = 0; it < kPerGroup; ++it) {
      const float p = fast_exp2(sc[it] - m);  // the chunk always holds key j0 <= s, so m is finite
      lsum += p;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(p, lo_bf16(vreg[it][i]), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(p, hi_bf16(vreg[it][i]), acc[2 * i + 1]);
      }
    }
    if (p16 == 0) red[grp] = lsum;
#pragma unroll
    for (int i = 0; i < 8; ++i) obuf[grp][p16 * 8 + i] = acc[i];
    __syncthreads();
    const long long pidx = ((long long)b * H + h) * C_max + chunk;
    if (tid < D) {
      float o = 0.f;
#pragma unroll
      for (int gg = 0; gg < kGroups; ++gg) o += obuf[gg][tid];
      ws_o[pidx * D + tid] = o;
    }
    if (tid == 0) {
      float l = 0.f;
#pragma unroll
      for (int gg = 0; gg < kGroups; ++gg) l += red[gg];
      ws_m[pidx] = m;
      ws_l[pidx] = l;
    }
    __syncthreads();
  }
}

template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const float *__restrict__ ws_o,
                                                             const float *__restrict__ ws_m,
                                                             const float *__restrict__ ws_l,
                                                             const int32_t *__restrict__ seqlens,
                                                             uint16_t *__restrict__ O, float *__restrict__ LSE,
                                                             int B, int T_max, int H, int W, int C_max) {
  __shared__ float wmax[2];
  const int bh = blockIdx.x;
  const int b = bh / H;
  const int d = threadIdx.x;
  const int s = seqlens[b];
  if (s < 0 || s >= T_max) {
    O[(long long)bh * D + d] = 0x7fc0;  // bf16 quiet NaN
    if (LSE != nullptr && d == 0) LSE[bh] = __builtin_nanf("");
    return;
  }
  const int lo = W < 0 ? 0 : max(0, s - W);
  const int nc = (s - lo + 1 + kCH - 1) / kCH;
  const long long base = (long long)bh * C_max;
  // max of the chunk maxima: threads stride over the chunks, then the waves reduce
  float M = -INFINITY;
  for (int ci = d; ci < nc; ci += D) M = fmaxf(M, ws_m[base + ci]);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, shfl_xor(M, m));
  if ((d & 63) == 0) wmax[d >> 6] = M;
  __syncthreads();
  M = wmax[0];
  if constexpr (D > 64) M = fmaxf(M, wmax[1]);
  // weighted sums, eight chunks' loads in flight per step
  float L = 0.f, o = 0.f;
  int ci = 0;
  for (; ci + 8 <= nc; ci += 8) {
    float mm[8], ll[8], oo[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      mm[u] = ws_m[base + ci + u];
      ll[u] = ws_l[base + ci + u];
      oo[u] = ws_o[(base + ci + u) * D + d];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float a = fast_exp2(mm[u] - M);
      L = __builtin_fmaf(ll[u], a, L);
      o = __builtin_fmaf(oo[u], a, o);
    }
  }
  for (; ci < nc; ++ci) {
    const float a = fast_exp2(ws_m[base + ci] - M);
    L = __builtin_fmaf(ws_l[base + ci], a, L);
    o = __builtin_fmaf(ws_o[(base + ci) * D + d], a, o);
  }
  O[(long long)bh * D + d] = __builtin_bit_cast(uint16_t, (__bf16)(o / L));
  if (LSE != nullptr && d == 0) LSE[bh] = (M + log2f(L)) * kLn2;
}

}  // namespace

// Split-KV partials of ncattn_decode_noalloc, for callers that cannot allocate.
// Each device the library runs on holds its own copy for the life of the process.
// Host code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): it uses the device address decode_scratch_ptr()
// obtains once per device.
static __device__ __attribute__((aligned(256))) char scratch[NCATTN_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device, filled on its first use
}  // namespace

hipError_t decode_scratch_ptr(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {
template <int D>
hipError_t launch_decode_kernels(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                                 const int32_t *seqlens, void *o, float *lse, int B, int T_max, int H, int KV,
                                 int window, float scale, void *workspace, hipStream_t s) {
  const int C_max = decode_chunks_max(T_max, window);
  const size_t parts = (size_t)B * H * C_max;
  float *ws_o = (float *)workspace;
  float *ws_m = ws_o + parts * D;
  float *ws_l = ws_m + parts;
  const long long blocks = (long long)B * KV * C_max;
  if (blocks > 0x7fffffffLL || (long long)B * H > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_split_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t *)q,
                     (const uint16_t *)k_new, (const uint16_t *)v_new, (uint16_t *)k_cache, (uint16_t *)v_cache,
                     seqlens, ws_o, ws_m, ws_l, B, T_max, H, KV, window, scale * kLog2e, C_max);
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((unsigned)(B * H)), dim3(D), 0, s, ws_o, ws_m, ws_l, seqlens,
                     (uint16_t *)o, lse, B, T_max, H, window, C_max);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_bf16(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                              const int32_t *seqlens, void *o, float *lse, int B, int T_max, int H, int KV, int D,
                              int window, float scale, void *workspace, hipStream_t s) {
  if (D == 64)
    return launch_decode_kernels<64>(q, k_new, v_new, k_cache, v_cache, seqlens, o, lse, B, T_max, H, KV, window,
                                     scale, workspace, s);
  if (D == 128)
    return launch_decode_kernels<128>(q, k_new, v_new, k_cache, v_cache, seqlens, o, lse, B, T_max, H, KV, window,
                                      scale, workspace, s);
  return hipErrorInvalidValue;
}

}  // namespace ncattn
