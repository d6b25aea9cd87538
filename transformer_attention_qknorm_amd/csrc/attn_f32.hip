// Attention forward and backward in fp32 throughout (head_dim 64 or 128).
//
// Same definitions as the bf16 MFMA path ("nanoGPT Administrator & Developer
// Guide" section 8; "nanochat Admin & Developer Guide" sections 3 and 6;
// backward = exact gradient), evaluated with plain fp32 FMA arithmetic and no
// rounding to a narrower type.  This path serves the fp32 precision the pages
// use on hardware without bf16 tensor cores ("nanochat Admin & Developer Guide",
// section 5), and the small fp32 workload; it is built for correctness, not speed.
//
// Four lanes share one row (query row in fwd/dq, key row in dkdv); each holds a
// quarter of head_dim, dot products are reduced over the 4 lanes.  Key (or query)
// rows are staged through LDS in chunks of 32.
#include "device_common.hpp"
#include "internal.hpp"

namespace ncattn {

namespace {

constexpr int kRows = 64;    // rows per block (4 lanes each -> 256 threads)
constexpr int kChunk = 32;   // staged rows per LDS chunk

__device__ __forceinline__ float quad_sum(float x) {
  x += shfl_xor(x, 1);
  x += shfl_xor(x, 2);
  return x;
}

__device__ __forceinline__ bool visible(int i, int j, int W) { return j <= i && (W < 0 || i - j <= W); }

// Copy rows [r0, r0 + kChunk) x D floats of a strided tensor into LDS (zero past nrows).
template <int D>
__device__ __forceinline__ void stage(float *dst, const float *src, long long stride, int r0, int nrows) {
  for (int x = threadIdx.x; x < kChunk * D / 4; x += blockDim.x) {
    const int r = x / (D / 4);
    const int c = (x % (D / 4)) * 4;
    f32x4 v = (r0 + r < nrows) ? *(const f32x4 *)(src + (long long)(r0 + r) * stride + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    *(f32x4 *)(dst + r * D + c) = v;
  }
}

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float *__restrict__ Q, const float *__restrict__ K,
                                                      const float *__restrict__ V, float *__restrict__ O,
                                                      float *__restrict__ LSE, int B, int T, int H, int KV, int W,
                                                      float scale) {
  constexpr int P = D / 4;
  __shared__ float ks[kChunk * D], vs[kChunk * D];
  const int nqb = (T + kRows - 1) / kRows;
  const int bh = blockIdx.x / nqb;
  const int b = bh / H, h = bh % H, kvh = h / (H / KV);
  const int q0 = (blockIdx.x % nqb) * kRows;
  const int row = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int i = q0 + row;
  const bool valid = i < T;
  const long long qs = (long long)H * D, kvs = (long long)KV * D;
  float q[P], o[P];
  for (int d = 0; d < P; ++d) {
    q[d] = valid ? Q[((long long)b * T + i) * qs + (long long)h * D + part * P + d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int lo = W < 0 ? 0 : max(0, q0 - W);
  const int hi = min(q0 + kRows - 1, T - 1);
  const float *Kb = K + (long long)b * T * kvs + (long long)kvh * D;
  const float *Vb = V + (long long)b * T * kvs + (long long)kvh * D;
  for (int j0 = lo; j0 <= hi; j0 += kChunk) {
    __syncthreads();
    stage<D>(ks, Kb, kvs, j0, T);
    stage<D>(vs, Vb, kvs, j0, T);
    __syncthreads();
    for (int jj = 0; jj < kChunk && j0 + jj <= hi; ++jj) {
      const int j = j0 + jj;
      float s = 0.f;
      for (int d = 0; d < P; ++d) s += q[d] * ks[jj * D + part * P + d];
      s = quad_sum(s) * scale;
      if (!(valid && visible(i, j, W))) continue;
      const float mn = fmaxf(m, s);
      const float a = expf(m - mn);  // exp(-inf) = 0 on the first key
      const float p = expf(s - mn);
      l = l * a + p;
      for (int d = 0; d < P; ++d) o[d] = o[d] * a + p * vs[jj * D + part * P + d];
      m = mn;
    }
  }
  if (!valid) return;
  for (int d = 0; d < P; ++d) O[((long long)b * T + i) * qs + (long long)h * D + part * P + d] = o[d] / l;
  if (part == 0) LSE[((long long)b * H + h) * T + i] = m + logf(l);
}

template <int D>
__global__ __launch_bounds__(256) void delta_f32_kernel(const float *__restrict__ O, const float *__restrict__ dO,
                                                        float *__restrict__ delta, int B, int T, int H) {
  constexpr int P = D / 4;
  const long long r = (long long)blockIdx.x * kRows + (threadIdx.x >> 2);
  const int part = threadIdx.x & 3;
  const long long n = (long long)B * T * H;
  float s = 0.f;
  if (r < n)
    for (int d = 0; d < P; ++d) s += O[r * D + part * P + d] * dO[r * D + part * P + d];
  s = quad_sum(s);
  if (r < n && part == 0) {
    const long long tok = r / H;
    const int h = (int)(r % H), b = (int)(tok / T), t = (int)(tok % T);
    delta[((long long)b * H + h) * T + t] = s;
  }
}

template <int D>
__global__ __launch_bounds__(256) void dq_f32_kernel(const float *__restrict__ Q, const float *__restrict__ K,
                                                     const float *__restrict__ V, const float *__restrict__ dO,
                                                     const float *__restrict__ LSE, const float *__restrict__ delta,
                                                     float *__restrict__ dQ, int B, int T, int H, int KV, int W,
                                                     float scale) {
  constexpr int P = D / 4;
  __shared__ float ks[kChunk * D], vs[kChunk * D];
  const int nqb = (T + kRows - 1) / kRows;
  const int bh = blockIdx.x / nqb;
  const int b = bh / H, h = bh % H, kvh = h / (H / KV);
  const int q0 = (blockIdx.x % nqb) * kRows;
  const int row = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int i = q0 + row;
  const bool valid = i < T;
  const long long qs = (long long)H * D, kvs = (long long)KV * D;
  float q[P], g[P], acc[P];
  for (int d = 0; d < P; ++d) {
    const long long off = ((long long)b * T + i) * qs + (long long)h * D + part * P + d;
    q[d] = valid ? Q[off] : 0.f;
    g[d] = valid ? dO[off] : 0.f;
    acc[d] = 0.f;
  }
  const long long ri = ((long long)b * H + h) * T + i;
  const float lse = valid ? LSE[ri] : 0.f;
  const float del = valid ? delta[ri] : 0.f;
  const int lo = W < 0 ? 0 : max(0, q0 - W);
  const int hi = min(q0 + kRows - 1, T - 1);
  const float *Kb = K + (long long)b * T * kvs + (long long)kvh * D;
  const float *Vb = V + (long long)b * T * kvs + (long long)kvh * D;
  for (int j0 = lo; j0 <= hi; j0 += kChunk) {
    __syncthreads();
    stage<D>(ks, Kb, kvs, j0, T);
    stage<D>(vs, Vb, kvs, j0, T);
    __syncthreads();
    for (int jj = 0; jj < kChunk && j0 + jj <= hi; ++jj) {
      const int j = j0 + jj;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < P; ++d) {
        s += q[d] * ks[jj * D + part * P + d];
        dp += g[d] * vs[jj * D + part * P + d];
      }
      s = quad_sum(s) * scale;
      dp = quad_sum(dp);
      if (!(valid && visible(i, j, W))) continue;
      const float ds = expf(s - lse) * (dp - del);
      for (int d = 0; d < P; ++d) acc[d] += ds * ks[jj * D + part * P + d];
    }
  }
  if (!valid) return;
  for (int d = 0; d < P; ++d) dQ[((long long)b * T + i) * qs + (long long)h * D + part * P + d] = acc[d] * scale;
}

template <int D>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(const float *__restrict__ Q, const float *__restrict__ K,
                                                       const float *__restrict__ V, const float *__restrict__ dO,
                                                       const float *__restrict__ LSE,
                                                       const float *__restrict__ delta, float *__restrict__ dK,
                                                       float *__restrict__ dV, int B, int T, int H, int KV, int W,
                                                       float scale) {
  constexpr int P = D / 4;
  __shared__ float qsh[kChunk * D], gsh[kChunk * D], lsh[kChunk], dsh[kChunk];
  const int nkb = (T + kRows - 1) / kRows;
  const int bk = blockIdx.x / nkb;
  const int b = bk / KV, kvh = bk % KV;
  const int G = H / KV;
  const int k0 = (blockIdx.x % nkb) * kRows;
  const int row = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int j = k0 + row;
  const bool valid = j < T;
  const long long qs = (long long)H * D, kvs = (long long)KV * D;
  float kk[P], vv[P], dk[P], dv[P];
  for (int d = 0; d < P; ++d) {
    const long long off = ((long long)b * T + j) * kvs + (long long)kvh * D + part * P + d;
    kk[d] = valid ? K[off] : 0.f;
    vv[d] = valid ? V[off] : 0.f;
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  const int kl = min(k0 + kRows - 1, T - 1);
  const int qhi = W < 0 ? T - 1 : min(T - 1, kl + W);
  for (int g = 0; g < G; ++g) {
    const int h = kvh * G + g;
    const float *Qb = Q + (long long)b * T * qs + (long long)h * D;
    const float *dOb = dO + (long long)b * T * qs + (long long)h * D;
    for (int i0 = k0; i0 <= qhi; i0 += kChunk) {
      __syncthreads();
      stage<D>(qsh, Qb, qs, i0, T);
      stage<D>(gsh, dOb, qs, i0, T);
      if (threadIdx.x < kChunk) {
        const int i = i0 + threadIdx.x;
        lsh[threadIdx.x] = i < T ? LSE[((long long)b * H + h) * T + i] : 0.f;
        dsh[threadIdx.x] = i < T ? delta[((long long)b * H + h) * T + i] : 0.f;
      }
      __syncthreads();
      for (int ii = 0; ii < kChunk && i0 + ii <= qhi; ++ii) {
        const int i = i0 + ii;
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < P; ++d) {
          s += qsh[ii * D + part * P + d] * kk[d];
          dp += gsh[ii * D + part * P + d] * vv[d];
        }
        s = quad_sum(s) * scale;
        dp = quad_sum(dp);
        if (!(valid && visible(i, j, W))) continue;
        const float p = expf(s - lsh[ii]);
        const float ds = p * (dp - dsh[ii]);
        for (int d = 0; d < P; ++d) {
          dv[d] += p * gsh[ii * D + part * P + d];
          dk[d] += ds * qsh[ii * D + part * P + d];
        }
      }
    }
  }
  if (!valid) return;
  for (int d = 0; d < P; ++d) {
    const long long off = ((long long)b * T + j) * kvs + (long long)kvh * D + part * P + d;
    dK[off] = dk[d] * scale;
    dV[off] = dv[d];
  }
}

template <int D>
hipError_t fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse, const AttnShape &sh,
                   hipStream_t s) {
  const long long nqb = (sh.T + kRows - 1) / kRows;
  const long long blocks = nqb * sh.B * sh.H;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_f32_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, s, q, k, v, o, lse, sh.B, sh.T, sh.H,
                     sh.KV, sh.window, sh.scale);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_f32(const float *q, const float *k, const float *v, const float *o, const float *lse,
                   const float *dout, float *dq, float *dk, float *dv, float *delta, const AttnShape &sh,
                   int stages, hipStream_t s) {
  const long long rows = (long long)sh.B * sh.T * sh.H;
  const long long nqb = (sh.T + kRows - 1) / kRows;
  const long long dblocks = (rows + kRows - 1) / kRows;
  const long long qblocks = nqb * sh.B * sh.H, kblocks = nqb * sh.B * sh.KV;
  if (dblocks > 0x7fffffffLL || qblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (stages & kBwdDelta)
    hipLaunchKernelGGL(delta_f32_kernel<D>, dim3((unsigned)dblocks), dim3(256), 0, s, o, dout, delta, sh.B, sh.T,
                     sh.H);
  if (stages & kBwdDkDv)
    hipLaunchKernelGGL(dkdv_f32_kernel<D>, dim3((unsigned)kblocks), dim3(256), 0, s, q, k, v, dout, lse, delta, dk, dv,
                     sh.B, sh.T, sh.H, sh.KV, sh.window, sh.scale);
  if (stages & kBwdDq)
    hipLaunchKernelGGL(dq_f32_kernel<D>, dim3((unsigned)qblocks), dim3(256), 0, s, q, k, v, dout, lse, delta, dq, sh.B,
                     sh.T, sh.H, sh.KV, sh.window, sh.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse, const AttnShape &sh,
                          hipStream_t s) {
  return sh.D == 64 ? fwd_f32<64>(q, k, v, o, lse, sh, s) : fwd_f32<128>(q, k, v, o, lse, sh, s);
}

hipError_t launch_bwd_f32(const float *q, const float *k, const float *v, const float *o, const float *lse,
                          const float *dout, float *dq, float *dk, float *dv, float *delta, const AttnShape &sh,
                          int stages, hipStream_t s) {
  return sh.D == 64 ? bwd_f32<64>(q, k, v, o, lse, dout, dq, dk, dv, delta, sh, stages, s)
                    : bwd_f32<128>(q, k, v, o, lse, dout, dq, dk, dv, delta, sh, stages, s);
}

}  // namespace ncattn
