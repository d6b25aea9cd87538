// QK-norm + RoPE, in place, for q [B][T][H][D] and k [B][T][KV][D].
//
// "nanochat Admin & Developer Guide", section 3 "The GPT Model (Internals)":
// queries and keys are RMS-normalised (weightless RMSNorm, per head) and carry
// rotary position embeddings.  Each row x becomes
//     y = gain * x / sqrt(mean(x^2) + eps),
//     (y_j, y_{j+D/2}) rotated by +theta_j, theta_j = pos * base^(-2j/D).
//
// HBM-bound elementwise work with a row reduction over D.  Layout of the work:
// one wave walks tokens (b, t) in a grid-stride loop; for each token it covers
// the H query rows and KV key rows, D/8 lanes per row.  A lane owns the four
// pair indices j in [4r, 4r+4) of its row slot r and their partners j + D/2,
// so the rotation is lane-local and cos/sin are computed once per token per
// lane and reused for all H + KV rows.  The angle is formed and reduced to
// [-pi, pi] in fp64 (positions reach ~10^4 radians), then sin/cos in fp32.
//
// The backward (same layout) takes the forward's inputs x and the gradients dy
// of its outputs and writes dx over dy: dn = R^T dy (pairs rotated by -theta),
// then dx = (g / r) (dn - x (dn . x) / (D r^2)), r = sqrt(mean(x^2) + eps), the
// two row sums (x . x and dn . x) reduced together.
#include "device_common.hpp"
#include "internal.hpp"

namespace ncattn {

struct InvFreq {
  double v[64];
};

template <int D, bool BF16>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(void *__restrict__ qp, void *__restrict__ kp, int B, int T,
                                                          int H, int KV, const int32_t *__restrict__ pos_offset,
                                                          InvFreq inv_freq, float eps, float gain) {
  constexpr int R = D / 8;          // lanes per row
  constexpr int ROWS = 64 / R;      // rows per wave pass
  constexpr int HALF = D / 2;
  const int lane = threadIdx.x & 63;
  const int slot = lane / R;        // row slot within the pass
  const int r = lane % R;           // which 4-pair group of the row
  const int j0 = 4 * r;
  double w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = inv_freq.v[j0 + i];

  const long long ntok = (long long)B * T;
  const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long long nwaves = ((long long)gridDim.x * blockDim.x) >> 6;
  const int nrows = H + KV;
  const double two_pi = 6.283185307179586;

  for (long long tok = wave; tok < ntok; tok += nwaves) {
    const int b = (int)(tok / T);
    const int t = (int)(tok % T);
    const double pos = (double)((pos_offset ? pos_offset[b] : 0) + t);
    float c[4], s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double th = pos * w[i];
      th -= two_pi * rint(th / two_pi);
      float tf = (float)th;
      s[i] = sinf(tf);
      c[i] = cosf(tf);
    }
    for (int row0 = 0; row0 < nrows; row0 += ROWS) {
      const int row = row0 + slot;
      if (row >= nrows) break;
      const bool isq = row < H;
      const long long base = isq ? ((long long)tok * H + row) * D : ((long long)tok * KV + (row - H)) * D;
      float a[4], bb[4];
      if constexpr (BF16) {
        uint16_t *x = (uint16_t *)(isq ? qp : kp) + base;
        u32x2 va = *(const u32x2 *)(x + j0);
        u32x2 vb = *(const u32x2 *)(x + HALF + j0);
        a[0] = lo_bf16(va[0]); a[1] = hi_bf16(va[0]); a[2] = lo_bf16(va[1]); a[3] = hi_bf16(va[1]);
        bb[0] = lo_bf16(vb[0]); bb[1] = hi_bf16(vb[0]); bb[2] = lo_bf16(vb[1]); bb[3] = hi_bf16(vb[1]);
      } else {
        float *x = (float *)(isq ? qp : kp) + base;
        f32x4 va = *(const f32x4 *)(x + j0);
        f32x4 vb = *(const f32x4 *)(x + HALF + j0);
#pragma unroll
        for (int i = 0; i < 4; ++i) { a[i] = va[i]; bb[i] = vb[i]; }
      }
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) ss += a[i] * a[i] + bb[i] * bb[i];
#pragma unroll
      for (int m = 1; m < R; m <<= 1) ss += shfl_xor(ss, m);
      const float inv = gain / sqrtf(ss / (float)D + eps);
      float ya[4], yb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xa = a[i] * inv, xb = bb[i] * inv;
        ya[i] = xa * c[i] - xb * s[i];
        yb[i] = xa * s[i] + xb * c[i];
      }
      if constexpr (BF16) {
        uint16_t *x = (uint16_t *)(isq ? qp : kp) + base;
        u32x2 oa, ob;
        oa[0] = pack_bf16x2(ya[0], ya[1]); oa[1] = pack_bf16x2(ya[2], ya[3]);
        ob[0] = pack_bf16x2(yb[0], yb[1]); ob[1] = pack_bf16x2(yb[2], yb[3]);
        *(u32x2 *)(x + j0) = oa;
        *(u32x2 *)(x + HALF + j0) = ob;
      } else {
        float *x = (float *)(isq ? qp : kp) + base;
        f32x4 oa, ob;
#pragma unroll
        for (int i = 0; i < 4; ++i) { oa[i] = ya[i]; ob[i] = yb[i]; }
        *(f32x4 *)(x + j0) = oa;
        *(f32x4 *)(x + HALF + j0) = ob;
      }
    }
  }
}

// Loads the lane's 4 pairs (x_j, x_{j+D/2}), j = j0..j0+3, of a row as fp32.
template <int D, bool BF16>
__device__ __forceinline__ void load_pairs(const void *base, long long off, int j0, float (&a)[4], float (&b)[4]) {
  constexpr int HALF = D / 2;
  if constexpr (BF16) {
    const uint16_t *x = (const uint16_t *)base + off;
    const u32x2 va = *(const u32x2 *)(x + j0);
    const u32x2 vb = *(const u32x2 *)(x + HALF + j0);
    a[0] = lo_bf16(va[0]); a[1] = hi_bf16(va[0]); a[2] = lo_bf16(va[1]); a[3] = hi_bf16(va[1]);
    b[0] = lo_bf16(vb[0]); b[1] = hi_bf16(vb[0]); b[2] = lo_bf16(vb[1]); b[3] = hi_bf16(vb[1]);
  } else {
    const float *x = (const float *)base + off;
    const f32x4 va = *(const f32x4 *)(x + j0);
    const f32x4 vb = *(const f32x4 *)(x + HALF + j0);
#pragma unroll
    for (int i = 0; i < 4; ++i) { a[i] = va[i]; b[i] = vb[i]; }
  }
}

template <int D, bool BF16>
__device__ __forceinline__ void store_pairs(void *base, long long off, int j0, const float (&a)[4], const float (&b)[4]) {
  constexpr int HALF = D / 2;
  if constexpr (BF16) {
    uint16_t *x = (uint16_t *)base + off;
    u32x2 oa, ob;
    oa[0] = pack_bf16x2(a[0], a[1]); oa[1] = pack_bf16x2(a[2], a[3]);
    ob[0] = pack_bf16x2(b[0], b[1]); ob[1] = pack_bf16x2(b[2], b[3]);
    *(u32x2 *)(x + j0) = oa;
    *(u32x2 *)(x + HALF + j0) = ob;
  } else {
    float *x = (float *)base + off;
    f32x4 oa, ob;
#pragma unroll
    for (int i = 0; i < 4; ++i) { oa[i] = a[i]; ob[i] = b[i]; }
    *(f32x4 *)(x + j0) = oa;
    *(f32x4 *)(x + HALF + j0) = ob;
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(void *__restrict__ dqp, void *__restrict__ dkp,
                                                              const void *__restrict__ qp,
                                                              const void *__restrict__ kp, int B, int T, int H,
                                                              int KV, const int32_t *__restrict__ pos_offset,
                                                              InvFreq inv_freq, float eps, float gain) {
  constexpr int R = D / 8;          // lanes per row
  constexpr int ROWS = 64 / R;      // rows per wave pass
  const int lane = threadIdx.x & 63;
  const int slot = lane / R;
  const int r = lane % R;
  const int j0 = 4 * r;
  double w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = inv_freq.v[j0 + i];

  const long long ntok = (long long)B * T;
  const long long wave = ((long long)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const long long nwaves = ((long long)gridDim.x * blockDim.x) >> 6;
  const int nrows = H + KV;
  const double two_pi = 6.283185307179586;

  for (long long tok = wave; tok < ntok; tok += nwaves) {
    const int b = (int)(tok / T);
    const int t = (int)(tok % T);
    const double pos = (double)((pos_offset ? pos_offset[b] : 0) + t);
    float c[4], s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double th = pos * w[i];
      th -= two_pi * rint(th / two_pi);
      const float tf = (float)th;
      s[i] = sinf(tf);
      c[i] = cosf(tf);
    }
    for (int row0 = 0; row0 < nrows; row0 += ROWS) {
      const int row = row0 + slot;
      if (row >= nrows) break;
      const bool isq = row < H;
      const long long off = isq ? ((long long)tok * H + row) * D : ((long long)tok * KV + (row - H)) * D;
      float xa[4], xb[4], ga[4], gb[4];
      load_pairs<D, BF16>(isq ? qp : kp, off, j0, xa, xb);
      load_pairs<D, BF16>(isq ? dqp : dkp, off, j0, ga, gb);
      float na[4], nb[4];
      float ss = 0.f, dot = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        na[i] = ga[i] * c[i] + gb[i] * s[i];   // rotation by -theta
        nb[i] = gb[i] * c[i] - ga[i] * s[i];
        ss += xa[i] * xa[i] + xb[i] * xb[i];
        dot += na[i] * xa[i] + nb[i] * xb[i];
      }
#pragma unroll
      for (int m = 1; m < R; m <<= 1) {
        ss += shfl_xor(ss, m);
        dot += shfl_xor(dot, m);
      }
      const float r2 = ss / (float)D + eps;
      const float g_r = gain / sqrtf(r2);
      const float coef = dot / ((float)D * r2);
      float da[4], db[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        da[i] = g_r * (na[i] - xa[i] * coef);
        db[i] = g_r * (nb[i] - xb[i] * coef);
      }
      store_pairs<D, BF16>(isq ? dqp : dkp, off, j0, da, db);
    }
  }
}

hipError_t launch_qknorm_rope_bwd(void *dq, void *dk, const void *q, const void *k, int B, int T, int H, int KV,
                                  int D, const int32_t *pos_offset, const double *inv_freq_host, float eps,
                                  float gain, bool bf16, hipStream_t s) {
  InvFreq f;
  for (int j = 0; j < 64; ++j) f.v[j] = j < D / 2 ? inv_freq_host[j] : 0.0;
  const long long ntok = (long long)B * T;
  long long blocks = (ntok + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  dim3 grid((unsigned)blocks), block(256);
  if (D == 128) {
    if (bf16) hipLaunchKernelGGL((qknorm_rope_bwd_kernel<128, true>), grid, block, 0, s, dq, dk, q, k, B, T, H, KV, pos_offset, f, eps, gain);
    else hipLaunchKernelGGL((qknorm_rope_bwd_kernel<128, false>), grid, block, 0, s, dq, dk, q, k, B, T, H, KV, pos_offset, f, eps, gain);
  } else {
    if (bf16) hipLaunchKernelGGL((qknorm_rope_bwd_kernel<64, true>), grid, block, 0, s, dq, dk, q, k, B, T, H, KV, pos_offset, f, eps, gain);
    else hipLaunchKernelGGL((qknorm_rope_bwd_kernel<64, false>), grid, block, 0, s, dq, dk, q, k, B, T, H, KV, pos_offset, f, eps, gain);
  }
  return hipGetLastError();
}

hipError_t launch_qknorm_rope(void *q, void *k, int B, int T, int H, int KV, int D, const int32_t *pos_offset,
                              const double *inv_freq_host, float eps, float gain, bool bf16, hipStream_t s) {
  InvFreq f;
  for (int j = 0; j < 64; ++j) f.v[j] = j < D / 2 ? inv_freq_host[j] : 0.0;
  const long long ntok = (long long)B * T;
  // 4 waves per block; enough blocks to fill 256 CUs several times, each wave
  // then walks several tokens so its per-lane setup is amortised.
  long long blocks = (ntok + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  dim3 grid((unsigned)blocks), block(256);
  if (D == 128) {
    if (bf16) hipLaunchKernelGGL((qknorm_rope_kernel<128, true>), grid, block, 0, s, q, k, B, T, H, KV, pos_offset, f, eps, gain);
    else hipLaunchKernelGGL((qknorm_rope_kernel<128, false>), grid, block, 0, s, q, k, B, T, H, KV, pos_offset, f, eps, gain);
  } else {
    if (bf16) hipLaunchKernelGGL((qknorm_rope_kernel<64, true>), grid, block, 0, s, q, k, B, T, H, KV, pos_offset, f, eps, gain);
    else hipLaunchKernelGGL((qknorm_rope_kernel<64, false>), grid, block, 0, s, q, k, B, T, H, KV, pos_offset, f, eps, gain);
  }
  return hipGetLastError();
}

}  // namespace ncattn
