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
// lane and reused for all H + KV rows.  The angle is formed in turns and
// reduced to [-1/2, 1/2] in fp64 (positions reach ~10^4 radians), then sin/cos
// by the hardware (v_sin_f32 / v_cos_f32) in fp32.
//
// The backward (same layout) takes the forward's inputs x and the gradients dy
// of its outputs and writes dx over dy: dn = R^T dy (pairs rotated by -theta),
// then dx = (g / r) (dn - x (dn . x) / (D r^2)), r = sqrt(mean(x^2) + eps), the
// two row sums (x . x and dn . x) reduced together.
#include "device_common.hpp"
#include "internal.hpp"

namespace ncattn {

struct InvFreq {
  double v[64];  // base^(-2j/D) / (2 pi): turns of the rotation per position
};

// Optional output of the forward: 1/r = 1/sqrt(mean(x^2) + eps) of every row,
// at rstd[token * stride + head] for q rows and [token * stride + k_off + kv head]
// for k rows (stride = n_head + n_kv_head, k_off = n_head for the layout
// [B][T][n_head + n_kv_head]).
struct RstdOut {
  float *rstd;
  long long stride;
  int k_off;
};

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

// cos / sin of the lane's 4 angles: pos * w[i] turns, reduced to [-1/2, 1/2] in
// fp64 (positions reach ~10^4 radians), then the hardware sin / cos of a turn
// fraction (v_sin_f32 / v_cos_f32 take their argument in turns).
__device__ __forceinline__ void rope_cos_sin(double pos, const double (&w)[4], float (&c)[4], float (&s)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    double turns = pos * w[i];
    turns -= rint(turns);
    const float tf = (float)turns;
    s[i] = __builtin_amdgcn_sinf(tf);
    c[i] = __builtin_amdgcn_cosf(tf);
  }
}

// Sum over the R lanes of a row (R = 8 or 16: aligned groups within a DPP row),
// every lane of the group receiving it: quad permutes, then half-row and row
// mirrors.
template <int R>
__device__ __forceinline__ float row_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
  if constexpr (R == 16)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, true));  // row_mirror
  return x;
}

// The rows of a token are walked in groups of kPasses passes of ROWS rows; every
// load of a group is issued before its first row is reduced, so that a wave keeps
// several passes of q/k in flight.  Rows past the last one re-read it and are not
// written.
constexpr int kPasses = 4;

template <int D, bool BF16>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(void *__restrict__ qp, void *__restrict__ kp, int B, int T,
                                                          int H, int KV, const int32_t *__restrict__ pos_offset,
                                                          InvFreq inv_freq, float eps, float gain, RstdOut ro) {
  constexpr int R = D / 8;          // lanes per row
  constexpr int ROWS = 64 / R;      // rows per wave pass
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

  for (long long tok = wave; tok < ntok; tok += nwaves) {
    const int b = (int)(tok / T);
    const int t = (int)(tok % T);
    float c[4], s[4];
    rope_cos_sin((double)((pos_offset ? pos_offset[b] : 0) + t), w, c, s);
    for (int row0 = 0; row0 < nrows; row0 += ROWS * kPasses) {
      float a[kPasses][4], bb[kPasses][4];
      long long off[kPasses];
#pragma unroll
      for (int p = 0; p < kPasses; ++p) {
        const int row = min(row0 + p * ROWS + slot, nrows - 1);
        off[p] = row < H ? ((long long)tok * H + row) * D : ((long long)tok * KV + (row - H)) * D;
        load_pairs<D, BF16>(row < H ? qp : kp, off[p], j0, a[p], bb[p]);
      }
#pragma unroll
      for (int p = 0; p < kPasses; ++p) {
        const int row = row0 + p * ROWS + slot;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) ss += a[p][i] * a[p][i] + bb[p][i] * bb[p][i];
        ss = row_sum<R>(ss);
        const float rs = 1.f / sqrtf(ss / (float)D + eps);
        const float inv = gain * rs;
        if (ro.rstd != nullptr && r == 0 && row < nrows)
          ro.rstd[tok * ro.stride + (row < H ? row : ro.k_off + row - H)] = rs;
        float ya[4], yb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float xa = a[p][i] * inv, xb = bb[p][i] * inv;
          ya[i] = xa * c[i] - xb * s[i];
          yb[i] = xa * s[i] + xb * c[i];
        }
        if (row < nrows) store_pairs<D, BF16>(row < H ? qp : kp, off[p], j0, ya, yb);
      }
    }
  }
}

// FROM_Y: qp / kp hold the forward's outputs y (not its inputs x) and rs.rstd
// each row's 1/r.  With n = R^T y = g x / r the same gradient is
//   dx = (g / r) R^T (dy - y (dy . y) / (g^2 D))
// (dn . x / r = (R^T dy) . (R^T y) / g = dy . y / g: the rotation keeps dot products).
template <int D, bool BF16, bool FROM_Y>
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(void *__restrict__ dqp, void *__restrict__ dkp,
                                                              const void *__restrict__ qp,
                                                              const void *__restrict__ kp, int B, int T, int H,
                                                              int KV, const int32_t *__restrict__ pos_offset,
                                                              InvFreq inv_freq, float eps, float gain, RstdOut rs) {
  constexpr int R = D / 8;
  constexpr int ROWS = 64 / R;
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

  for (long long tok = wave; tok < ntok; tok += nwaves) {
    const int b = (int)(tok / T);
    const int t = (int)(tok % T);
    float c[4], s[4];
    rope_cos_sin((double)((pos_offset ? pos_offset[b] : 0) + t), w, c, s);
    for (int row0 = 0; row0 < nrows; row0 += ROWS * kPasses) {
      float xa[kPasses][4], xb[kPasses][4], ga[kPasses][4], gb[kPasses][4];
      long long off[kPasses];
#pragma unroll
      for (int p = 0; p < kPasses; ++p) {
        const int row = min(row0 + p * ROWS + slot, nrows - 1);
        off[p] = row < H ? ((long long)tok * H + row) * D : ((long long)tok * KV + (row - H)) * D;
        load_pairs<D, BF16>(row < H ? qp : kp, off[p], j0, xa[p], xb[p]);
        load_pairs<D, BF16>(row < H ? dqp : dkp, off[p], j0, ga[p], gb[p]);
      }
#pragma unroll
      for (int p = 0; p < kPasses; ++p) {
        const int row = row0 + p * ROWS + slot;
        float da[4], db[4];
        if constexpr (!FROM_Y) {
          float na[4], nb[4];
          float ss = 0.f, dot = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            na[i] = ga[p][i] * c[i] + gb[p][i] * s[i];  // rotation by -theta
            nb[i] = gb[p][i] * c[i] - ga[p][i] * s[i];
            ss += xa[p][i] * xa[p][i] + xb[p][i] * xb[p][i];
            dot += na[i] * xa[p][i] + nb[i] * xb[p][i];
          }
          ss = row_sum<R>(ss);
          dot = row_sum<R>(dot);
          const float r2 = ss / (float)D + eps;
          const float g_r = gain / sqrtf(r2);
          const float coef = dot / ((float)D * r2);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            da[i] = g_r * (na[i] - xa[p][i] * coef);
            db[i] = g_r * (nb[i] - xb[p][i] * coef);
          }
        } else {
          // xa / xb hold y here
          float dot = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) dot += ga[p][i] * xa[p][i] + gb[p][i] * xb[p][i];
          dot = row_sum<R>(dot);
          const int rr = min(row, nrows - 1);
          const float g_r = gain * rs.rstd[tok * rs.stride + (rr < H ? rr : rs.k_off + rr - H)];
          const float coef = gain == 0.f ? 0.f : dot / (gain * gain * (float)D);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float ua = ga[p][i] - xa[p][i] * coef, ub = gb[p][i] - xb[p][i] * coef;
            da[i] = g_r * (ua * c[i] + ub * s[i]);  // rotation by -theta
            db[i] = g_r * (ub * c[i] - ua * s[i]);
          }
        }
        if (row < nrows) store_pairs<D, BF16>(row < H ? dqp : dkp, off[p], j0, da, db);
      }
    }
  }
}

hipError_t launch_qknorm_rope_bwd(void *dq, void *dk, const void *q, const void *k, int B, int T, int H, int KV,
                                  int D, const int32_t *pos_offset, const double *inv_freq_host, float eps,
                                  float gain, bool bf16, hipStream_t s, const float *rstd, long long rstd_stride,
                                  int rstd_k_off) {
  InvFreq f;
  for (int j = 0; j < 64; ++j) f.v[j] = j < D / 2 ? inv_freq_host[j] / 6.283185307179586 : 0.0;
  const RstdOut rs{(float *)rstd, rstd_stride, rstd_k_off};
  const long long ntok = (long long)B * T;
  long long blocks = (ntok + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  dim3 grid((unsigned)blocks), block(256);
#define NC_QKB(DD, BF, FY)                                                                                     \
  hipLaunchKernelGGL((qknorm_rope_bwd_kernel<DD, BF, FY>), grid, block, 0, s, dq, dk, q, k, B, T, H, KV, pos_offset, \
                     f, eps, gain, rs)
  const bool fy = rstd != nullptr;
  if (D == 128) {
    if (bf16) { if (fy) NC_QKB(128, true, true); else NC_QKB(128, true, false); }
    else { if (fy) NC_QKB(128, false, true); else NC_QKB(128, false, false); }
  } else {
    if (bf16) { if (fy) NC_QKB(64, true, true); else NC_QKB(64, true, false); }
    else { if (fy) NC_QKB(64, false, true); else NC_QKB(64, false, false); }
  }
#undef NC_QKB
  return hipGetLastError();
}

hipError_t launch_qknorm_rope(void *q, void *k, int B, int T, int H, int KV, int D, const int32_t *pos_offset,
                              const double *inv_freq_host, float eps, float gain, bool bf16, hipStream_t s,
                              float *rstd, long long rstd_stride, int rstd_k_off) {
  InvFreq f;
  for (int j = 0; j < 64; ++j) f.v[j] = j < D / 2 ? inv_freq_host[j] / 6.283185307179586 : 0.0;
  const RstdOut ro{rstd, rstd_stride, rstd_k_off};
  const long long ntok = (long long)B * T;
  // 4 waves per block; enough blocks to fill 256 CUs several times, each wave
  // then walks several tokens so its per-lane setup is amortised.
  long long blocks = (ntok + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  dim3 grid((unsigned)blocks), block(256);
  if (D == 128) {
    if (bf16) hipLaunchKernelGGL((qknorm_rope_kernel<128, true>), grid, block, 0, s, q, k, B, T, H, KV, pos_offset, f, eps, gain, ro);
    else hipLaunchKernelGGL((qknorm_rope_kernel<128, false>), grid, block, 0, s, q, k, B, T, H, KV, pos_offset, f, eps, gain, ro);
  } else {
    if (bf16) hipLaunchKernelGGL((qknorm_rope_kernel<64, true>), grid, block, 0, s, q, k, B, T, H, KV, pos_offset, f, eps, gain, ro);
    else hipLaunchKernelGGL((qknorm_rope_kernel<64, false>), grid, block, 0, s, q, k, B, T, H, KV, pos_offset, f, eps, gain, ro);
  }
  return hipGetLastError();
}

}  // namespace ncattn
