// Attention forward with fp8 inputs: q, k, v stored as OCP e4m3 bytes with one
// descale factor per tensor, o in bf16, fp32 accumulation, head_dim 128, on the
// gfx950 fp8 MFMA (v_mfma_f32_32x32x64_f8f6f4).
//
// Computes, per query head h (kv head h / G) and query row i, with x = dx x8
// the value an fp8 tensor x8 with descale dx stands for,
//   O_i = sum_j softmax_j(scale q_i . k_j) v_j,  LSE_i = log sum_j exp(scale q_i . k_j)
// over the visible keys j <= i, i - j <= W: the forward of the bf16 kernel on
// those values ("nanochat Admin & Developer Guide", section 6, Attention: FA3
// with SDPA fallback, which runs in bf16 or fp8).
//
// Work decomposition and launch order are the bf16 forward's: one workgroup of 4
// waves per (b, h, 128-row query block), wave w owning rows 32w..32w+31, the
// query rows' fp8 bytes held in registers as the MFMA B operand of S^T = K Q^T.
// A tile of 64 keys is 64 x 128 bytes for K and for V, the byte geometry of a
// 64-wide bf16 tile, so both are copied global -> LDS directly with that tile's
// chunk permutation.  One 32x32x64 MFMA contracts 64 positions: S^T of a tile is
// 2 key blocks x 2 steps over the head, and O^T += V^T P one MFMA per 32-wide
// block of the head over all 64 keys of the tile.
//
// The contraction positions of an fp8 MFMA pair lane l's byte p of A with lane
// l's byte p of B (rows / columns l % 32, halves l / 32), so any assignment of
// keys to (half, byte) works as long as A and B share it.  P is taken straight
// from the S^T accumulators: lane (q, half h) holds keys 32 kb + 8 i + 4 h + j at
// element 4 i + j of block kb, and becomes byte p = 16 kb + 4 i + j of the B
// operand.  The A operand V^T gathers the same keys for its row d with the
// 8-bit transposing LDS read: in each group of 16 lanes, byte k of lane i's
// result is byte i % 8 of the 8 bytes addressed by lane 2 k + i / 8, so lane
// 2 k + e points at the 8 bytes of row key(8 r + k) that hold columns
// 16 (lane group) + 8 e .. + 8 of the head, and four such reads (r = 0..3) fill
// the 32 bytes.
//
// Softmax: each row keeps an exponent reference m (O and the row sum are
// rescaled when it moves) that trails the running row max by less than 0.8 in
// base-2 exponent units, so P = exp2((s - m) c) < 2^0.8 = 1.74; P is computed
// already multiplied by 2^8 (2^8 P <= 446 fits e4m3's largest finite value, 448)
// and converted to fp8 by rounding to nearest, which keeps P >= 2^-14 in e4m3's
// normal range; the row sum is taken over the same fp32 2^8 P, so the factor
// cancels in O.  Moving m only when the max has grown by 0.8 spares most tiles
// the rescale once a row's first tiles have been seen.  Each probability thus
// enters O with a relative error of at most 2^-4 (e4m3 keeps 3 fraction bits),
// or an absolute one of at most 2^-18 (relative to the reference) below the
// normal range.
#include "attn_tiles.hpp"
#include "internal.hpp"

namespace ncattn {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kRows8 = 128;  // query rows per workgroup
using T8 = Geom<64>;         // a 64-key tile of 128-byte rows

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const char *p) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)(p));
}

// Key held at byte p of a lane in half h of the P (and V^T) operands.
__device__ __forceinline__ int pv_key(int p, int h) {
  return 32 * (p >> 4) + 8 * ((p >> 2) & 3) + 4 * h + (p & 3);
}

// -inf on the elements of a straddling tile that are not visible (element e of
// sacc[kb] is key k0 + 32 kb + 8 (e >> 2) + 4 hh + (e & 3) of query q_lane).
__device__ __forceinline__ void mask_tile_fp8(f32x16 (&sacc)[2], int k0, int q_lane, int W, int hh) {
  const int d0 = k0 + 4 * hh - q_lane;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int off = 32 * kb + 8 * (e >> 2) + (e & 3);
      const bool vis = (d0 <= -off) & ((W < 0) | (d0 + W >= -off));
      sacc[kb][e] = vis ? sacc[kb][e] : -INFINITY;
    }
}

// c: scale dq dk log2 e (raw scores to exponent base 2); lse_scale: scale dq dk;
// o_scale: dv.
__global__ __launch_bounds__(256, 2) void attn_fwd_fp8_kernel(const uint8_t *__restrict__ Q,
                                                             const uint8_t *__restrict__ K,
                                                             const uint8_t *__restrict__ V,
                                                             uint16_t *__restrict__ O, float *__restrict__ LSE,
                                                             int B, int T, int H, int KV, int W, float c,
                                                             float lse_scale, float o_scale) {
  __shared__ __attribute__((aligned(1024))) char kb0[T8::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char kb1[T8::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vb0[T8::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vb1[T8::kTileBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;
  // launch order as the bf16 forward's: heaviest query blocks first, the G heads
  // of a (b, kv head) B KV blocks apart
  const int nqb = (T + kRows8 - 1) / kRows8;
  const int G = H / KV;
  const int BH = B * H;
  const int BKV = B * KV;
  const int qblk = nqb - 1 - (int)(blockIdx.x / BH);
  const int jb = (int)(blockIdx.x % BH);
  const int bkv = jb % BKV;
  const int b = bkv / KV;
  const int kvh = bkv % KV;
  const int h = kvh * G + jb / BKV;
  const int q0 = qblk * kRows8;
  const int qw0 = q0 + 32 * wave;
  const int q_lane = qw0 + (lane & 31);
  const long long q_stride = (long long)H * 128;  // bytes
  const long long kv_stride = (long long)KV * 128;

  const TileSrc ksrc = make_tile_src((const uint16_t *)(K + (long long)b * T * kv_stride + (long long)kvh * 128),
                                     kv_stride / 2, T);
  const TileSrc vsrc = make_tile_src((const uint16_t *)(V + (long long)b * T * kv_stride + (long long)kvh * 128),
                                     kv_stride / 2, T);
  const int voff = tile_lane_voff<64>(ksrc.stride, tid);

  // key tiles of the block, and the contiguous range of them this wave needs
  const int p_last_blk = min(q0 + kRows8 - 1, T - 1);
  const int t0 = (W < 0 ? 0 : max(0, q0 - W)) / kTileN;
  const int t1 = p_last_blk / kTileN;
  const int pw_last = min(qw0 + 31, T - 1);
  const bool wave_active = qw0 < T;
  const int tw0 = max(t0, (W < 0 ? 0 : max(0, qw0 - W)) / kTileN);
  const int tw1 = wave_active ? pw_last / kTileN : t0 - 1;
  auto in_range = [&](int t) { return t >= tw0 && t <= tw1; };
  auto masked = [&](int t) {
    const int k0 = t * kTileN;
    return !(k0 + kTileN - 1 <= qw0 && (W < 0 || pw_last - k0 <= W));
  };

  tile_load_lds<64>(kb0, ksrc, voff, t0 * kTileN);
  tile_load_lds<64>(vb0, vsrc, voff, t0 * kTileN);

  // Q^T operand: lane (row q_lane, half hh) holds head bytes 64 m + 32 hh + [0, 32) for step m
  i32x8 qreg[2];
  {
    const int qr = min(q_lane, T - 1);
    const uint8_t *qp = Q + ((long long)b * T + qr) * q_stride + (long long)h * 128 + 32 * hh;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const i32x4 lo = *(const i32x4 *)(qp + 64 * m);
      const i32x4 hi = *(const i32x4 *)(qp + 64 * m + 16);
      qreg[m] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  // LDS offsets: K rows (lane & 31) of each key block at chunks 4 m + 2 hh + {0, 1};
  // V^T source addresses of the transposing reads (row pv_key(8 r + k, hh), the
  // 8 bytes at head column 32 db + 16 (lane group & 1) + 8 e)
  int koff[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int x = 0; x < 2; ++x) koff[m][x] = swz<64>(lane & 31, 4 * m + 2 * hh + x);
  int voffr[4][4];
  {
    const int s = lane & 15, k = s >> 1, e = s & 1, g1 = (lane >> 4) & 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = pv_key(8 * r + k, hh);
#pragma unroll
      for (int db = 0; db < 4; ++db) voffr[r][db] = swz<64>(row, 2 * db + g1) + 8 * e;
    }
  }

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // exponent reference of the raw scores (both halves of a row agree)
  float l_run = 0.f;        // this lane's partial row sum of 2^8 P (its 32 of every 64 keys)

  lds_loads_done_barrier();

  auto step = [&](const char *kc, const char *vc, char *kn, char *vn, int t) {
    if (t + 1 <= t1) {
      tile_load_lds<64>(kn, ksrc, voff, (t + 1) * kTileN);
      tile_load_lds<64>(vn, vsrc, voff, (t + 1) * kTileN);
    }
    if (in_range(t)) {
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const i32x4 lo = *(const i32x4 *)(kc + koff[m][0] + 32 * kb * T8::kRowBytes);
          const i32x4 hi = *(const i32x4 *)(kc + koff[m][1] + 32 * kb * T8::kRowBytes);
          sacc[kb] = mfma_fp8(i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}, qreg[m], sacc[kb]);
        }
      }
      if (masked(t)) mask_tile_fp8(sacc, t * kTileN, q_lane, W, hh);
      float tmax = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, sacc[kb][e]);
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      // move the reference when the max has grown by 0.8 (base-2 units) or more,
      // or on the first visible tile (alpha = exp2(-inf) = 0 on zeros)
      const bool move = (tmax - m_run) * c >= 0.8f;
      if (__any(move)) {
        const float alpha = move ? fast_exp2((m_run - tmax) * c) : 1.f;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
        l_run *= alpha;
        m_run = move ? tmax : m_run;
      }
      // 2^8 P = exp2((s - m) c + 8)
      const float nmc = m_run == -INFINITY ? 0.f : 8.f - m_run * c;
      i32x8 pop;
      float ls = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, e0 = 4 * (w & 3);
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = fast_exp2(__builtin_fmaf(sacc[kb][e0 + j], c, nmc));
          ls += p[j];
        }
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        x = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], x, true);
        pop[w] = x;
      }
      l_run += ls;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        i32x8 a;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const i32x2 v = lds_read_tr8(vc + voffr[r][db]);
          a[2 * r] = v[0];
          a[2 * r + 1] = v[1];
        }
        oacc[db] = mfma_fp8(a, pop, oacc[db]);
      }
    }
    lds_loads_done_barrier();
  };
  for (int t = t0; t <= t1; t += 2) {
    step(kb0, vb0, kb1, vb1, t);
    if (t + 1 > t1) break;
    step(kb1, vb1, kb0, vb0, t + 1);
  }

  if (!wave_active || q_lane >= T) return;
  const float l_tot = l_run + shfl_xor(l_run, 32);
  const float inv = o_scale / l_tot;
  uint16_t *op = O + ((long long)b * T + q_lane) * (long long)H * 128 + (long long)h * 128;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * hh;
      u32x2 w;
      w[0] = pack_bf16x2(oacc[db][4 * i + 0] * inv, oacc[db][4 * i + 1] * inv);
      w[1] = pack_bf16x2(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
      *(u32x2 *)(op + d) = w;
    }
  if (hh == 0 && LSE) LSE[((long long)b * H + h) * T + q_lane] = m_run * lse_scale + logf(l_tot) - 8.f * kLn2;
}

}  // namespace

hipError_t launch_fwd_fp8(const void *q, const void *k, const void *v, float q_descale, float k_descale,
                          float v_descale, void *o, float *lse, const AttnShape &sh, hipStream_t s) {
  if (sh.D != 128) return hipErrorInvalidValue;
  const long long blocks = (long long)((sh.T + kRows8 - 1) / kRows8) * sh.B * sh.H;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const float sc = sh.scale * q_descale * k_descale;
  hipLaunchKernelGGL(attn_fwd_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t *)q,
                     (const uint8_t *)k, (const uint8_t *)v, (uint16_t *)o, lse, sh.B, sh.T, sh.H, sh.KV,
                     sh.window, sc * kLog2e, sc, v_descale);
  return hipGetLastError();
}

}  // namespace ncattn
