// Attention forward, bf16 in/out, fp32 accumulation, head_dim 128, gfx950 MFMA.
//
// Computes, per query head h (kv head h / G) and query row i,
//   O_i = sum_j softmax_j(scale * q_i . k_j) v_j,  LSE_i = log sum_j exp(scale q_i . k_j)
// over the visible keys j <= i, i - j <= W ("nanoGPT Administrator & Developer
// Guide", section 8, CausalSelfAttention; "nanochat Admin & Developer Guide",
// sections 3 and 6 for windows and GQA).  The softmax is evaluated online over key
// tiles (an exact reformulation of the dense one).
//
// Work decomposition: one workgroup (4 waves) per (b, h, 128-row query block);
// wave w owns query rows 32w..32w+31 of the block.  Key/value tiles of 64 rows
// are double-buffered in LDS.  Each wave computes S^T = K Q^T (keys as MFMA rows,
// queries as columns) so that every lane holds one query's scores: the row max and
// row sum are lane-local plus one exchange with lane l^32, and the probabilities
// feed O^T += V^T P^T directly as the MFMA B operand (V^T comes from LDS with
// transposing reads).  Tiles entirely outside a wave's window are skipped; masks
// are applied only on tiles that straddle the causal diagonal or window edge.
#include "attn_tiles.hpp"
#include "internal.hpp"

namespace ncattn {

namespace {

constexpr int kBlockM = 128;
constexpr float kRescaleThreshold = 8.0f;  // log2 units: lazily rescale O when the max grows by > 2^8

__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(const uint16_t *__restrict__ Q,
                                                               const uint16_t *__restrict__ K,
                                                               const uint16_t *__restrict__ V,
                                                               uint16_t *__restrict__ O, float *__restrict__ LSE,
                                                               int B, int T, int H, int KV, int W, float scale) {
  __shared__ __attribute__((aligned(16))) char smem[4 * kTileBytes];  // [buf][K|V]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nqb = (T + kBlockM - 1) / kBlockM;
  const int BH = B * H;
  const int qblk = nqb - 1 - (int)(blockIdx.x / BH);  // heaviest (latest) query blocks first
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / H;
  const int h = bh % H;
  const int kvh = h / (H / KV);
  const int q0 = qblk * kBlockM;
  const int qw0 = q0 + 32 * wave;          // first query row of this wave
  const int q_lane = qw0 + (lane & 31);    // the query row this lane holds
  const int hh = lane >> 5;
  const float c = scale * kLog2e;

  const long long q_stride = (long long)H * kD;
  const long long kv_stride = (long long)KV * kD;
  const uint16_t *Kb = K + (long long)b * T * kv_stride + (long long)kvh * kD;
  const uint16_t *Vb = V + (long long)b * T * kv_stride + (long long)kvh * kD;

  // Q^T operand in registers: lane holds q row q_lane, d = 16 s + 8 hh + [0, 8).
  bf16x8 qreg[8];
  {
    const bool valid = q_lane < T;
    const uint16_t *qp = Q + ((long long)b * T + (valid ? q_lane : 0)) * q_stride + (long long)h * kD + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 w = valid ? *(const u32x4 *)(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u};
      qreg[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // Key tiles this block needs.
  const int q_last_blk = min(q0 + kBlockM - 1, T - 1);
  const int k_lo = W < 0 ? 0 : max(0, q0 - W);
  const int t0 = k_lo / kTileN;
  const int t1 = q_last_blk / kTileN;
  const int qw_last = min(qw0 + 31, T - 1);
  const bool wave_active = qw0 < T;

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of raw scores (both half-waves agree)
  float l_run = 0.f;        // this lane's partial row sum (its 32 of every 64 keys)

  TileRegs kr, vr;
  tile_load(kr, Kb, kv_stride, t0 * kTileN, T, tid);
  tile_load(vr, Vb, kv_stride, t0 * kTileN, T, tid);
  tile_store_lds(smem, kr, tid);
  tile_store_lds(smem + kTileBytes, vr, tid);
  __syncthreads();

  for (int t = t0; t <= t1; ++t) {
    const int buf = (t - t0) & 1;
    const char *Ks = smem + buf * 2 * kTileBytes;
    const char *Vs = Ks + kTileBytes;
    const bool has_next = t < t1;
    if (has_next) {
      tile_load(kr, Kb, kv_stride, (t + 1) * kTileN, T, tid);
      tile_load(vr, Vb, kv_stride, (t + 1) * kTileN, T, tid);
    }
    const int k0 = t * kTileN;
    const bool skip = !wave_active || k0 > qw_last || (W >= 0 && qw0 - (k0 + kTileN - 1) > W);
    if (!skip) {
      const bool need_mask = !(k0 + kTileN - 1 <= qw0 && (W < 0 || qw_last - k0 <= W));
      // S^T = K Q^T for the 64 keys of the tile: two 32-key blocks.
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) acc = mfma32(lds_row_operand(Ks, 32 * kb, s, lane), qreg[s], acc);
        sacc[kb] = acc;
      }
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = k0 + 32 * kb + 8 * (e >> 2) + 4 * hh + (e & 3);
            const bool vis = key <= q_lane && (W < 0 || q_lane - key <= W);
            if (!vis) sacc[kb][e] = -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kb][e]);
      mt = fmaxf(mt, shfl_xor(mt, 32));
      // Lazy rescale: move the reference max only when it grows by more than
      // 2^kRescaleThreshold in probability terms (exact either way: the same
      // reference scales O and l).
      const bool grow = mt > m_run + kRescaleThreshold / c;
      if (__any(grow)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_new) * c);
        if (m_new != m_run) {
          l_run *= alpha;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
          m_run = m_new;
        }
      }
      const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = fast_exp2(__builtin_fmaf(sacc[kb][e], c, -mc));
          sacc[kb][e] = p;
          ls += p;
        }
      l_run += ls;
      // O^T += V^T P^T over the 4 key steps of 16.
#pragma unroll
      for (int cs = 0; cs < 4; ++cs) {
        const bf16x8 pb = acc_to_operand(sacc[cs >> 1], cs & 1);
#pragma unroll
        for (int db = 0; db < 4; ++db) oacc[db] = mfma32(lds_col_operand(Vs, 32 * db, cs, lane), pb, oacc[db]);
      }
    }
    if (has_next) {
      char *nxt = smem + (buf ^ 1) * 2 * kTileBytes;
      tile_store_lds(nxt, kr, tid);
      tile_store_lds(nxt + kTileBytes, vr, tid);
    }
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_tot = l_run + shfl_xor(l_run, 32);
  const float inv_l = 1.f / l_tot;
  if (q_lane < T) {
    uint16_t *op = O + ((long long)b * T + q_lane) * q_stride + (long long)h * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * i + 4 * hh;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * i + 0] * inv_l, oacc[db][4 * i + 1] * inv_l);
        w[1] = pack_bf16x2(oacc[db][4 * i + 2] * inv_l, oacc[db][4 * i + 3] * inv_l);
        *(u32x2 *)(op + d) = w;
      }
    if (hh == 0) LSE[((long long)b * H + h) * T + q_lane] = m_run * scale + logf(l_tot);
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, const AttnShape &sh,
                           hipStream_t s) {
  const int nqb = (sh.T + kBlockM - 1) / kBlockM;
  const long long blocks = (long long)nqb * sh.B * sh.H;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t *)q,
                     (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)o, lse, sh.B, sh.T, sh.H, sh.KV, sh.window,
                     sh.scale);
  return hipGetLastError();
}

}  // namespace ncattn
