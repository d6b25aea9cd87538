// Attention forward, bf16 in/out, fp32 accumulation, head_dim 128, gfx950 MFMA.
//
// Computes, per query head h (kv head h / G) and query row i,
//   O_i = sum_j softmax_j(scale * q_i . k_j) v_j,  LSE_i = log sum_j exp(scale q_i . k_j)
// over the visible keys j <= i, i - j <= W ("nanoGPT Administrator & Developer
// Guide", section 8, CausalSelfAttention; "nanochat Admin & Developer Guide",
// sections 3 and 6 for windows and GQA).  The softmax is evaluated online over key
// tiles (an exact reformulation of the dense one).
//
// Work decomposition: one workgroup (4 waves) per (b, h, 128-row query block),
// heaviest (latest) query blocks first; wave w owns query rows 32w..32w+31 of the
// block and keeps them in registers.  Key/value tiles of 64 rows are copied
// global -> LDS directly (no register staging), double-buffered, so the copy of
// tile t+1 overlaps the math on tile t.  Each wave computes S^T = K Q^T (keys as
// MFMA rows, queries as columns) so that every lane holds one query's scores: the
// row max and row sum are lane-local plus one exchange with lane l^32, and the
// probabilities feed O^T += V^T P^T directly as the MFMA B operand (V^T comes
// from LDS with transposing reads).  All LDS read addresses are per-lane
// constants computed once.  Tiles entirely outside a wave's window are skipped;
// masks are applied only on tiles that straddle the causal diagonal or the
// window edge.
#include "attn_tiles.hpp"
#include "internal.hpp"

namespace ncattn {

namespace {

constexpr int kBlockM = 128;
constexpr int kBufBytes = 2 * kTileBytes;  // K tile + V tile
constexpr float kRescaleThreshold = 8.0f;  // log2 units: rescale O only when the max grows by > 2^8

struct FwdState {
  f32x16 oacc[4];
  float m_run;  // running reference max of raw scores (both half-waves agree)
  float l_run;  // this lane's partial row sum (its 32 of every 64 keys)
};

// One 64-key tile: S^T, online softmax, O^T += V^T P^T.
template <bool kMask>
__device__ __forceinline__ void fwd_tile(FwdState &st, const char *ks, const char *vs, const TileLane &L,
                                         const bf16x8 (&qreg)[8], int k0, int q_lane, int W, float c, int hh) {
  f32x16 sacc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s)
      acc = mfma32(row_operand(ks, L, s, kb), qreg[s], acc);
    sacc[kb] = acc;
  }
  if constexpr (kMask) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 32 * kb + 8 * (e >> 2) + 4 * hh + (e & 3);
        const bool vis = key <= q_lane && (W < 0 || q_lane - key <= W);
        if (!vis) sacc[kb][e] = -INFINITY;
      }
  }
  float mt = sacc[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kb][e]);
  mt = fmaxf(mt, shfl_xor(mt, 32));
  // Lazy rescale: move the reference max only when it grows by more than
  // 2^kRescaleThreshold in probability terms (exact either way: the same
  // reference scales O and l).
  if (__any(mt > st.m_run + kRescaleThreshold / c)) {
    const float m_new = fmaxf(st.m_run, mt);
    if (m_new != st.m_run) {
      const float alpha = (st.m_run == -INFINITY) ? 0.f : fast_exp2((st.m_run - m_new) * c);
      st.l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) st.oacc[i][e] *= alpha;
      st.m_run = m_new;
    }
  }
  const float mc = (st.m_run == -INFINITY) ? 0.f : st.m_run * c;
  float ls = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = fast_exp2(__builtin_fmaf(sacc[kb][e], c, -mc));
      sacc[kb][e] = p;
      ls += p;
    }
  st.l_run += ls;
#pragma unroll
  for (int cs = 0; cs < 4; ++cs) {
    const bf16x8 pb = acc_to_operand(sacc[cs >> 1], cs & 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) st.oacc[db] = mfma32(col_operand(vs, L, db, cs), pb, st.oacc[db]);
  }
}

__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(const uint16_t *__restrict__ Q,
                                                               const uint16_t *__restrict__ K,
                                                               const uint16_t *__restrict__ V,
                                                               uint16_t *__restrict__ O, float *__restrict__ LSE,
                                                               int B, int T, int H, int KV, int W, float scale) {
  // Two separate LDS objects for the double buffer, so that the compiler can tell
  // the direct-to-LDS copy into one from the reads of the other and does not
  // wait for the copy before reading.
  __shared__ __attribute__((aligned(1024))) char buf0[kBufBytes];  // K | V
  __shared__ __attribute__((aligned(1024))) char buf1[kBufBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nqb = (T + kBlockM - 1) / kBlockM;
  const int BH = B * H;
  const int qblk = nqb - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int b = bh / H;
  const int h = bh % H;
  const int kvh = h / (H / KV);
  const int q0 = qblk * kBlockM;
  const int qw0 = q0 + 32 * wave;
  const int q_lane = qw0 + (lane & 31);
  const int hh = lane >> 5;
  const float c = scale * kLog2e;

  const long long q_stride = (long long)H * kD;
  const long long kv_stride = (long long)KV * kD;
  const uint16_t *Kb = K + (long long)b * T * kv_stride + (long long)kvh * kD;
  const uint16_t *Vb = V + (long long)b * T * kv_stride + (long long)kvh * kD;
  const TileLoader tl = make_tile_loader(kv_stride, tid);

  const int q_last_blk = min(q0 + kBlockM - 1, T - 1);
  const int k_lo = W < 0 ? 0 : max(0, q0 - W);
  const int t0 = k_lo / kTileN;
  const int t1 = q_last_blk / kTileN;

  tile_load_lds(buf0, Kb, tl, t0 * kTileN, T);
  tile_load_lds(buf0 + kTileBytes, Vb, tl, t0 * kTileN, T);

  // Q^T operand in registers: lane holds q row q_lane, d = 16 s + 8 hh + [0, 8).
  bf16x8 qreg[8];
  {
    const int qr = min(q_lane, T - 1);
    const uint16_t *qp = Q + ((long long)b * T + qr) * q_stride + (long long)h * kD + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 16 * s));
  }
  const TileLane L = make_tile_lane(lane);
  const int qw_last = min(qw0 + 31, T - 1);
  const bool wave_active = qw0 < T;

  FwdState st;
#pragma unroll
  for (int i = 0; i < 4; ++i) st.oacc[i] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  lds_loads_done_barrier();

  // One tile of work on `cur` while the next tile is copied into `nxt`.
  auto step = [&](const char *cur, char *nxt, int t) {
    if (t < t1) {
      tile_load_lds(nxt, Kb, tl, (t + 1) * kTileN, T);
      tile_load_lds(nxt + kTileBytes, Vb, tl, (t + 1) * kTileN, T);
    }
    const int k0 = t * kTileN;
    const bool skip = !wave_active || k0 > qw_last || (W >= 0 && qw0 - (k0 + kTileN - 1) > W);
    if (!skip) {
      const bool need_mask = !(k0 + kTileN - 1 <= qw0 && (W < 0 || qw_last - k0 <= W));
      if (need_mask)
        fwd_tile<true>(st, cur, cur + kTileBytes, L, qreg, k0, q_lane, W, c, hh);
      else
        fwd_tile<false>(st, cur, cur + kTileBytes, L, qreg, k0, q_lane, W, c, hh);
    }
    lds_loads_done_barrier();
  };
  for (int t = t0; t <= t1; t += 2) {
    step(buf0, buf1, t);
    if (t + 1 > t1) break;
    step(buf1, buf0, t + 1);
  }

  if (!wave_active) return;
  const float l_tot = st.l_run + shfl_xor(st.l_run, 32);
  const float inv_l = 1.f / l_tot;
  if (q_lane < T) {
    uint16_t *op = O + ((long long)b * T + q_lane) * q_stride + (long long)h * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * i + 4 * hh;
        u32x2 w;
        w[0] = pack_bf16x2(st.oacc[db][4 * i + 0] * inv_l, st.oacc[db][4 * i + 1] * inv_l);
        w[1] = pack_bf16x2(st.oacc[db][4 * i + 2] * inv_l, st.oacc[db][4 * i + 3] * inv_l);
        *(u32x2 *)(op + d) = w;
      }
    if (hh == 0) LSE[((long long)b * H + h) * T + q_lane] = st.m_run * scale + logf(l_tot);
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
