// Attention backward, bf16 in/out, fp32 accumulation, head_dim 128, gfx950 MFMA.
//
// The exact gradient of sum(O * dO) through the forward ("nanochat (Python)"
// catalog, AI / Model & kernels / Backward pass: autograd of the forward).  With
// P_ij = exp(scale q_i.k_j - LSE_i) on visible pairs and D_i = sum_d dO_i O_i:
//   dV_j = sum_i P_ij dO_i            dP_ij = dO_i . v_j
//   dS_ij = P_ij (dP_ij - D_i)        dQ_i = scale sum_j dS_ij k_j
//   dK_j = scale sum_i dS_ij q_i      (dK, dV summed over the G heads of a group)
// (D_i equals sum_j P_ij dP_ij, the softmax-Jacobian term, because O_i = sum_j P_ij v_j.)
//
// Three kernels, no atomics (deterministic):
//   1. bwd_delta: D_i per (b, h, i) into the workspace.
//   2. bwd_dkdv: one workgroup per (b, kv head, 128-key block), wave w owns keys
//      32w..32w+31 and keeps K, V for them in registers; it walks 64-row query
//      tiles (Q, dO, LSE, D staged in LDS, double-buffered) for every query head of
//      the group, computing S = Q K^T, dP = dO V^T (queries as MFMA rows, the
//      wave's keys as columns), then dV^T += dO^T P and dK^T += Q^T dS with
//      transposing LDS reads of dO and Q.
//   3. bwd_dq: one workgroup per (b, h, 128-row query block), like the forward:
//      S^T = K Q^T and dP^T = V dO^T with Q, dO in registers, dQ^T += K^T dS^T.
// Tiles with no visible pair are skipped; masks only on straddling tiles.
#include "attn_tiles.hpp"
#include "internal.hpp"

namespace ncattn {

namespace {

constexpr int kBlockM = 128;  // query rows per dq workgroup
constexpr int kBlockN = 128;  // keys per dkdv workgroup

// ---------------------------------------------------------------- D_i = dO . O
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t *__restrict__ O,
                                                        const uint16_t *__restrict__ dO, float *__restrict__ delta,
                                                        int B, int T, int H) {
  // 16 lanes per (token, head) row, 16 rows per block
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  const long long nrows = (long long)B * T * H;
  float s = 0.f;
  if (row < nrows) {
    const u32x4 a = *(const u32x4 *)(O + row * kD + part * 8);
    const u32x4 g = *(const u32x4 *)(dO + row * kD + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) s += lo_bf16(a[i]) * lo_bf16(g[i]) + hi_bf16(a[i]) * hi_bf16(g[i]);
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) s += shfl_xor(s, m);
  if (row < nrows && part == 0) {
    const long long tok = row / H;
    const int h = (int)(row % H);
    const int b = (int)(tok / T);
    const int t = (int)(tok % T);
    delta[((long long)b * H + h) * T + t] = s;
  }
}

// ---------------------------------------------------------------- dK, dV
constexpr int kQBuf = 2 * kTileBytes + 2 * kTileN * 4;  // Q tile, dO tile, lse2[64], delta[64]

// One 32-query block (rows 32 qb.. of the staged tile) against this wave's 32 keys.
__device__ __forceinline__ void dkdv_block(bool need_mask, f32x16 (&dkacc)[4], f32x16 (&dvacc)[4], const char *qs, const char *dos,
                                           const float *lse2, const float *dl, const TileLane &L,
                                           const bf16x8 (&kreg)[8], const bf16x8 (&vreg)[8], int qb, int qtile0,
                                           int key_lane, int T, int W, float c, int hh) {
  f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    sacc = mfma32(row_operand(qs, L, s, qb), kreg[s], sacc);
    dpacc = mfma32(row_operand(dos, L, s, qb), vreg[s], dpacc);
  }
  // rows of this lane's accumulator elements: 32 qb + 8 i + 4 hh + j
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r0 = 32 * qb + 8 * i + 4 * hh;
    const f32x4 l4 = *(const f32x4 *)(lse2 + r0);
    const f32x4 d4 = *(const f32x4 *)(dl + r0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * i + j;
      float p = fast_exp2(__builtin_fmaf(sacc[e], c, -l4[j]));
      if (need_mask) {
        const int qi = qtile0 + r0 + j;
        const bool vis = qi < T && key_lane <= qi && (W < 0 || qi - key_lane <= W);
        if (!vis) p = 0.f;
      }
      sacc[e] = p;
      dpacc[e] = p * (dpacc[e] - d4[j]);
    }
  }
  // dV^T += dO^T P and dK^T += Q^T dS, contraction over the 32 query rows.
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    const bf16x8 pb = acc_to_operand(sacc, c2);
    const bf16x8 dsb = acc_to_operand(dpacc, c2);
    const int cs = 2 * qb + c2;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      dvacc[db] = mfma32(col_operand(dos, L, db, cs), pb, dvacc[db]);
      dkacc[db] = mfma32(col_operand(qs, L, db, cs), dsb, dkacc[db]);
    }
  }
}

__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(const uint16_t *__restrict__ Q,
                                                          const uint16_t *__restrict__ K,
                                                          const uint16_t *__restrict__ V,
                                                          const uint16_t *__restrict__ dO,
                                                          const float *__restrict__ LSE,
                                                          const float *__restrict__ delta, uint16_t *__restrict__ dK,
                                                          uint16_t *__restrict__ dV, int B, int T, int H, int KV,
                                                          int W, float scale) {
  // Two separate LDS objects for the double buffer (Q | dO | lse2 | delta each),
  // so the compiler can tell the copy into one from the reads of the other.
  __shared__ __attribute__((aligned(1024))) char buf0[kQBuf];
  __shared__ __attribute__((aligned(1024))) char buf1[kQBuf];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hh = lane >> 5;
  const int G = H / KV;
  const int BKV = B * KV;
  // key blocks near the start of the sequence see the most queries: schedule them first
  const int kblk = (int)(blockIdx.x / BKV);
  const int bk = (int)(blockIdx.x % BKV);
  const int b = bk / KV;
  const int kvh = bk % KV;
  const int k0 = kblk * kBlockN;
  const int kw0 = k0 + 32 * wave;
  const int key_lane = kw0 + (lane & 31);  // the key column this lane holds
  const float c = scale * kLog2e;

  const long long q_stride = (long long)H * kD;
  const long long kv_stride = (long long)KV * kD;
  const TileLoader tl = make_tile_loader(q_stride, tid);

  // Query tiles that can see any key of the block, times the G heads of the group.
  const int k_last_blk = min(k0 + kBlockN - 1, T - 1);
  const int q_hi = W < 0 ? T - 1 : min(T - 1, k_last_blk + W);
  const int qt0 = k0 / kTileN;
  const int nq = q_hi / kTileN - qt0 + 1;
  const int n_iter = nq * G;

  auto stage = [&](int it, char *base) {
    const int qt = qt0 + it / G;
    const int h = kvh * G + it % G;
    const long long hoff = (long long)b * T * q_stride + (long long)h * kD;
    tile_load_lds(base, Q + hoff, tl, qt * kTileN, T);
    tile_load_lds(base + kTileBytes, dO + hoff, tl, qt * kTileN, T);
    if (tid < 128) {  // waves 0, 1: 64 lse rows and 64 delta rows, 4 bytes per lane
      const int qi = min(qt * kTileN + lane, T - 1);
      const float *src = (tid < 64 ? LSE : delta) + ((long long)b * H + h) * T + qi;
      typedef __attribute__((address_space(3))) void lds_void;
      typedef __attribute__((address_space(1))) const void glb_void;
      __builtin_amdgcn_global_load_lds((glb_void *)src, (lds_void *)(base + 2 * kTileBytes + (tid >> 6) * kTileN * 4),
                                       4, 0, 0);
    }
  };

  stage(0, buf0);

  bf16x8 kreg[8], vreg[8];
  {
    const int kr = min(key_lane, T - 1);
    const long long off = ((long long)b * T + kr) * kv_stride + (long long)kvh * kD + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(K + off + 16 * s));
      vreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(V + off + 16 * s));
    }
  }
  const TileLane L = make_tile_lane(lane);
  const int kw_last = min(kw0 + 31, T - 1);
  const bool wave_active = kw0 < T;

  f32x16 dkacc[4], dvacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dkacc[i] = f32x16{};
    dvacc[i] = f32x16{};
  }

  lds_loads_done_barrier();

  auto step = [&](char *cur, char *nxt, int it) {
    const char *qs = cur;
    const char *dos = cur + kTileBytes;
    float *lse2 = (float *)(cur + 2 * kTileBytes);
    const float *dl = lse2 + kTileN;
    if (it + 1 < n_iter) stage(it + 1, nxt);
    const int qtile0 = (qt0 + it / G) * kTileN;
    // the staged lse is natural-log; scale it to log2 units in place once per tile
    if (tid < kTileN) lse2[tid] *= kLog2e;
    __syncthreads();
    const bool skip = !wave_active || qtile0 + kTileN - 1 < kw0 || (W >= 0 && qtile0 - kw_last > W);
    if (!skip) {
#pragma unroll 1
      for (int qb = 0; qb < 2; ++qb) {
        const int qr0 = qtile0 + 32 * qb;
        if (qr0 + 31 < kw0 || (W >= 0 && qr0 - kw_last > W)) continue;
        const bool need_mask = !(qr0 >= kw_last && (W < 0 || qr0 + 31 - kw0 <= W) && qr0 + 31 < T);
        dkdv_block(need_mask, dkacc, dvacc, qs, dos, lse2, dl, L, kreg, vreg, qb, qtile0, key_lane, T, W, c, hh);
      }
    }
    lds_loads_done_barrier();
  };
  for (int it = 0; it < n_iter; it += 2) {
    step(buf0, buf1, it);
    if (it + 1 >= n_iter) break;
    step(buf1, buf0, it + 1);
  }

  if (!wave_active || key_lane >= T) return;
  const long long off = ((long long)b * T + key_lane) * kv_stride + (long long)kvh * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * hh;
      u32x2 wk, wv;
      wk[0] = pack_bf16x2(dkacc[db][4 * i + 0] * scale, dkacc[db][4 * i + 1] * scale);
      wk[1] = pack_bf16x2(dkacc[db][4 * i + 2] * scale, dkacc[db][4 * i + 3] * scale);
      wv[0] = pack_bf16x2(dvacc[db][4 * i + 0], dvacc[db][4 * i + 1]);
      wv[1] = pack_bf16x2(dvacc[db][4 * i + 2], dvacc[db][4 * i + 3]);
      *(u32x2 *)(dK + off + d) = wk;
      *(u32x2 *)(dV + off + d) = wv;
    }
}

// ---------------------------------------------------------------- dQ
struct DqState {
  f32x16 dqacc[4];
};

// One 64-key tile: S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
template <bool kMask>
__device__ __forceinline__ void dq_tile(DqState &st, const char *ks, const char *vs, const TileLane &L,
                                        const bf16x8 (&qreg)[8], const bf16x8 (&doreg)[8], int k0, int q_lane,
                                        int W, float c, float lse2, float del, int hh) {
  f32x16 sacc[2], dpacc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 a = f32x16{}, g = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      a = mfma32(row_operand(ks, L, s, kb), qreg[s], a);
      g = mfma32(row_operand(vs, L, s, kb), doreg[s], g);
    }
    sacc[kb] = a;
    dpacc[kb] = g;
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float p = fast_exp2(__builtin_fmaf(sacc[kb][e], c, -lse2));
      if constexpr (kMask) {
        const int key = k0 + 32 * kb + 8 * (e >> 2) + 4 * hh + (e & 3);
        const bool vis = key <= q_lane && (W < 0 || q_lane - key <= W);
        if (!vis) p = 0.f;
      }
      dpacc[kb][e] = p * (dpacc[kb][e] - del);
    }
#pragma unroll
  for (int cs = 0; cs < 4; ++cs) {
    const bf16x8 dsb = acc_to_operand(dpacc[cs >> 1], cs & 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) st.dqacc[db] = mfma32(col_operand(ks, L, db, cs), dsb, st.dqacc[db]);
  }
}

__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(const uint16_t *__restrict__ Q,
                                                        const uint16_t *__restrict__ K,
                                                        const uint16_t *__restrict__ V,
                                                        const uint16_t *__restrict__ dO,
                                                        const float *__restrict__ LSE,
                                                        const float *__restrict__ delta, uint16_t *__restrict__ dQ,
                                                        int B, int T, int H, int KV, int W, float scale) {
  __shared__ __attribute__((aligned(1024))) char buf0[2 * kTileBytes];  // K | V, double buffer
  __shared__ __attribute__((aligned(1024))) char buf1[2 * kTileBytes];
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

  const bool valid = q_lane < T;
  bf16x8 qreg[8], doreg[8];
  {
    const int qr = min(q_lane, T - 1);
    const long long off = ((long long)b * T + qr) * q_stride + (long long)h * kD + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(Q + off + 16 * s));
      doreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(dO + off + 16 * s));
    }
  }
  const long long ri = ((long long)b * H + h) * T + min(q_lane, T - 1);
  const float lse2 = valid ? LSE[ri] * kLog2e : INFINITY;  // rows past T get P = 0
  const float del = valid ? delta[ri] : 0.f;
  const TileLane L = make_tile_lane(lane);
  const int qw_last = min(qw0 + 31, T - 1);
  const bool wave_active = qw0 < T;

  DqState st;
#pragma unroll
  for (int i = 0; i < 4; ++i) st.dqacc[i] = f32x16{};

  lds_loads_done_barrier();

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
        dq_tile<true>(st, cur, cur + kTileBytes, L, qreg, doreg, k0, q_lane, W, c, lse2, del, hh);
      else
        dq_tile<false>(st, cur, cur + kTileBytes, L, qreg, doreg, k0, q_lane, W, c, lse2, del, hh);
    }
    lds_loads_done_barrier();
  };
  for (int t = t0; t <= t1; t += 2) {
    step(buf0, buf1, t);
    if (t + 1 > t1) break;
    step(buf1, buf0, t + 1);
  }

  if (!wave_active || !valid) return;
  uint16_t *dqp = dQ + ((long long)b * T + q_lane) * q_stride + (long long)h * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * hh;
      u32x2 w;
      w[0] = pack_bf16x2(st.dqacc[db][4 * i + 0] * scale, st.dqacc[db][4 * i + 1] * scale);
      w[1] = pack_bf16x2(st.dqacc[db][4 * i + 2] * scale, st.dqacc[db][4 * i + 3] * scale);
      *(u32x2 *)(dqp + d) = w;
    }
}

}  // namespace

hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                           const void *dout, void *dq, void *dk, void *dv, float *delta, const AttnShape &sh,
                           int stages, hipStream_t s) {
  const long long rows = (long long)sh.B * sh.T * sh.H;
  const long long dblocks = (rows + 15) / 16;
  const long long nkb = (sh.T + kBlockN - 1) / kBlockN;
  const long long nqb = (sh.T + kBlockM - 1) / kBlockM;
  const long long kvblocks = nkb * sh.B * sh.KV;
  const long long qblocks = nqb * sh.B * sh.H;
  if (dblocks > 0x7fffffffLL || kvblocks > 0x7fffffffLL || qblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (stages & kBwdDelta)
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)dblocks), dim3(256), 0, s, (const uint16_t *)o,
                     (const uint16_t *)dout, delta, sh.B, sh.T, sh.H);
  if (stages & kBwdDkDv)
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)kvblocks), dim3(256), 0, s, (const uint16_t *)q,
                     (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dout, lse, delta, (uint16_t *)dk,
                     (uint16_t *)dv, sh.B, sh.T, sh.H, sh.KV, sh.window, sh.scale);
  if (stages & kBwdDq)
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)qblocks), dim3(256), 0, s, (const uint16_t *)q,
                     (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dout, lse, delta, (uint16_t *)dq,
                     sh.B, sh.T, sh.H, sh.KV, sh.window, sh.scale);
  return hipGetLastError();
}

}  // namespace ncattn
