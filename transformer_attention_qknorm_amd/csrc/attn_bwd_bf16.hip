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
// Stores -D_i (the initial value of the dP - D accumulators of the dK/dV stage)
// and LSE_i * log2(e), the exponent offset of P in base 2.
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t *__restrict__ O,
                                                        const uint16_t *__restrict__ dO,
                                                        const float *__restrict__ LSE, float *__restrict__ ndelta,
                                                        float *__restrict__ lse2, int B, int T, int H) {
  // 8 lanes per (token, head) row, 32 bytes of O and of dO each; a wave covers 8
  // rows per pass and issues the loads of two passes before reducing.
  const long long nrows = (long long)B * T * H;
  const int part = threadIdx.x & 7;
  const long long row_base = ((long long)blockIdx.x * 256 + (threadIdx.x & ~7)) / 8 * 2;  // 64 rows per block
  float s[2];
  u32x4 a[2][2], g[2][2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const long long row = row_base + p;
    const long long r = row < nrows ? row : nrows - 1;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      a[p][c] = *(const u32x4 *)(O + r * kD + part * 16 + 8 * c);
      g[p][c] = *(const u32x4 *)(dO + r * kD + part * 16 + 8 * c);
    }
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc += lo_bf16(a[p][c][i]) * lo_bf16(g[p][c][i]) + hi_bf16(a[p][c][i]) * hi_bf16(g[p][c][i]);
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) acc += shfl_xor(acc, m);
    s[p] = acc;
  }
  if (part < 2) {
    const long long row = row_base + part;
    if (row < nrows) {
      const long long tok = row / H;
      const int h = (int)(row % H);
      const int b = (int)(tok / T);
      const int t = (int)(tok % T);
      const long long ri = ((long long)b * H + h) * T + t;
      ndelta[ri] = -(part == 0 ? s[0] : s[1]);
      lse2[ri] = LSE[ri] * kLog2e;
    }
  }
}

// ---------------------------------------------------------------- dK, dV
constexpr int kQBuf = 2 * kTileBytes + 2 * kTileN * 4;  // Q tile, dO tile, lse2[64], delta[64]

// S = Q K^T and dP - D = dO V^T - D for one 32-query block (rows 32 qb.. of the
// staged tile) against this wave's 32 keys (queries as rows, the wave's keys as
// columns).  The dP accumulator starts at -D of its query rows (staged next to
// the tile), so it ends holding dP - D.
__device__ __forceinline__ void dkdv_sdp(f32x16 &sacc, f32x16 &dpacc, const char *qs, const char *dos,
                                         const float *ndl, const TileLane &L, const bf16x8 (&kreg)[8],
                                         const bf16x8 (&vreg)[8], int qb, int hh) {
  bf16x8 qa[8], da[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qa[s] = row_operand(qs, L, s, qb);
    da[s] = row_operand(dos, L, s, qb);
  }
  sacc = f32x16{};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 d4 = *(const f32x4 *)(ndl + 32 * qb + 8 * i + 4 * hh);
#pragma unroll
    for (int j = 0; j < 4; ++j) dpacc[4 * i + j] = d4[j];
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    sacc = mfma32(qa[s], kreg[s], sacc);
    dpacc = mfma32(da[s], vreg[s], dpacc);
  }
}

// P = exp2(S c - LSE log2 e) and dS = P (dP - D) as bf16 MFMA operands (pk, dk:
// element pairs of accumulator rows 8 i + 4 hh + j, the layout acc_to_operand
// gives), and dS rearranged for the workspace: `out` holds this lane's 16
// consecutive queries of its key's [key][query] tile row, starting at query
// 32 qb + 16 hh (see ds_store).
__device__ __forceinline__ void dkdv_p_ds(const f32x16 &sacc, const f32x16 &dmd, const float *lse2, bool need_mask,
                                          int qb, int qtile0, int key_lane, int T, int W, float c, int hh,
                                          uint32_t (&pk)[8], uint32_t (&dk)[8], u32x4 (&out)[2]) {
  // rows of this lane's accumulator elements: 32 qb + 8 i + 4 hh + j
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r0 = 32 * qb + 8 * i + 4 * hh;
    const f32x4 l4 = *(const f32x4 *)(lse2 + r0);
    float p[4], ds[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * i + j;
      p[j] = fast_exp2(__builtin_fmaf(sacc[e], c, -l4[j]));
      if (need_mask) {
        const int qi = qtile0 + r0 + j;
        const bool vis = qi < T && key_lane <= qi && (W < 0 || qi - key_lane <= W);
        if (!vis) p[j] = 0.f;
      }
      ds[j] = p[j] * dmd[e];
    }
    pk[2 * i] = pack_bf16x2(p[0], p[1]);
    pk[2 * i + 1] = pack_bf16x2(p[2], p[3]);
    dk[2 * i] = pack_bf16x2(ds[0], ds[1]);
    dk[2 * i + 1] = pack_bf16x2(ds[2], ds[3]);
  }
  // The two half-waves hold interleaved groups of 4 queries of the same key
  // (h = 0: 0-3, 8-11, 16-19, 24-27; h = 1: 4-7, ...).  v_permlane32_swap of
  // (dk[k], dk[4 + k]) hands lane l < 32 its partner's dk[k] in the second value
  // and lane l >= 32 its partner's dk[4 + k] in the first, so that every lane then
  // owns 16 consecutive queries (32 B).
  uint32_t x[4], y[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto r = __builtin_amdgcn_permlane32_swap(dk[k], dk[4 + k], false, false);
    x[k] = r[0];
    y[k] = r[1];
  }
  out[0] = u32x4{x[0], x[1], y[0], y[1]};
  out[1] = u32x4{x[2], x[3], y[2], y[3]};
}

// Writes a lane's 32 dS bytes (from dkdv_p_ds) into its workspace tile row.
__device__ __forceinline__ void ds_store(uint16_t *ds_row, const u32x4 (&out)[2], int qb, int hh) {
  u32x4 *dst = (u32x4 *)(ds_row + 32 * qb + 16 * hh);
  dst[0] = out[0];
  dst[1] = out[1];
}

// dV^T += dO^T P and dK^T += Q^T dS, contraction over the 32 query rows of block qb.
__device__ __forceinline__ void dkdv_acc(f32x16 (&dkacc)[4], f32x16 (&dvacc)[4], const uint32_t (&pk)[8],
                                         const uint32_t (&dk)[8], const char *qs, const char *dos, const TileLane &L,
                                         int qb) {
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    const int cs = 2 * qb + c2;
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[4 * c2], pk[4 * c2 + 1], pk[4 * c2 + 2], pk[4 * c2 + 3]});
    const bf16x8 dsb = __builtin_bit_cast(bf16x8, u32x4{dk[4 * c2], dk[4 * c2 + 1], dk[4 * c2 + 2], dk[4 * c2 + 3]});
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      dvacc[db] = mfma32(col_operand(dos, L, db, cs), pb, dvacc[db]);
      dkacc[db] = mfma32(col_operand(qs, L, db, cs), dsb, dkacc[db]);
    }
  }
}

// Interleave the next n MFMAs of the scheduling region with the vector ALU work
// (k VALU instructions after each), so the matrix cores and the VALU run together.
template <int N, int K>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, K, 0);  // VALU
  }
}

__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(const uint16_t *__restrict__ Q,
                                                          const uint16_t *__restrict__ K,
                                                          const uint16_t *__restrict__ V,
                                                          const uint16_t *__restrict__ dO,
                                                          const float *__restrict__ lse2g,
                                                          const float *__restrict__ delta, uint16_t *__restrict__ dK,
                                                          uint16_t *__restrict__ dV, uint16_t *__restrict__ dsband,
                                                          int B, int T, int H, int KV, int W, float scale, int nqt,
                                                          int nbw) {
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
  const int kt = kw0 / kTileN;              // key tile of this wave's keys, and their first row in it
  const int kofs = kw0 % kTileN;
  const float c = scale * kLog2e;

  const long long q_stride = (long long)H * kD;
  const long long kv_stride = (long long)KV * kD;
  const int voff = tile_lane_voff((int)(q_stride * 2), tid);

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
    tile_load_lds(base, make_tile_src(Q + hoff, q_stride, T), voff, qt * kTileN);
    tile_load_lds(base + kTileBytes, make_tile_src(dO + hoff, q_stride, T), voff, qt * kTileN);
    if (wave < 2) {  // waves 0, 1: 64 lse rows and 64 delta rows, 4 bytes per lane (zeros past T)
      const float *row = (wave == 0 ? lse2g : delta) + ((long long)b * H + h) * T;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)row, (short)0, T * 4, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(base + 2 * kTileBytes + wave * kTileN * 4), 4,
                                               lane * 4, qt * kTileN * 4, 0, 0);
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
    const float *lse2 = (const float *)(cur + 2 * kTileBytes);
    const float *ndl = lse2 + kTileN;
    if (it + 1 < n_iter) stage(it + 1, nxt);
    const int qtile0 = (qt0 + it / G) * kTileN;
    const bool skip = !wave_active || qtile0 + kTileN - 1 < kw0 || (W >= 0 && qtile0 - kw_last > W);
    if (!skip) {
      const int qt = qtile0 / kTileN;
      const int h = kvh * G + it % G;
      const long long tile = (((long long)b * H + h) * nqt + qt) * nbw + (kt - ds_kt_lo(qt, W));
      uint16_t *ds_row = dsband + tile * (kTileN * kTileN) + (kofs + (lane & 31)) * kTileN;
      bool act[2], msk[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qr0 = qtile0 + 32 * qb;
        act[qb] = !(qr0 + 31 < kw0 || (W >= 0 && qr0 - kw_last > W));
        msk[qb] = !(qr0 >= kw_last && (W < 0 || qr0 + 31 - kw0 <= W) && qr0 + 31 < T);
      }
      if (act[0] && act[1] && !msk[0] && !msk[1]) {
        // steady state, one straight-line block: the S/dP MFMAs of query block 1
        // run under the P/dS arithmetic of block 0, and the dV/dK MFMAs of block
        // 0 under that of block 1
        f32x16 s0, p0, s1, p1;
        uint32_t pk0[8], dk0[8], pk1[8], dk1[8];
        u32x4 out0[2], out1[2];
        dkdv_sdp(s0, p0, qs, dos, ndl, L, kreg, vreg, 0, hh);
        __builtin_amdgcn_sched_barrier(0);
        dkdv_sdp(s1, p1, qs, dos, ndl, L, kreg, vreg, 1, hh);
        dkdv_p_ds(s0, p0, lse2, false, 0, qtile0, key_lane, T, W, c, hh, pk0, dk0, out0);
        ds_store(ds_row, out0, 0, hh);
        interleave_mfma_valu<16, 5>();
        __builtin_amdgcn_sched_barrier(0);
        dkdv_acc(dkacc, dvacc, pk0, dk0, qs, dos, L, 0);
        dkdv_p_ds(s1, p1, lse2, false, 1, qtile0, key_lane, T, W, c, hh, pk1, dk1, out1);
        ds_store(ds_row, out1, 1, hh);
        interleave_mfma_valu<16, 5>();
        __builtin_amdgcn_sched_barrier(0);
        dkdv_acc(dkacc, dvacc, pk1, dk1, qs, dos, L, 1);
      } else {
#pragma unroll 1
        for (int qb = 0; qb < 2; ++qb) {
          if (!act[qb]) continue;
          f32x16 s0, p0;
          uint32_t pk0[8], dk0[8];
          dkdv_sdp(s0, p0, qs, dos, ndl, L, kreg, vreg, qb, hh);
          u32x4 out[2];
          dkdv_p_ds(s0, p0, lse2, msk[qb], qb, qtile0, key_lane, T, W, c, hh, pk0, dk0, out);
          ds_store(ds_row, out, qb, hh);
          dkdv_acc(dkacc, dvacc, pk0, dk0, qs, dos, L, qb);
        }
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
// dQ = scale dS K from the dS tiles the dK/dV stage stored: one GEMM per tile.
// A dS^T tile ([key][query], 64 x 64 bf16, 128-byte rows) is staged with its
// 16-byte chunks permuted per row, chunk' = chunk ^ (4 ((row >> 1) & 1)), which
// keeps the transposing reads below free of bank conflicts.
__device__ __forceinline__ int ds_swz(int row, int chunk) { return row * 128 + ((chunk ^ (((row >> 1) & 1) << 2)) << 4); }

// Direct global -> LDS copy of one dS^T tile (8 KB) by the 4 waves: wave w,
// instruction i fills rows 16 w + 8 i + [0, 8), lane l row + l/8, position l%8.
__device__ __forceinline__ void ds_tile_load(char *lds_tile, const uint16_t *src_tile, int tid) {
  const int lane = tid & 63, w = tid >> 6;
  typedef __attribute__((address_space(3))) void lds_void;
  typedef __attribute__((address_space(1))) const void glb_void;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * w + 8 * i + (lane >> 3);
    const int chunk = (lane & 7) ^ (((row >> 1) & 1) << 2);
    const char *src = (const char *)src_tile + row * 128 + chunk * 16;
    __builtin_amdgcn_global_load_lds((glb_void *)src, (lds_void *)(lds_tile + (16 * w + 8 * i) * 128), 16, 0, 0);
  }
}

__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(const uint16_t *__restrict__ K,
                                                        const uint16_t *__restrict__ dsband,
                                                        uint16_t *__restrict__ dQ, int B, int T, int H, int KV,
                                                        int W, float scale, int nqt, int nbw) {
  // double buffer: [K tile | dS^T tile of query tile 2 qblk | of query tile 2 qblk + 1]
  __shared__ __attribute__((aligned(1024))) char buf0[kTileBytes + 2 * 8192];
  __shared__ __attribute__((aligned(1024))) char buf1[kTileBytes + 2 * 8192];
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

  const long long kv_stride = (long long)KV * kD;
  const uint16_t *Kb = K + (long long)b * T * kv_stride + (long long)kvh * kD;
  const TileSrc ksrc = make_tile_src(Kb, kv_stride, T);
  const int voff = tile_lane_voff(ksrc.stride, tid);
  const uint16_t *dsh = dsband + (long long)bh * nqt * nbw * (kTileN * kTileN);

  const int q_last_blk = min(q0 + kBlockM - 1, T - 1);
  const int t0 = (W < 0 ? 0 : max(0, q0 - W)) / kTileN;
  const int t1 = q_last_blk / kTileN;
  const int qw_last = min(qw0 + 31, T - 1);
  const bool wave_active = qw0 < T;
  const int tw0 = max(t0, (W < 0 ? 0 : max(0, qw0 - W)) / kTileN);
  const int tw1 = wave_active ? qw_last / kTileN : t0 - 1;

  // copies for key tile t: K, and the dS^T tiles of the block's two query tiles
  // that see tile t
  auto load = [&](char *buf, int t) {
    tile_load_lds(buf, ksrc, voff, t * kTileN);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int qt = 2 * qblk + sub;
      const int j = t - ds_kt_lo(qt, W);
      if (qt < nqt && j >= 0 && t <= qt)
        ds_tile_load(buf + kTileBytes + sub * 8192, dsh + ((long long)qt * nbw + j) * (kTileN * kTileN), tid);
    }
  };

  const TileLane L = make_tile_lane(lane);
  // per-lane offsets of the dS^T operand (query column 32 (wave & 1) + l%32, keys
  // {16 c + x + k, 16 c + x + 8 + k}, x = 4 (l/32) + ((l%16) >> 2)); + 2048 B per c
  int soff[2];
  {
    const int g = lane >> 4, r = lane & 15;
    const int x = 4 * (g >> 1) + (r >> 2);
    const int qc = 32 * (wave & 1) + ((g & 1) << 4) + 4 * (r & 3);
#pragma unroll
    for (int half = 0; half < 2; ++half) soff[half] = ds_swz(x + 8 * half, qc >> 3) + (qc & 7) * 2;
  }
  const int ssub = (wave >> 1) * 8192;

  f32x16 dqacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dqacc[i] = f32x16{};

  load(buf0, t0);
  lds_loads_done_barrier();

  auto step = [&](const char *cur, char *nxt, int t) {
    if (t < t1) load(nxt, t + 1);
    if (t >= tw0 && t <= tw1) {
      const int k0 = t * kTileN;
      const bool need_mask = !(k0 + kTileN - 1 <= qw0 && (W < 0 || qw_last - k0 <= W));
      const char *st = cur + kTileBytes + ssub;
      // every operand of the tile is read from LDS before the first MFMA
      u32x4 dsw[4];
      bf16x8 kop[4][4];
#pragma unroll
      for (int cs = 0; cs < 4; ++cs) {
        const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(st + soff[0] + cs * 16 * 128));
        const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(st + soff[1] + cs * 16 * 128));
        dsw[cs] = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int db = 0; db < 4; ++db) kop[cs][db] = col_operand(cur, L, db, cs);
      }
      if (need_mask) {
        // operand element e holds key k0 + 16 cs + 4 hh + (e & 3) + 8 (e >> 2)
#pragma unroll
        for (int cs = 0; cs < 4; ++cs)
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            uint32_t keep = 0u;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int e = 2 * e2 + half;
              const int key = k0 + 16 * cs + 4 * hh + (e & 3) + 8 * (e >> 2);
              const bool vis = key <= q_lane && (W < 0 || q_lane - key <= W);
              keep |= vis ? (0xffffu << (16 * half)) : 0u;
            }
            dsw[cs][e2] &= keep;
          }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cs = 0; cs < 4; ++cs) {
        const bf16x8 dsb = __builtin_bit_cast(bf16x8, dsw[cs]);
#pragma unroll
        for (int db = 0; db < 4; ++db) dqacc[db] = mfma32(kop[cs][db], dsb, dqacc[db]);
      }
    }
    lds_loads_done_barrier();
  };
  for (int t = t0; t <= t1; t += 2) {
    step(buf0, buf1, t);
    if (t + 1 > t1) break;
    step(buf1, buf0, t + 1);
  }

  if (!wave_active || q_lane >= T) return;
  uint16_t *dqp = dQ + ((long long)b * T + q_lane) * ((long long)H * kD) + (long long)h * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * hh;
      u32x2 w;
      w[0] = pack_bf16x2(dqacc[db][4 * i + 0] * scale, dqacc[db][4 * i + 1] * scale);
      w[1] = pack_bf16x2(dqacc[db][4 * i + 2] * scale, dqacc[db][4 * i + 3] * scale);
      *(u32x2 *)(dqp + d) = w;
    }
}

}  // namespace

size_t bwd_workspace_bytes(int B, int T, int H, int W, bool bf16) {
  const size_t rows = ((size_t)B * H * T * sizeof(float) + 255) & ~(size_t)255;
  if (!bf16) return rows;
  const DsBand band = ds_band(T, W);
  return 2 * rows + (size_t)B * H * band.nqt * band.nbw * (kTileN * kTileN) * 2;
}

hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                           const void *dout, void *dq, void *dk, void *dv, void *workspace, const AttnShape &sh,
                           int stages, hipStream_t s) {
  const size_t row_bytes = ((size_t)sh.B * sh.H * sh.T * sizeof(float) + 255) & ~(size_t)255;
  float *delta = (float *)workspace;
  float *lse2 = (float *)((char *)workspace + row_bytes);
  uint16_t *dsband = (uint16_t *)((char *)workspace + 2 * row_bytes);
  const DsBand band = ds_band(sh.T, sh.window);
  const long long rows = (long long)sh.B * sh.T * sh.H;
  const long long dblocks = (rows + 63) / 64;
  const long long nkb = (sh.T + kBlockN - 1) / kBlockN;
  const long long nqb = (sh.T + kBlockM - 1) / kBlockM;
  const long long kvblocks = nkb * sh.B * sh.KV;
  const long long qblocks = nqb * sh.B * sh.H;
  if (dblocks > 0x7fffffffLL || kvblocks > 0x7fffffffLL || qblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (stages & kBwdDelta)
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)dblocks), dim3(256), 0, s, (const uint16_t *)o,
                       (const uint16_t *)dout, lse, delta, lse2, sh.B, sh.T, sh.H);
  if (stages & kBwdDkDv)
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)kvblocks), dim3(256), 0, s, (const uint16_t *)q,
                       (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dout, lse2, delta, (uint16_t *)dk,
                       (uint16_t *)dv, dsband, sh.B, sh.T, sh.H, sh.KV, sh.window, sh.scale, band.nqt, band.nbw);
  if (stages & kBwdDq)
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)qblocks), dim3(256), 0, s, (const uint16_t *)k, dsband,
                       (uint16_t *)dq, sh.B, sh.T, sh.H, sh.KV, sh.window, sh.scale, band.nqt, band.nbw);
  return hipGetLastError();
}

}  // namespace ncattn
