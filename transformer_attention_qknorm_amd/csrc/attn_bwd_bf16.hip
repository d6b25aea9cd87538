// Attention backward, bf16 in/out, fp32 accumulation, head_dim 64 or 128, gfx950 MFMA.
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
//      32w..32w+31 and keeps K for them in registers, V of the block staged once
//      in LDS; it walks 32-row query tiles (Q, dO, LSE, D staged in LDS,
//      double-buffered) for every query head of the group, computing S = Q K^T,
//      dP = dO V^T (queries as MFMA rows, the wave's keys as columns), then
//      dV^T += dO^T P and dK^T += Q^T dS with transposing LDS reads of dO and Q.
//      Sized for two workgroups per CU (at most 256 registers per wave, 67 KB of
//      LDS at head_dim 128), so each SIMD runs waves of two workgroups that are
//      not tied by a barrier: one's P/dS arithmetic runs beside the other's
//      MFMAs.
//   3. bwd_dq: one workgroup per (b, h, 128-row query block), like the forward:
//      S^T = K Q^T and dP^T = V dO^T with Q, dO in registers, dQ^T += K^T dS^T.
// Both contraction stages recompute S and dP; P and dS enter the dV, dK and dQ
// products as bf16 hi + lo (fp32 precision, see split_bf16x2).  Tiles with no
// visible pair are skipped; masks only on straddling tiles.
#include "attn_tiles.hpp"
#include "internal.hpp"

namespace ncattn {

namespace {

constexpr int kBlockN = 128;  // keys per dkdv workgroup
constexpr int kDqRows = 128;  // query rows per dq workgroup

// ---------------------------------------------------------------- D_i = dO . O
// Stores -D_i (the initial value of the dP - D accumulators of the dK/dV stage)
// and LSE_i * log2(e), the exponent offset of P in base 2.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t *__restrict__ O,
                                                        const uint16_t *__restrict__ dO,
                                                        const float *__restrict__ LSE, float *__restrict__ ndelta,
                                                        float *__restrict__ lse2, int B, int T, int H) {
  // 8 lanes per (token, head) row, D / 4 bytes of O and of dO each; a wave covers
  // 8 rows per pass and issues the loads of two passes before reducing.
  constexpr int kC = D / 64;  // 16-byte loads per lane and row
  const long long nrows = (long long)B * T * H;
  const int part = threadIdx.x & 7;
  const long long row_base = ((long long)blockIdx.x * 256 + (threadIdx.x & ~7)) / 8 * 2;  // 64 rows per block
  float s[2];
  u32x4 a[2][kC], g[2][kC];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const long long row = row_base + p;
    const long long r = row < nrows ? row : nrows - 1;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      a[p][c] = *(const u32x4 *)(O + r * D + part * (D / 8) + 8 * c);
      g[p][c] = *(const u32x4 *)(dO + r * D + part * (D / 8) + 8 * c);
    }
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < kC; ++c)
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
// The bf16 value nearest x, and the bf16 value nearest the remainder: x is
// carried into the dV and dK products as hi + lo, so those products see P and dS
// to about 16 significant bits rather than bf16's 8 (only the final rounding of
// dK and dV to bf16 remains).  Packs the pair (x0, x1) into (hi, lo) dwords.
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(x0, x1);
  lo = pack_bf16x2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u));
}

// -inf on the scores of a straddling tile that are not visible (a query row past
// T, a key after the query, or one further back than the window): element e of
// the lane holds query row qtile0 + 32 qb + 8 (e / 4) + 4 hh + e % 4 against key
// key_lane.  Applied before the exponentials, so their block stays free of
// branches.
__device__ __forceinline__ void dkdv_mask(f32x16 &sacc, int qb, int qtile0, int key_lane, int T, int W, int hh) {
  const int r0 = qtile0 + 32 * qb + 4 * hh;  // query row of element 0
  const int d0 = r0 - key_lane;
  const int rlim = T - r0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int off = 8 * (e >> 2) + (e & 3);
    const bool vis = (off < rlim) & (d0 + off >= 0) & ((W < 0) | (d0 + off <= W));
    sacc[e] = vis ? sacc[e] : -INFINITY;
  }
}

// P = exp2(S c - LSE log2 e) and dS = P (dP - D) of one element pair (row i of
// 8, pair jp of 2: accumulator elements 4 i + 2 jp, + 1) as bf16 MFMA operands,
// each as a hi + lo pair (pk/pl, dk/dl[2 i + jp]: the layout acc_to_operand
// gives).  Scores masked to -inf give P = 0 (c > 0).
__device__ __forceinline__ void dkdv_p_ds_pair(const f32x16 &sacc, const f32x16 &dmd, const f32x4 (&l4)[4],
                                               float c, int i, int jp, uint32_t (&pk)[8], uint32_t (&pl)[8],
                                               uint32_t (&dk)[8], uint32_t (&dl)[8]) {
  const int e = 4 * i + 2 * jp;
  const float p0 = fast_exp2(__builtin_fmaf(sacc[e], c, -l4[i][2 * jp]));
  const float p1 = fast_exp2(__builtin_fmaf(sacc[e + 1], c, -l4[i][2 * jp + 1]));
  split_bf16x2(p0, p1, pk[2 * i + jp], pl[2 * i + jp]);
  split_bf16x2(p0 * dmd[e], p1 * dmd[e + 1], dk[2 * i + jp], dl[2 * i + jp]);
}

// From S and dP - D of the 32 query rows of the staged tile (rows 8 i + 4 hh + j
// of the lane's accumulators, i < 4): P and dS, then dV^T += dO^T (P_hi + P_lo)
// and dK^T += Q^T (dS_hi + dS_lo), contraction over those rows in two halves of
// 16.  The second half's exponentials and splits are placed among the first
// half's MFMAs (each group fenced), so that one wave's arithmetic runs while its
// own MFMAs execute.
template <int D>
__device__ __forceinline__ void dkdv_p_ds_acc(f32x16 (&dkacc)[Geom<D>::kDBlocks], f32x16 (&dvacc)[Geom<D>::kDBlocks],
                                              const f32x16 &sacc, const f32x16 &dmd, const float *lse2, float c,
                                              int hh, const char *qs, const char *dos, const TileLane<D> &L) {
  constexpr int NB = Geom<D>::kDBlocks;
  constexpr int kPer = 4 / NB;  // element pairs of the second half per block of the first
  f32x4 l4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) l4[i] = *(const f32x4 *)(lse2 + 8 * i + 4 * hh);
  uint32_t pk[8], pl[8], dk[8], dl[8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) dkdv_p_ds_pair(sacc, dmd, l4, c, i, jp, pk, pl, dk, dl);
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) {
    const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[4 * c2], pk[4 * c2 + 1], pk[4 * c2 + 2], pk[4 * c2 + 3]});
    const bf16x8 pbl = __builtin_bit_cast(bf16x8, u32x4{pl[4 * c2], pl[4 * c2 + 1], pl[4 * c2 + 2], pl[4 * c2 + 3]});
    const bf16x8 dsb = __builtin_bit_cast(bf16x8, u32x4{dk[4 * c2], dk[4 * c2 + 1], dk[4 * c2 + 2], dk[4 * c2 + 3]});
    const bf16x8 dsl = __builtin_bit_cast(bf16x8, u32x4{dl[4 * c2], dl[4 * c2 + 1], dl[4 * c2 + 2], dl[4 * c2 + 3]});
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      const bf16x8 a = col_operand(dos, L, db, c2);
      const bf16x8 qa = col_operand(qs, L, db, c2);
      if (c2 == 0) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          const int q = db * kPer + k;
          dkdv_p_ds_pair(sacc, dmd, l4, c, 2 + q / 2, q % 2, pk, pl, dk, dl);
        }
      }
      dvacc[db] = mfma32(a, pb, dvacc[db]);
      dkacc[db] = mfma32(qa, dsb, dkacc[db]);
      dvacc[db] = mfma32(a, pbl, dvacc[db]);
      dkacc[db] = mfma32(qa, dsl, dkacc[db]);
      if (c2 == 0) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ---------------------------------------------------------------- QK-norm + RoPE backward epilogue
// For the fused backward (ncattn_bwd_qknorm_rope): the gradient dy that dK / dQ
// hold for a post-norm row y = R(g x / r) is carried back to the raw row x
// ("nanochat Admin & Developer Guide", section 3: weightless RMSNorm of q and k,
// then rotary embedding; "nanochat (Python)" catalog, Backward pass: the chain
// rule through that forward).  With n = R^T y = g x / r the gradient
//   dx = (g / r) (R^T dy - (x / r) ((R^T dy) . (x / r)) / D)
// becomes, since the rotation keeps dot products,
//   dx = (g / r) R^T (dy - y (dy . y) / (g^2 D)):
// it needs the post-norm row y (the attention's own input) and 1/r, which the
// forward stored, not the raw row.  Each pair (j, j + D/2) is rotated by -theta_j.
// The row is held by the lane pair (l, l ^ 32) in accumulator layout: element
// 4 i + j of block db is d = 32 db + 8 i + 4 hh + j, so the pair partner d + D/2
// is block db + D/64 of the same lane, and the row sum needs one exchange.
struct NormRopeBwd {
  const float *rstd;          // 1/r per row: [B][T][rstd_stride], q rows at head h, k rows at rstd_k_off + kv head
  long long rstd_stride;
  int rstd_k_off;
  const int32_t *pos_offset;  // device [B] or NULL
  double turns[64];           // base^(-2j/D) / 2 pi for j < D/2: turns per position
  float gain;
};

// The norm's arguments as a fused kernel keeps them: copied into LDS at its
// start and read back by its epilogue, so that none of them occupies registers
// through the main loop (the loop needs all of them).
template <int D>
struct NormRopeLds {
  double turns[D / 2];
  const float *rstd;
  const int32_t *pos_offset;
  long long rstd_stride;
  int rstd_k_off;
  float gain;
};

template <int D>
__device__ __forceinline__ void stage_norm_rope(NormRopeLds<D> &s, const NormRopeBwd &nb, int tid) {
  if (tid < D / 2) s.turns[tid] = nb.turns[tid];
  if (tid == 0) {
    s.rstd = nb.rstd;
    s.pos_offset = nb.pos_offset;
    s.rstd_stride = nb.rstd_stride;
    s.rstd_k_off = nb.rstd_k_off;
    s.gain = nb.gain;
  }
}

template <int D>
__device__ __forceinline__ void norm_rope_bwd_row(f32x16 (&g)[Geom<D>::kDBlocks], const uint16_t *yrow, float rs,
                                                  double pos, const NormRopeLds<D> &nb, int hh) {
  constexpr int NB = Geom<D>::kDBlocks, HB = NB / 2;
  float y[NB][16];
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x2 w = *(const u32x2 *)(yrow + 32 * db + 8 * i + 4 * hh);
      y[db][4 * i + 0] = lo_bf16(w[0]);
      y[db][4 * i + 1] = hi_bf16(w[0]);
      y[db][4 * i + 2] = lo_bf16(w[1]);
      y[db][4 * i + 3] = hi_bf16(w[1]);
    }
  float dot = 0.f;
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dot += g[db][e] * y[db][e];
  dot += shfl_xor(dot, 32);
  const float coef = nb.gain == 0.f ? 0.f : dot / (nb.gain * nb.gain * (float)D);
  const float g_r = nb.gain * rs;
#pragma unroll
  for (int db = 0; db < HB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      // pair index 32 db + 8 (e >> 2) + 4 hh + (e & 3)
      double turns = pos * nb.turns[32 * db + 8 * (e >> 2) + 4 * hh + (e & 3)];
      turns -= rint(turns);
      const float tf = (float)turns;
      const float sn = __builtin_amdgcn_sinf(tf), cs = __builtin_amdgcn_cosf(tf);
      const float ua = g[db][e] - y[db][e] * coef, ub = g[db + HB][e] - y[db + HB][e] * coef;
      g[db][e] = g_r * (ua * cs + ub * sn);  // rotation by -theta
      g[db + HB][e] = g_r * (ub * cs - ua * sn);
    }
}

// S = Q K^T and dP - D = dO V^T - D for the 32 query rows of block qb of the
// staged tile against the wave's 32 keys (queries as rows, the wave's keys as
// columns), with V^T read from the workgroup's V tile in LDS (key block kw).
// The dP accumulator starts at -D of its query rows (staged next to the tile),
// so it ends holding dP - D.  Operands are read two MFMA pairs ahead.
template <int D>
__device__ __forceinline__ void dkdv_sdp(f32x16 &sacc, f32x16 &dpacc, const char *qs, const char *dos,
                                          const char *vs, const float *ndl, const TileLane<D> &L,
                                          const bf16x8 (&kreg)[Geom<D>::kSteps], int qb, int kw, int hh) {
  constexpr int kSteps = Geom<D>::kSteps;
  constexpr int kAhead = 2;
  bf16x8 qa[kSteps], da[kSteps], va[kSteps];
#pragma unroll
  for (int s = 0; s < kAhead; ++s) {
    qa[s] = row_operand(qs, L, s, qb);
    da[s] = row_operand(dos, L, s, qb);
    va[s] = row_operand(vs, L, s, kw);
  }
  sacc = f32x16{};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 d4 = *(const f32x4 *)(ndl + 32 * qb + 8 * i + 4 * hh);
#pragma unroll
    for (int j = 0; j < 4; ++j) dpacc[4 * i + j] = d4[j];
  }
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    if (s + kAhead < kSteps) {
      qa[s + kAhead] = row_operand(qs, L, s + kAhead, qb);
      da[s + kAhead] = row_operand(dos, L, s + kAhead, qb);
      va[s + kAhead] = row_operand(vs, L, s + kAhead, kw);
    }
    sacc = mfma32(qa[s], kreg[s], sacc);
    dpacc = mfma32(da[s], va[s], dpacc);
  }
}

template <int D, bool FUSE>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(const uint16_t *__restrict__ Q,
                                                        const uint16_t *__restrict__ K,
                                                        const uint16_t *__restrict__ V,
                                                        const uint16_t *__restrict__ dO,
                                                        const float *__restrict__ lse2g,
                                                        const float *__restrict__ delta, uint16_t *__restrict__ dK,
                                                        uint16_t *__restrict__ dV, int B, int T, int H, int KV,
                                                        int W, float scale, NormRopeBwd nb) {
  using Gm = Geom<D>;
  constexpr int kSteps = Gm::kSteps;
  constexpr int kTileBytes = Gm::kTileBytes;
  // Q | dO | lse2 | delta of 32 query rows, double-buffered in two LDS objects
  // (so the compiler can tell the copy into one from the reads of the other),
  // and V of the block's 128 keys
  constexpr int kR = 32;  // query rows per staged tile
  constexpr int kHalfTile = kR * Gm::kRowBytes;
  constexpr int kBuf = 2 * kHalfTile + 2 * 64 * 4;
  __shared__ __attribute__((aligned(1024))) char buf0[kBuf];
  __shared__ __attribute__((aligned(1024))) char buf1[kBuf];
  __shared__ __attribute__((aligned(1024))) char vtile[kBlockN * Gm::kRowBytes];
  __shared__ NormRopeLds<D> nrs;  // fused only
  const int tid = threadIdx.x;
  if constexpr (FUSE) stage_norm_rope<D>(nrs, nb, tid);  // read after the loop's barriers
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kw = wave;        // key sub-block (32 keys) of this wave
  const int hh = lane >> 5;
  const int G = H / KV;
  // key blocks near the start of the sequence see the most queries: launched
  // first; within one block row the (b, kv head) pairs (B KV apart, so with B KV
  // a multiple of 8 every block of one pair runs on the same XCD)
  const int BKV = B * KV;
  const int kblk = (int)(blockIdx.x / BKV);
  const int bk = (int)(blockIdx.x % BKV);
  const int b = bk / KV;
  const int kvh = bk % KV;
  const int k0 = kblk * kBlockN;
  const int kw0 = k0 + 32 * kw;
  const int key_lane = kw0 + (lane & 31);
  const float c = scale * kLog2e;

  const long long q_stride = (long long)H * D;
  const long long kv_stride = (long long)KV * D;
  const int voff = tile_lane_voff<D>((int)(q_stride * 2), tid);

  const int k_last_blk = min(k0 + kBlockN - 1, T - 1);
  const int q_hi = W < 0 ? T - 1 : min(T - 1, k_last_blk + W);
  const int qt0 = k0 / kR;
  const int nq = q_hi / kR - qt0 + 1;
  const int n_iter = nq * G;

  struct Pos {
    int qt, g;
  };
  auto advance = [&](Pos p) {
    if (++p.g == G) {
      p.g = 0;
      ++p.qt;
    }
    return p;
  };
  const long long qbase = (long long)b * T * q_stride + (long long)kvh * G * D;
  const long long rbase = ((long long)b * H + (long long)kvh * G) * T;

  auto stage = [&](const Pos &p, char *base) {
    const long long hoff = qbase + (long long)p.g * D;
    tile_load_lds<D, 4, kR>(base, make_tile_src(Q + hoff, q_stride, T), voff, p.qt * kR);
    tile_load_lds<D, 4, kR>(base + kHalfTile, make_tile_src(dO + hoff, q_stride, T), voff, p.qt * kR);
    if (wave < 2) {  // waves 0, 1: 64 lse rows and 64 delta rows, 4 bytes per lane (zeros past T)
      // the row address is the same on every lane: taken from the first (both
      // 32-bit halves; the builtin moves one dword), so the buffer resource is
      // built in scalar registers
      const unsigned long long ra =
          (unsigned long long)((wave == 0 ? lse2g : delta) + rbase + (long long)p.g * T);
      const unsigned ra_lo = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)ra);
      const unsigned ra_hi = (unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)(ra >> 32));
      const float *row = (const float *)(((unsigned long long)ra_hi << 32) | ra_lo);
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)row, (short)0, T * 4, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(base + 2 * kHalfTile + wave * 64 * 4), 4,
                                               lane * 4, p.qt * kR * 4, 0, 0);
    }
  };

  {  // V of the block's 128 keys, rows past T as zeros
    const TileSrc vsrc = make_tile_src(V + (long long)b * T * kv_stride + (long long)kvh * D, kv_stride, T);
    const int vvoff = tile_lane_voff<D>(vsrc.stride, tid);
    tile_load_lds<D, 4>(vtile, vsrc, vvoff, k0);
    tile_load_lds<D, 4>(vtile + kTileBytes, vsrc, vvoff, k0 + kTileN);
  }
  Pos pos{qt0, 0};
  stage(pos, buf0);

  bf16x8 kreg[kSteps];
  {
    const int kr = min(key_lane, T - 1);
    const long long off = ((long long)b * T + kr) * kv_stride + (long long)kvh * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) kreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(K + off + 16 * s));
  }
  const TileLane<D> L = make_tile_lane<D>(lane);
  const int kw_last = min(kw0 + 31, T - 1);
  const bool wave_active = kw0 < T;

  f32x16 dkacc[Gm::kDBlocks], dvacc[Gm::kDBlocks];
#pragma unroll
  for (int i = 0; i < Gm::kDBlocks; ++i) {
    dkacc[i] = f32x16{};
    dvacc[i] = f32x16{};
  }

  lds_loads_done_barrier();

  auto step = [&](char *cur, char *nxt, int it) {
    const char *qs = cur;
    const char *dos = cur + kHalfTile;
    const float *lse2 = (const float *)(cur + 2 * kHalfTile);
    const float *ndl = lse2 + 64;
    const Pos p = pos;
    pos = advance(pos);
    if (it + 1 < n_iter) stage(pos, nxt);
    const int qr0 = p.qt * kR;
    const bool act = wave_active && !(qr0 + 31 < kw0 || (W >= 0 && qr0 - kw_last > W));
    if (act) {
      const bool msk = !(qr0 >= kw_last && (W < 0 || qr0 + 31 - kw0 <= W) && qr0 + 31 < T);
      f32x16 s0, p0;
      dkdv_sdp<D>(s0, p0, qs, dos, vtile, ndl, L, kreg, 0, kw, hh);
      if (msk) dkdv_mask(s0, 0, qr0, key_lane, T, W, hh);
      dkdv_p_ds_acc<D>(dkacc, dvacc, s0, p0, lse2, c, hh, qs, dos, L);
    }
    lds_loads_done_barrier();
  };
  for (int it = 0; it < n_iter; it += 2) {
    step(buf0, buf1, it);
    if (it + 1 >= n_iter) break;
    step(buf1, buf0, it + 1);
  }

  if (!wave_active || key_lane >= T) return;
  const long long off = ((long long)b * T + key_lane) * kv_stride + (long long)kvh * D;
  float kscale = scale;
  if constexpr (FUSE) {
#pragma unroll
    for (int db = 0; db < Gm::kDBlocks; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dkacc[db][e] *= scale;
    // the norm's arguments, from their copy in LDS
    const double posd = (double)((nrs.pos_offset ? nrs.pos_offset[b] : 0) + key_lane);
    const float rs = nrs.rstd[((long long)b * T + key_lane) * nrs.rstd_stride + nrs.rstd_k_off + kvh];
    norm_rope_bwd_row<D>(dkacc, K + off, rs, posd, nrs, hh);
    kscale = 1.f;
  }
#pragma unroll
  for (int db = 0; db < Gm::kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * hh;
      u32x2 wk, wv;
      wk[0] = pack_bf16x2(dkacc[db][4 * i + 0] * kscale, dkacc[db][4 * i + 1] * kscale);
      wk[1] = pack_bf16x2(dkacc[db][4 * i + 2] * kscale, dkacc[db][4 * i + 3] * kscale);
      wv[0] = pack_bf16x2(dvacc[db][4 * i + 0], dvacc[db][4 * i + 1]);
      wv[1] = pack_bf16x2(dvacc[db][4 * i + 2], dvacc[db][4 * i + 3]);
      *(u32x2 *)(dK + off + d) = wk;
      *(u32x2 *)(dV + off + d) = wv;
    }
}

// S^T = K Q^T (or dP^T = V dO^T) of one 64-key tile against the wave's 32
// queries: keys as MFMA rows (two 32-key blocks), queries as columns; element e of
// acc[kb] is key 32 kb + 8 (e >> 2) + 4 hh + (e & 3) of the lane's query.  The
// row operands are read four MFMAs ahead of their use.
template <int D>
__device__ __forceinline__ void dq_st_tile(f32x16 (&acc)[2], const char *tile, const TileLane<D> &L,
                                           const bf16x8 (&breg)[Geom<D>::kSteps]) {
  constexpr int kAhead = 4;
  constexpr int kN = 2 * Geom<D>::kSteps;
  bf16x8 op[kN];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) op[i] = row_operand(tile, L, i >> 1, i & 1);
  acc[0] = f32x16{};
  acc[1] = f32x16{};
#pragma unroll
  for (int i = 0; i < kN; ++i) {  // i = 2 s + kb
    if (i + kAhead < kN) op[i + kAhead] = row_operand(tile, L, (i + kAhead) >> 1, (i + kAhead) & 1);
    acc[i & 1] = mfma32(op[i], breg[i >> 1], acc[i & 1]);
  }
}

// dP^T = V dO^T for the tile (as dq_st_tile), with the exponentials of the
// tile's scores placed among its MFMAs (P = exp2(S c - LSE log2 e) in place of
// S^T, 32 / (2 D / 16) after each MFMA), so that one wave's exponentials run
// while its own MFMAs execute.  Operands read four MFMAs ahead.
template <int D>
__device__ __forceinline__ void dq_dp_tile_exp(f32x16 (&dpacc)[2], const char *vs, const TileLane<D> &L,
                                               const bf16x8 (&dreg)[Geom<D>::kSteps], f32x16 (&sacc)[2], float c,
                                               float lse2_q) {
  constexpr int kAhead = 4;
  constexpr int kN = 2 * Geom<D>::kSteps;
  constexpr int kPer = 32 / kN;
  bf16x8 op[kN];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) op[i] = row_operand(vs, L, i >> 1, i & 1);
  dpacc[0] = f32x16{};
  dpacc[1] = f32x16{};
#pragma unroll
  for (int i = 0; i < kN; ++i) {  // i = 2 s + kb
    if (i + kAhead < kN) op[i + kAhead] = row_operand(vs, L, (i + kAhead) >> 1, (i + kAhead) & 1);
    dpacc[i & 1] = mfma32(op[i], dreg[i >> 1], dpacc[i & 1]);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int x = i * kPer + k;
      sacc[x >> 4][x & 15] = fast_exp2(__builtin_fmaf(sacc[x >> 4][x & 15], c, -lse2_q));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// -inf on the elements of a straddling tile that are not visible: with
// d0 = k0 + 4 hh - q_lane, element (kb, e) has key - query = d0 + off(kb, e).
__device__ __forceinline__ void dq_mask_tile(f32x16 (&sacc)[2], int k0, int q_lane, int W, int hh) {
  const int d0 = k0 + 4 * hh - q_lane;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int off = 32 * kb + 8 * (e >> 2) + (e & 3);
      const bool vis = d0 <= -off && (W < 0 || d0 + W >= -off);
      sacc[kb][e] = vis ? sacc[kb][e] : -INFINITY;
    }
}

// ---------------------------------------------------------------- dQ
// dQ_i = scale sum_j dS_ij k_j, with dS recomputed per tile: one workgroup per
// (b, h, 128-row query block), laid out like the forward (wave w owns query rows
// 32 w .. 32 w + 31; Q^T and dO^T of its rows in registers, one query per lane
// pair).  Per 64-key tile, with K and V copied global -> LDS one tile ahead:
//   S^T = K Q^T and dP^T = V dO^T (keys as MFMA rows, the wave's queries as
//   columns), P = exp2(S c - LSE log2 e) (masked on straddling tiles),
//   dS = P (dP - D), and dQ^T += K^T (dS_hi + dS_lo) straight from the
// accumulators (K^T through transposing LDS reads).  Nothing is stored between
// the stages, so the backward needs no O(T^2) workspace, and dS enters the dQ
// product in fp32 precision (hi + lo).
template <int D, bool FUSE>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(const uint16_t *__restrict__ Q,
                                                        const uint16_t *__restrict__ K,
                                                        const uint16_t *__restrict__ V,
                                                        const uint16_t *__restrict__ dO,
                                                        const float *__restrict__ lse2g,
                                                        const float *__restrict__ ndelta, uint16_t *__restrict__ dQ,
                                                        int B, int T, int H, int KV, int W, float scale,
                                                        NormRopeBwd nb) {
  using Gm = Geom<D>;
  constexpr int kSteps = Gm::kSteps;
  __shared__ __attribute__((aligned(1024))) char kb0[Gm::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char kb1[Gm::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vb0[Gm::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vb1[Gm::kTileBytes];
  __shared__ NormRopeLds<D> nrs;  // fused only
  const int tid = threadIdx.x;
  if constexpr (FUSE) stage_norm_rope<D>(nrs, nb, tid);  // read after the loop's barriers
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // launch order as the forward's: heaviest query blocks first, the G heads of a
  // (b, kv head) B KV blocks apart (same XCD when B KV is a multiple of 8)
  const int nqb = (T + kDqRows - 1) / kDqRows;
  const int G = H / KV;
  const int BH = B * H;
  const int BKV = B * KV;
  const int qblk = nqb - 1 - (int)(blockIdx.x / BH);
  const int j = (int)(blockIdx.x % BH);
  const int bkv = j % BKV;
  const int b = bkv / KV;
  const int kvh = bkv % KV;
  const int h = kvh * G + j / BKV;
  const int q0 = qblk * kDqRows;
  const int qw0 = q0 + 32 * wave;
  const int hh = lane >> 5;
  const int q_lane = qw0 + (lane & 31);
  const int qr = min(q_lane, T - 1);
  const float c = scale * kLog2e;
  const long long q_stride = (long long)H * D;
  const long long kv_stride = (long long)KV * D;
  const TileSrc ksrc = make_tile_src(K + (long long)b * T * kv_stride + (long long)kvh * D, kv_stride, T);
  const TileSrc vsrc = make_tile_src(V + (long long)b * T * kv_stride + (long long)kvh * D, kv_stride, T);
  const int voff = tile_lane_voff<D>(ksrc.stride, tid);

  const int q_last_blk = min(q0 + kDqRows - 1, T - 1);
  const int t0 = (W < 0 ? 0 : max(0, q0 - W)) / kTileN;
  const int t1 = q_last_blk / kTileN;
  const int qw_last = min(qw0 + 31, T - 1);
  const bool wave_active = qw0 < T;
  const int tw0 = max(t0, (W < 0 ? 0 : max(0, qw0 - W)) / kTileN);
  const int tw1 = wave_active ? qw_last / kTileN : t0 - 1;

  tile_load_lds<D>(kb0, ksrc, voff, t0 * kTileN);
  tile_load_lds<D>(vb0, vsrc, voff, t0 * kTileN);

  // Q^T and dO^T operands of this lane's query (d = 16 s + 8 hh + [0, 8)), its
  // LSE log2 e and -D
  bf16x8 qreg[kSteps], dreg[kSteps];
  {
    const long long off = ((long long)b * T + qr) * q_stride + (long long)h * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      qreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(Q + off + 16 * s));
      dreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(dO + off + 16 * s));
    }
  }
  const long long ri = ((long long)b * H + h) * T + qr;
  const float lse2_q = lse2g[ri];
  const float nd_q = ndelta[ri];
  const TileLane<D> L = make_tile_lane<D>(lane);

  f32x16 dqacc[Gm::kDBlocks];
#pragma unroll
  for (int i = 0; i < Gm::kDBlocks; ++i) dqacc[i] = f32x16{};

  lds_loads_done_barrier();

  auto step = [&](const char *ks, const char *vs, char *kfill, char *vfill, int t) {
    if (t + 1 <= t1) {
      tile_load_lds<D>(kfill, ksrc, voff, (t + 1) * kTileN);
      tile_load_lds<D>(vfill, vsrc, voff, (t + 1) * kTileN);
    }
    if (t >= tw0 && t <= tw1) {
      const int k0 = t * kTileN;
      f32x16 sacc[2], dpacc[2];
      dq_st_tile(sacc, ks, L, qreg);
      // scheduling of those 16 MFMAs and their LDS operand reads: each read four
      // MFMAs ahead of its use
#pragma unroll
      for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (!(k0 + kTileN - 1 <= qw0 && (W < 0 || qw_last - k0 <= W))) dq_mask_tile(sacc, k0, q_lane, W, hh);
      // P in place of S^T (among the dP MFMAs), then dS^T = P (dP - D)
      dq_dp_tile_exp(dpacc, vs, L, dreg, sacc, c, lse2_q);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] *= dpacc[kb][e] + nd_q;
#pragma unroll
      for (int cs = 0; cs < 4; ++cs) {
        bf16x8 dh, dl;
        acc_to_operand_split(sacc[cs >> 1], cs & 1, dh, dl);
#pragma unroll
        for (int db = 0; db < Gm::kDBlocks; ++db) {
          const bf16x8 a = col_operand(ks, L, db, cs);
          dqacc[db] = mfma32(a, dh, dqacc[db]);
          dqacc[db] = mfma32(a, dl, dqacc[db]);
        }
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
  const long long qoff = ((long long)b * T + q_lane) * q_stride + (long long)h * D;
  uint16_t *dqp = dQ + qoff;
  float qscale = scale;
  if constexpr (FUSE) {
#pragma unroll
    for (int db = 0; db < Gm::kDBlocks; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dqacc[db][e] *= scale;
    const double pos = (double)((nrs.pos_offset ? nrs.pos_offset[b] : 0) + q_lane);
    const float rs = nrs.rstd[((long long)b * T + q_lane) * nrs.rstd_stride + h];
    norm_rope_bwd_row<D>(dqacc, Q + qoff, rs, pos, nrs, hh);
    qscale = 1.f;
  }
#pragma unroll
  for (int db = 0; db < Gm::kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * hh;
      u32x2 w;
      w[0] = pack_bf16x2(dqacc[db][4 * i + 0] * qscale, dqacc[db][4 * i + 1] * qscale);
      w[1] = pack_bf16x2(dqacc[db][4 * i + 2] * qscale, dqacc[db][4 * i + 3] * qscale);
      *(u32x2 *)(dqp + d) = w;
    }
}


template <int D, bool FUSE>
hipError_t launch_bwd_kernels(const void *q, const void *k, const void *v, const void *o, const float *lse,
                              const void *dout, void *dq, void *dk, void *dv, void *workspace, const AttnShape &sh,
                              int stages, const NormRopeBwd &nq, const NormRopeBwd &nk, hipStream_t s) {
  const size_t row_bytes = bwd_row_bytes(sh.B, sh.T, sh.H);
  float *delta = (float *)workspace;
  float *lse2 = (float *)((char *)workspace + row_bytes);
  const long long rows = (long long)sh.B * sh.T * sh.H;
  const long long dblocks = (rows + 63) / 64;
  const long long nkb = (sh.T + kBlockN - 1) / kBlockN;
  const long long nqb = (sh.T + kDqRows - 1) / kDqRows;
  const long long kvblocks = nkb * sh.B * sh.KV;
  const long long qblocks = nqb * sh.B * sh.H;
  if (dblocks > 0x7fffffffLL || kvblocks > 0x7fffffffLL || qblocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (stages & kBwdDelta)
    hipLaunchKernelGGL(bwd_delta_kernel<D>, dim3((unsigned)dblocks), dim3(256), 0, s, (const uint16_t *)o,
                       (const uint16_t *)dout, lse, delta, lse2, sh.B, sh.T, sh.H);
  if (stages & kBwdDkDv)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, FUSE>), dim3((unsigned)kvblocks), dim3(256), 0, s, (const uint16_t *)q,
                       (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dout, lse2, delta, (uint16_t *)dk,
                       (uint16_t *)dv, sh.B, sh.T, sh.H, sh.KV, sh.window, sh.scale, nk);
  if (stages & kBwdDq)
    hipLaunchKernelGGL((bwd_dq_kernel<D, FUSE>), dim3((unsigned)qblocks), dim3(256), 0, s, (const uint16_t *)q,
                       (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dout, lse2, delta, (uint16_t *)dq,
                       sh.B, sh.T, sh.H, sh.KV, sh.window, sh.scale, nq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                           const void *dout, void *dq, void *dk, void *dv, void *workspace, const AttnShape &sh,
                           int stages, hipStream_t s) {
  const NormRopeBwd none{};
  if (sh.D == 64)
    return launch_bwd_kernels<64, false>(q, k, v, o, lse, dout, dq, dk, dv, workspace, sh, stages, none, none, s);
  if (sh.D == 128)
    return launch_bwd_kernels<128, false>(q, k, v, o, lse, dout, dq, dk, dv, workspace, sh, stages, none, none, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_bf16_qknorm_rope(const void *q, const void *k, const void *v, const void *o, const float *lse,
                                       const void *dout, const float *rstd, void *dq, void *dk, void *dv,
                                       void *workspace, const AttnShape &sh, const int32_t *pos_offset,
                                       const double *inv_freq_host, float gain, hipStream_t s) {
  NormRopeBwd nb{};
  for (int j = 0; j < sh.D / 2; ++j) nb.turns[j] = inv_freq_host[j] / 6.283185307179586;
  nb.rstd = rstd;
  nb.rstd_stride = (long long)sh.H + sh.KV;
  nb.rstd_k_off = sh.H;
  nb.pos_offset = pos_offset;
  nb.gain = gain;
  if (sh.D == 64)
    return launch_bwd_kernels<64, true>(q, k, v, o, lse, dout, dq, dk, dv, workspace, sh, kBwdAll, nb, nb, s);
  if (sh.D == 128)
    return launch_bwd_kernels<128, true>(q, k, v, o, lse, dout, dq, dk, dv, workspace, sh, kBwdAll, nb, nb, s);
  return hipErrorInvalidValue;
}

}  // namespace ncattn
