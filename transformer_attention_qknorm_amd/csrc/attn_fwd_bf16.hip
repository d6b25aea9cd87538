// Attention forward, bf16 in/out, fp32 accumulation, head_dim 64 or 128, gfx950 MFMA.
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
// global -> LDS directly (no register staging).  Each wave computes S^T = K Q^T
// (keys as MFMA rows, queries as columns) so that every lane holds one query's
// scores: the row max and row sum are lane-local plus one exchange with lane
// l^32, and the probabilities feed O^T += V^T P^T directly as the MFMA B operand
// (V^T comes from LDS with transposing reads).
//
// Software pipeline: in step t a wave issues the S^T MFMAs of tile t+1 (their K
// operands read four MFMAs ahead) with the softmax exponentials of tile t placed
// among them, then O += P V for tile t; two workgroups share a CU, so a SIMD runs
// two such waves.  K therefore runs one tile ahead of V: step t reads K(t+1) and
// V(t) while K(t+2) and V(t+1) are being copied into the other halves of two LDS
// rings.
// Tiles entirely outside a wave's window are skipped; masks are applied only on
// tiles that straddle the causal diagonal or the window edge.
//
// Exponent reference: a row's offset is the max of its first tile with a visible
// key and stays fixed, so O is never rescaled and no tile max is needed after the
// first.  That is exact as long as no probability exceeds 2^64 (the sums stay far
// inside fp32); a tile whose row sum does exceed it sends the workgroup through a
// second pass that computes the exact row maxima first and repeats the loop with
// them.
#include "attn_tiles.hpp"
#include "internal.hpp"

namespace ncattn {

namespace {

constexpr int kBlockM = 128;
constexpr float kSumLimit = 18446744073709551616.0f;  // 2^64

template <int D>
struct FwdState {
  f32x16 oacc[Geom<D>::kDBlocks];
  float m_ref;  // exponent reference of the raw scores (both half-waves agree; -inf: none yet)
  float l_run;  // this lane's partial row sum (its 32 of every 64 keys)
};

// The K operands are read from LDS four MFMAs ahead of their use (the reads are
// fenced in place, so their latency hides under the MFMAs in between).
template <int D>
__device__ __forceinline__ void s_tile(f32x16 (&sacc)[2], const char *ks, const TileLane<D> &L,
                                       const bf16x8 (&qreg)[Geom<D>::kSteps]) {
  constexpr int kAhead = 4;
  constexpr int kN = 2 * Geom<D>::kSteps;
  bf16x8 kop[kN];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) kop[i] = row_operand(ks, L, i >> 1, i & 1);
  sacc[0] = f32x16{};
  sacc[1] = f32x16{};
#pragma unroll
  for (int i = 0; i < kN; ++i) {  // i = 2 s + kb
    if (i + kAhead < kN) kop[i + kAhead] = row_operand(ks, L, (i + kAhead) >> 1, (i + kAhead) & 1);
    sacc[i & 1] = mfma32(kop[i], qreg[i >> 1], sacc[i & 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// s_tile for tile t+1 with tile t's exponentials (softmax_exp below) placed
// among its MFMAs, 32 / (2 D / 16) of them after each MFMA, so that one wave's
// exponentials run while its own MFMAs execute.
template <int D>
__device__ __forceinline__ void s_tile_exp(f32x16 (&snext)[2], const char *ks, const TileLane<D> &L,
                                           const bf16x8 (&qreg)[Geom<D>::kSteps], FwdState<D> &st,
                                           f32x16 (&scur)[2], float c, bool &overflow) {
  constexpr int kAhead = 4;
  constexpr int kN = 2 * Geom<D>::kSteps;
  constexpr int kPer = 32 / kN;
  const float nmc = (st.m_ref == -INFINITY) ? 0.f : -st.m_ref * c;
  float ls = 0.f;
  bf16x8 kop[kN];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) kop[i] = row_operand(ks, L, i >> 1, i & 1);
  snext[0] = f32x16{};
  snext[1] = f32x16{};
#pragma unroll
  for (int i = 0; i < kN; ++i) {  // i = 2 s + kb
    if (i + kAhead < kN) kop[i + kAhead] = row_operand(ks, L, (i + kAhead) >> 1, (i + kAhead) & 1);
    snext[i & 1] = mfma32(kop[i], qreg[i >> 1], snext[i & 1]);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int x = i * kPer + k;
      const float p = fast_exp2(__builtin_fmaf(scur[x >> 4][x & 15], c, nmc));
      scur[x >> 4][x & 15] = p;
      ls += p;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  overflow |= ls > kSumLimit;
  st.l_run += ls;
}

// Masks a tile that straddles the causal diagonal or the window edge.  Element e
// of sacc[kb] is key k0 + 32 kb + 8 (e >> 2) + 4 hh + (e & 3) of query q_lane.
// With d0 = k0 + 4 hh - q_lane, element (kb, e) has key - query = d0 + off(kb, e)
// for a compile-time off, so each condition is one compare of d0 (or of
// d0 + W) against a constant.
__device__ __forceinline__ void mask_tile(f32x16 (&sacc)[2], int k0, int q_lane, int W, int hh) {
  const int d0 = k0 + 4 * hh - q_lane;
  if (W < 0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int off = 32 * kb + 8 * (e >> 2) + (e & 3);
        const float x = sacc[kb][e];
        sacc[kb][e] = d0 <= -off ? x : -INFINITY;  // key <= query
      }
  } else {
    const int d0w = d0 + W;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int off = 32 * kb + 8 * (e >> 2) + (e & 3);
        const float x = sacc[kb][e];
        sacc[kb][e] = (d0 <= -off && d0w >= -off) ? x : -INFINITY;  // and query - key <= W
      }
  }
}

// Row max of a tile, agreed by the lane pair (l, l^32).
__device__ __forceinline__ float tile_max(const f32x16 (&sacc)[2]) {
  float mt = sacc[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kb][e]);
  return fmaxf(mt, shfl_xor(mt, 32));
}

// Gives rows without a reference yet (their O and l are still zero) the max of
// this tile.
template <int D>
__device__ __forceinline__ void init_ref(FwdState<D> &st, const f32x16 (&sacc)[2]) {
  if (__any(st.m_ref == -INFINITY)) {
    const float mt = tile_max(sacc);
    if (st.m_ref == -INFINITY) st.m_ref = mt;
  }
}

// Probabilities (in place) and the row-sum update; a row sum above 2^64 (or
// infinite) raises `overflow`.
template <int D>
__device__ __forceinline__ void softmax_exp(FwdState<D> &st, f32x16 (&sacc)[2], float c, bool &overflow) {
  const float nmc = (st.m_ref == -INFINITY) ? 0.f : -st.m_ref * c;
  float ls = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = fast_exp2(__builtin_fmaf(sacc[kb][e], c, nmc));
      sacc[kb][e] = p;
      ls += p;
    }
  overflow |= ls > kSumLimit;
  st.l_run += ls;
}

// O^T += V^T P^T with the probabilities as bf16 hi + lo (two MFMAs per block):
// a single bf16 P leaves O off by ~2^-9 relative before its own rounding, which
// moves the stored O by an ulp often enough to matter downstream (the backward's
// D = dO . O) and to miss 2e-2 where |O| >= 4.
template <int D>
__device__ __forceinline__ void pv_tile(FwdState<D> &st, const f32x16 (&pacc)[2], const char *vs,
                                        const TileLane<D> &L) {
#pragma unroll
  for (int cs = 0; cs < 4; ++cs) {
    bf16x8 pb, pl;
    acc_to_operand_split(pacc[cs >> 1], cs & 1, pb, pl);
#pragma unroll
    for (int db = 0; db < Geom<D>::kDBlocks; ++db) {
      const bf16x8 a = col_operand(vs, L, db, cs);
      st.oacc[db] = mfma32(a, pb, st.oacc[db]);
      st.oacc[db] = mfma32(a, pl, st.oacc[db]);
    }
  }
}

// QK-norm + RoPE of the query rows, for the fused forward: rotation turns per
// position of pair j < D/2 (base^(-2j/D) / 2 pi), epsilon, gain, position offsets.
struct QkNormRope {
  double turns[64];
  float eps, gain;
  const int32_t *pos_offset;  // device [B] or NULL
  float *rstd;                // NULL, or each query row's 1/r at rstd[token * rstd_stride + head]
  long long rstd_stride;
};

// FUSE: the query rows arrive raw; the prologue normalises and rotates them in
// registers ("nanochat Admin & Developer Guide", section 3: weightless RMSNorm of
// q, then rotary embedding) and writes them back through Qw (the same array as Q,
// each row touched by the one lane pair that owns it).
template <int D, bool FUSE>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(const uint16_t *__restrict__ Q,
                                                               const uint16_t *__restrict__ K,
                                                               const uint16_t *__restrict__ V,
                                                               uint16_t *__restrict__ O, float *__restrict__ LSE,
                                                               const int32_t *__restrict__ q_pos0, int B, int Tq,
                                                               int Tk, int H, int KV, int W, float scale,
                                                               uint16_t *Qw, QkNormRope qn) {
  // Two-slot rings for K and V, each slot its own LDS object so the compiler can
  // tell a copy into one slot from reads of the other.
  using Gm = Geom<D>;
  constexpr int kSteps = Gm::kSteps;
  __shared__ __attribute__((aligned(1024))) char kb0[Gm::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char kb1[Gm::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vb0[Gm::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char vb1[Gm::kTileBytes];
  __shared__ int overflow_flag;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // Launch order: query blocks heaviest (latest) first; within one block row the
  // query head's group index g major and (b, kv head) minor, so that the G heads
  // reading one (b, kv head)'s K/V get block indexes B KV apart: workgroups are
  // dealt to the 8 XCDs (each with its own L2) round-robin, so with B KV a
  // multiple of 8 they share an XCD and its L2.
  const int nqb = (Tq + kBlockM - 1) / kBlockM;
  const int G = H / KV;
  const int BH = B * H;
  const int BKV = B * KV;
  const int qblk = nqb - 1 - (int)(blockIdx.x / BH);
  const int j = (int)(blockIdx.x % BH);
  const int bkv = j % BKV;
  const int b = bkv / KV;
  const int kvh = bkv % KV;
  const int h = kvh * G + j / BKV;
  const int q0 = qblk * kBlockM;  // query rows of the block (index into Q / O)
  const int qw0 = q0 + 32 * wave;
  const int hh = lane >> 5;
  const float c = scale * kLog2e;
  const long long q_stride = (long long)H * D;
  const long long kv_stride = (long long)KV * D;

  // Query row r sits at position s0 + r of a sequence whose keys are rows
  // [0, s0 + Tq) of K / V (s0 = 0 for a whole sequence; the cache length before a
  // chunk for a prefill, which must leave the chunk inside the Tk rows).
  const int s0 = q_pos0 ? q_pos0[b] : 0;
  if (s0 < 0 || s0 > Tk - Tq) {
    // invalid cache length: this block's rows of o and lse are NaN
    const int qr = qw0 + (lane & 31);
    if (qr < Tq) {
      uint16_t *op = O + ((long long)b * Tq + qr) * q_stride + (long long)h * D;
      for (int d = 4 * hh; d < D; d += 8) *(u32x2 *)(op + d) = u32x2{0x7fc07fc0u, 0x7fc07fc0u};
      if (hh == 0 && LSE) LSE[((long long)b * H + h) * Tq + qr] = __builtin_nanf("");
    }
    return;
  }
  const int nkeys = s0 + Tq;
  const int q_lane = s0 + qw0 + (lane & 31);  // position of this lane's query
  const int pw0 = s0 + qw0;                   // position of the wave's first query
  const uint16_t *Kb = K + (long long)b * Tk * kv_stride + (long long)kvh * D;
  const uint16_t *Vb = V + (long long)b * Tk * kv_stride + (long long)kvh * D;
  const TileSrc ksrc = make_tile_src(Kb, kv_stride, nkeys);
  const TileSrc vsrc = make_tile_src(Vb, kv_stride, nkeys);
  const int voff = tile_lane_voff<D>(ksrc.stride, tid);

  // key tiles of the block, and the contiguous range of them this wave needs
  const int p_last_blk = s0 + min(q0 + kBlockM - 1, Tq - 1);
  const int t0 = (W < 0 ? 0 : max(0, s0 + q0 - W)) / kTileN;
  const int t1 = p_last_blk / kTileN;
  const int pw_last = s0 + min(qw0 + 31, Tq - 1);
  const bool wave_active = qw0 < Tq;
  const int tw0 = max(t0, (W < 0 ? 0 : max(0, pw0 - W)) / kTileN);
  const int tw1 = wave_active ? pw_last / kTileN : t0 - 1;  // empty range if inactive
  auto in_range = [&](int t) { return t >= tw0 && t <= tw1; };
  auto masked = [&](int t) {
    const int k0 = t * kTileN;
    return !(k0 + kTileN - 1 <= pw0 && (W < 0 || pw_last - k0 <= W));
  };

  tile_load_lds<D>(kb0, ksrc, voff, t0 * kTileN);
  tile_load_lds<D>(vb0, vsrc, voff, t0 * kTileN);
  if (t0 + 1 <= t1) tile_load_lds<D>(kb1, ksrc, voff, (t0 + 1) * kTileN);

  // Q^T operand in registers: lane holds the query of row qw0 + l%32, d = 16 s + 8 hh + [0, 8).
  bf16x8 qreg[kSteps];
  if constexpr (!FUSE) {
    const int qr = min(qw0 + (lane & 31), Tq - 1);
    const uint16_t *qp = Q + ((long long)b * Tq + qr) * q_stride + (long long)h * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qreg[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qp + 16 * s));
  } else {
    // The row's D elements are split between lanes l and l ^ 32 (D/2 each); the
    // rotation pairs d and d + D/2 are steps s and s + kSteps/2 of the same lane.
    const int qrow = qw0 + (lane & 31);
    const int qr = min(qrow, Tq - 1);
    uint16_t *qp = Qw + ((long long)b * Tq + qr) * q_stride + (long long)h * D + 8 * hh;
    u32x4 raw[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) raw[s] = *(const u32x4 *)(qp + 16 * s);
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) ss += lo_bf16(raw[s][i]) * lo_bf16(raw[s][i]) + hi_bf16(raw[s][i]) * hi_bf16(raw[s][i]);
    ss += shfl_xor(ss, 32);
    const float rs = 1.f / sqrtf(ss / (float)D + qn.eps);
    const float inv = qn.gain * rs;
    if (qn.rstd != nullptr && hh == 0 && qrow < Tq) qn.rstd[((long long)b * Tq + qrow) * qn.rstd_stride + h] = rs;
    const double pos = (double)((qn.pos_offset ? qn.pos_offset[b] : 0) + qr);
    constexpr int kHalf = kSteps / 2;
#pragma unroll
    for (int s = 0; s < kHalf; ++s) {
      u32x4 ya, yb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float ra[2], rb[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j0 = 16 * s + 2 * i + e;  // pair index for hh = 0; hh = 1 adds 8
          // both candidates as uniform (scalar) loads, then a per-lane select: a
          // per-lane index into the argument block would become a vector load
          double f_lo = qn.turns[j0], f_hi = qn.turns[j0 + 8];
          asm("" : "+s"(f_lo), "+s"(f_hi));
          double turns = pos * (hh ? f_hi : f_lo);
          turns -= rint(turns);
          const float tf = (float)turns;
          const float sn = __builtin_amdgcn_sinf(tf), cs = __builtin_amdgcn_cosf(tf);
          const float a = (e ? hi_bf16(raw[s][i]) : lo_bf16(raw[s][i])) * inv;
          const float bb = (e ? hi_bf16(raw[s + kHalf][i]) : lo_bf16(raw[s + kHalf][i])) * inv;
          ra[e] = a * cs - bb * sn;
          rb[e] = a * sn + bb * cs;
        }
        ya[i] = pack_bf16x2(ra[0], ra[1]);
        yb[i] = pack_bf16x2(rb[0], rb[1]);
      }
      raw[s] = ya;
      raw[s + kHalf] = yb;
    }
    if (qrow < Tq) {
#pragma unroll
      for (int s = 0; s < kSteps; ++s) *(u32x4 *)(qp + 16 * s) = raw[s];
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) qreg[s] = __builtin_bit_cast(bf16x8, raw[s]);
  }
  const TileLane<D> L = make_tile_lane<D>(lane);

  FwdState<D> st;
  float m_init = -INFINITY;
  if (tid == 0) overflow_flag = 0;

#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      // Rare: a probability exceeded 2^64 against its row's reference.  Compute
      // the exact row maxima over the wave's tiles, then repeat the loop.
      if (!overflow_flag) break;
#pragma unroll 1
      for (int t = t0; t <= t1; ++t) {
        tile_load_lds<D>(kb0, ksrc, voff, t * kTileN);
        lds_loads_done_barrier();
        if (in_range(t)) {
          f32x16 sx[2];
          s_tile(sx, kb0, L, qreg);
          mask_tile(sx, t * kTileN, q_lane, W, hh);
          m_init = fmaxf(m_init, tile_max(sx));
        }
        __syncthreads();
      }
      tile_load_lds<D>(kb0, ksrc, voff, t0 * kTileN);
      tile_load_lds<D>(vb0, vsrc, voff, t0 * kTileN);
      if (t0 + 1 <= t1) tile_load_lds<D>(kb1, ksrc, voff, (t0 + 1) * kTileN);
    }
#pragma unroll
    for (int i = 0; i < Gm::kDBlocks; ++i) st.oacc[i] = f32x16{};
    st.m_ref = m_init;
    st.l_run = 0.f;
    bool overflow = false;

    lds_loads_done_barrier();
    f32x16 scur[2], snext[2];
    if (in_range(t0)) s_tile(scur, kb0, L, qreg);
    __syncthreads();  // every wave is done with K(t0) before its slot is refilled

    // Step t: S of tile t+1 from kcur, softmax + PV of tile t from vcur; copies of
    // K(t+2) into kfill and V(t+1) into vfill run meanwhile.
    auto step = [&](const char *kcur, char *kfill, const char *vcur, char *vfill, int t) {
      if (t + 2 <= t1) tile_load_lds<D>(kfill, ksrc, voff, (t + 2) * kTileN);
      if (t + 1 <= t1) tile_load_lds<D>(vfill, vsrc, voff, (t + 1) * kTileN);
      const bool cur = in_range(t), next = in_range(t + 1);
      if (cur) {
        if (masked(t)) mask_tile(scur, t * kTileN, q_lane, W, hh);
        init_ref(st, scur);
      }
      if (cur && next) {
        // steady state: one straight-line block holding the S MFMAs of tile t+1
        // with the exponentials of tile t among them, then the PV MFMAs of tile t
        s_tile_exp(snext, kcur, L, qreg, st, scur, c, overflow);
        pv_tile(st, scur, vcur, L);
        scur[0] = snext[0];
        scur[1] = snext[1];
      } else if (cur) {
        softmax_exp(st, scur, c, overflow);
        pv_tile(st, scur, vcur, L);
      } else if (next) {
        s_tile(scur, kcur, L, qreg);
      }
      lds_loads_done_barrier();
    };
    for (int t = t0; t <= t1; t += 2) {
      step(kb1, kb0, vb0, vb1, t);
      if (t + 1 > t1) break;
      step(kb0, kb1, vb1, vb0, t + 1);
    }
    if (__any(overflow) && lane == 0) overflow_flag = 1;
    __syncthreads();
  }

  if (!wave_active) return;
  const float l_tot = st.l_run + shfl_xor(st.l_run, 32);
  const float inv_l = 1.f / l_tot;
  const int qr = qw0 + (lane & 31);
  if (qr < Tq) {
    uint16_t *op = O + ((long long)b * Tq + qr) * q_stride + (long long)h * D;
#pragma unroll
    for (int db = 0; db < Gm::kDBlocks; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * i + 4 * hh;
        u32x2 w;
        w[0] = pack_bf16x2(st.oacc[db][4 * i + 0] * inv_l, st.oacc[db][4 * i + 1] * inv_l);
        w[1] = pack_bf16x2(st.oacc[db][4 * i + 2] * inv_l, st.oacc[db][4 * i + 3] * inv_l);
        *(u32x2 *)(op + d) = w;
      }
    if (hh == 0 && LSE) LSE[((long long)b * H + h) * Tq + qr] = st.m_ref * scale + logf(l_tot);
  }
}

}  // namespace

template <int D, bool FUSE>
hipError_t launch_fwd_kernel(const void *q, const void *k, const void *v, void *o, float *lse,
                             const int32_t *q_pos0, int B, int Tq, int Tk, int H, int KV, int W, float scale,
                             void *qw, const QkNormRope &qn, hipStream_t s) {
  const int nqb = (Tq + kBlockM - 1) / kBlockM;
  const long long blocks = (long long)nqb * B * H;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, FUSE>), dim3((unsigned)blocks), dim3(256), 0, s, (const uint16_t *)q,
                     (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)o, lse, q_pos0, B, Tq, Tk, H, KV, W, scale,
                     (uint16_t *)qw, qn);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16_rows(const void *q, const void *k, const void *v, void *o, float *lse,
                                const int32_t *q_pos0, int B, int Tq, int Tk, int H, int KV, int D, int W,
                                float scale, hipStream_t s) {
  const QkNormRope none{};
  if (D == 64)
    return launch_fwd_kernel<64, false>(q, k, v, o, lse, q_pos0, B, Tq, Tk, H, KV, W, scale, nullptr, none, s);
  if (D == 128)
    return launch_fwd_kernel<128, false>(q, k, v, o, lse, q_pos0, B, Tq, Tk, H, KV, W, scale, nullptr, none, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16_qknorm_rope(void *q, const void *k, const void *v, void *o, float *lse,
                                       const AttnShape &sh, const int32_t *pos_offset,
                                       const double *inv_freq_host, float eps, float gain, hipStream_t s,
                                       float *rstd, long long rstd_stride) {
  QkNormRope qn{};
  for (int j = 0; j < sh.D / 2; ++j) qn.turns[j] = inv_freq_host[j] / 6.283185307179586;
  qn.eps = eps;
  qn.gain = gain;
  qn.pos_offset = pos_offset;
  qn.rstd = rstd;
  qn.rstd_stride = rstd_stride;
  if (sh.D == 64)
    return launch_fwd_kernel<64, true>(q, k, v, o, lse, nullptr, sh.B, sh.T, sh.T, sh.H, sh.KV, sh.window, sh.scale,
                                       q, qn, s);
  if (sh.D == 128)
    return launch_fwd_kernel<128, true>(q, k, v, o, lse, nullptr, sh.B, sh.T, sh.T, sh.H, sh.KV, sh.window,
                                        sh.scale, q, qn, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse, const AttnShape &sh,
                           hipStream_t s) {
  return launch_fwd_bf16_rows(q, k, v, o, lse, nullptr, sh.B, sh.T, sh.T, sh.H, sh.KV, sh.D, sh.window, sh.scale, s);
}

}  // namespace ncattn
