// Tile-level building blocks of the bf16 MFMA attention kernels (head_dim D =
// 64 or 128, a template parameter of every kernel).
//
// Data layout in LDS: a tile of 64 rows x D bf16 (2 D bytes per row) is stored
// with its 16-byte chunks permuted per row, chunk' = chunk ^ f(row).  Two read
// patterns hit such a tile and both are free of bank conflicts (64 banks of 4
// bytes, i.e. 256 bytes per bank row) under the permutation:
//   * straight 16-byte reads of one chunk column by 16 consecutive rows
//     (MFMA operands whose contraction index runs along the row), and
//   * 8-byte transposing reads (ds_read_b64_tr_b16) that gather 4 rows x 4
//     chunks per 32 lanes (MFMA operands whose contraction index runs down the
//     rows).
// D = 128 (256-byte rows, 16 chunks): f(row) = ((row & 3) << 2) | ((row >> 2) & 3),
// a bijection on the low 4 bits of the row, so 16 consecutive rows hit 16
// distinct chunk slots and rows r..r+3 hit disjoint groups of four.
// D = 64 (128-byte rows, 8 chunks, two rows per bank row): the bank slot of
// (row, chunk') is 8 (row & 1) + chunk'.  With m = (row >> 1) & 7,
// f(row) = ((m & 1) << 2) | (m >> 1) is a bijection on m (16 consecutive rows:
// distinct slots) and flips bit 2 between rows r and r + 2 for r = 0 mod 4
// (rows r..r+3 over four chunks of one half: distinct slots).
#pragma once

#include "device_common.hpp"

namespace ncattn {

constexpr int kTileN = 64;  // rows of a K/V (or Q/dO) tile

template <int D>
struct Geom {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static constexpr int kRowBytes = 2 * D;                 // one bf16 row of a tile
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
  static constexpr int kTileBytes = kTileN * kRowBytes;
  static constexpr int kSteps = D / 16;                   // MFMA k-steps over head_dim
  static constexpr int kDBlocks = D / 32;                 // 32-wide blocks of head_dim
  static constexpr int kCopyRows = 1024 / kRowBytes;      // rows one direct-copy instruction fills
};

template <int D>
__device__ __forceinline__ int swz_f(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else {
    const int m = (row >> 1) & 7;
    return ((m & 1) << 2) | (m >> 1);
  }
}

template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * Geom<D>::kRowBytes + ((chunk ^ swz_f<D>(row)) << 4);
}

// Direct global -> LDS copy of a 64 x D bf16 tile by the NW waves of a block,
// bypassing registers (buffer_load_dwordx4 ... lds: lane l of an instruction
// writes 16 bytes at the wave-uniform LDS base + 16 l, so one instruction fills
// kCopyRows = 1024 / (2 D) whole rows).  Instruction i of wave w fills tile rows
// kCopyRows (NW i + w) + [0, kCopyRows); lane l of it covers row
// kCopyRows (NW i + w) + l / kChunks at LDS chunk position l % kChunks, so it
// fetches global chunk (l % kChunks) ^ f(row) of that row (f depends only on
// row bits that do not change with i: a lane constant).  The source is a buffer
// resource over the `nrows` rows of one (batch, head) slice: the lane's part of
// the address is a constant VGPR and the tile's row offset a scalar, so a copy
// costs no vector ALU work, and rows at or past `nrows` fall outside the
// resource and arrive as zeros (finite data that every caller masks out or
// multiplies by 0).
typedef __attribute__((address_space(3))) void lds_void;

struct TileSrc {
  __amdgpu_buffer_rsrc_t rsrc;
  int stride;  // row stride in bytes
};

// rows [0, nrows) of a row-major slice starting at `base`, `row_stride_elems` bf16 apart
__device__ __forceinline__ TileSrc make_tile_src(const uint16_t *base, long long row_stride_elems, int nrows) {
  TileSrc s;
  s.stride = (int)(row_stride_elems * 2);
  s.rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, nrows * s.stride, 0x00020000);
  return s;
}

// lane constant: byte offset of this lane's 16-byte piece for instruction 0
template <int D>
__device__ __forceinline__ int tile_lane_voff(int row_stride_bytes, int tid) {
  using Gm = Geom<D>;
  const int lane = tid & 63, w = tid >> 6;
  const int lane_row = Gm::kCopyRows * w + lane / Gm::kChunks;
  return lane_row * row_stride_bytes + (((lane % Gm::kChunks) ^ swz_f<D>(lane_row)) << 4);
}

template <int D, int NW = 4, int ROWS = kTileN>
__device__ __forceinline__ void tile_load_lds(char *lds_tile, const TileSrc &src, int voff, int row0) {
  using Gm = Geom<D>;
  constexpr int kRowsPerRound = Gm::kCopyRows * NW;
  static_assert(ROWS % kRowsPerRound == 0, "whole copy rounds");
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < ROWS / kRowsPerRound; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.rsrc,
                                             (lds_void *)(lds_tile + (kRowsPerRound * i + Gm::kCopyRows * w) *
                                                                         Gm::kRowBytes),
                                             16, voff, (row0 + kRowsPerRound * i) * src.stride, 0, 0);
}

// Wait for this thread's direct-to-LDS loads, then a block barrier.
__device__ __forceinline__ void lds_loads_done_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
}

// Per-lane LDS offsets of the two operand patterns used on a 64 x D tile,
// computed once per kernel (row and chunk permutations are lane constants).
template <int D>
struct TileLane {
  int roff[Geom<D>::kSteps];       // row operand (rows l%32, chunk 2s + l/32); +32 rows = +32 kRowBytes
  int coff[Geom<D>::kDBlocks][2];  // transposed operand, d-block db, rows (16c + x) and (16c + x + 8)
};

template <int D>
__device__ __forceinline__ TileLane<D> make_tile_lane(int lane) {
  TileLane<D> L;
  const int h = lane >> 5;
#pragma unroll
  for (int s = 0; s < Geom<D>::kSteps; ++s) L.roff[s] = swz<D>(lane & 31, 2 * s + h);
  const int g = lane >> 4, r = lane & 15;
  const int x = 4 * (g >> 1) + (r >> 2);
#pragma unroll
  for (int db = 0; db < Geom<D>::kDBlocks; ++db) {
    const int d = 32 * db + ((g & 1) << 4) + 4 * (r & 3);
#pragma unroll
    for (int half = 0; half < 2; ++half) L.coff[db][half] = swz<D>(x + 8 * half, d >> 3) + (d & 7) * 2;
  }
  return L;
}

template <int D>
__device__ __forceinline__ bf16x8 col_operand(const char *t, const TileLane<D> &L, int db, int cs) {
  constexpr int kRowBytes = Geom<D>::kRowBytes;
  const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(t + L.coff[db][0] + cs * 16 * kRowBytes));
  const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(t + L.coff[db][1] + cs * 16 * kRowBytes));
  const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, w);
}

template <int D>
__device__ __forceinline__ bf16x8 row_operand(const char *t, const TileLane<D> &L, int s, int rowblk) {
  return *(const bf16x8 *)(t + L.roff[s] + rowblk * 32 * Geom<D>::kRowBytes);
}

// Operand of a 32x32x16 MFMA taken from a 32x32 fp32 accumulator block (rows =
// contraction index): step c2 (0 or 1) of the block uses rows {16c2 + 4h + k,
// 16c2 + 8 + 4h + k}, i.e. accumulator elements 8c2 + k and 8c2 + 4 + k of lane l.
__device__ __forceinline__ bf16x8 acc_to_operand(const f32x16 &acc, int c2) {
  const u32x4 w = {pack_bf16x2(acc[8 * c2 + 0], acc[8 * c2 + 1]), pack_bf16x2(acc[8 * c2 + 2], acc[8 * c2 + 3]),
                   pack_bf16x2(acc[8 * c2 + 4], acc[8 * c2 + 5]), pack_bf16x2(acc[8 * c2 + 6], acc[8 * c2 + 7])};
  return __builtin_bit_cast(bf16x8, w);
}

// The same operand as bf16 hi + lo: hi is each value rounded to bf16, lo the
// remainder rounded to bf16, so hi + lo carries the fp32 value to about 16
// significant bits (a contraction fed both loses only ~2^-16 relative).
__device__ __forceinline__ void acc_to_operand_split(const f32x16 &acc, int c2, bf16x8 &hi, bf16x8 &lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x0 = acc[8 * c2 + 2 * i], x1 = acc[8 * c2 + 2 * i + 1];
    h[i] = pack_bf16x2(x0, x1);
    l[i] = pack_bf16x2(x0 - __uint_as_float(h[i] << 16), x1 - __uint_as_float(h[i] & 0xffff0000u));
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

}  // namespace ncattn
