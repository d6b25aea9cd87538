// Tile-level building blocks of the bf16 MFMA attention kernels (head_dim 128).
//
// Data layout in LDS: a tile of 64 rows x 128 bf16 (256 B per row) is stored
// with its 16-byte chunks permuted per row, chunk' = chunk ^ f(row) with
// f(row) = ((row & 3) << 2) | ((row >> 2) & 3).  Two read patterns hit such a
// tile and both are free of bank conflicts under this permutation:
//   * straight 16-byte reads of one chunk column by 16 consecutive rows
//     (MFMA operands whose contraction index runs along the row), and
//   * 8-byte transposing reads (ds_read_b64_tr_b16) that gather 4 rows x 4
//     chunks per 16-lane group (MFMA operands whose contraction index runs
//     down the rows).
#pragma once

#include "device_common.hpp"

namespace ncattn {

constexpr int kD = 128;          // head_dim of the MFMA path
constexpr int kRowBytes = kD * 2;  // one bf16 row of a tile
constexpr int kTileN = 64;         // rows of a K/V (or Q/dO) tile
constexpr int kTileBytes = kTileN * kRowBytes;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (((row & 3) << 2) | ((row >> 2) & 3))) << 4);
}

__device__ __forceinline__ int swz_f(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Direct global -> LDS copy of a 64 x 128 bf16 tile (16 KB) by the NW waves of a
// block, bypassing registers (buffer_load_dwordx4 ... lds: lane l of an
// instruction writes 16 bytes at the wave-uniform LDS base + 16 l).  Instruction
// i of wave w fills tile rows 4 (NW i + w) + [0, 4); lane l of it covers row
// 4 (NW i + w) + l/16 at LDS chunk position l%16, so it fetches global chunk
// (l%16) ^ f(row) of that row (f depends on the row's low 4 bits only, a lane
// constant).  The source is a buffer resource over the `nrows` rows of one
// (batch, head) slice: the lane's part of the address is a constant VGPR and the
// tile's row offset a scalar, so a copy costs no vector ALU work, and rows at or
// past `nrows` fall outside the resource and arrive as zeros (finite data that
// every caller masks out or multiplies by 0).
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
__device__ __forceinline__ int tile_lane_voff(int row_stride_bytes, int tid) {
  const int lane = tid & 63, w = tid >> 6;
  const int lane_row = 4 * w + (lane >> 4);
  return lane_row * row_stride_bytes + (((lane & 15) ^ swz_f(lane_row)) << 4);
}

template <int NW = 4>
__device__ __forceinline__ void tile_load_lds(char *lds_tile, const TileSrc &src, int voff, int row0) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < 16 / NW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src.rsrc, (lds_void *)(lds_tile + (4 * NW * i + 4 * w) * kRowBytes), 16,
                                             voff, (row0 + 4 * NW * i) * src.stride, 0, 0);
}

// Wait for this thread's direct-to-LDS loads, then a block barrier.
__device__ __forceinline__ void lds_loads_done_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
}

// Per-lane LDS offsets of the two operand patterns used on a 64 x 128 tile,
// computed once per kernel (row and chunk permutations are lane constants).
struct TileLane {
  int roff[8];     // row operand (rows l%32, chunk 2s + l/32), s = 0..7; +32 rows = +8192 B
  int coff[4][2];  // transposed operand, d-block db, rows (16c + x) and (16c + x + 8); +16 rows = +4096 B
};

__device__ __forceinline__ TileLane make_tile_lane(int lane) {
  TileLane L;
  const int h = lane >> 5;
#pragma unroll
  for (int s = 0; s < 8; ++s) L.roff[s] = swz(lane & 31, 2 * s + h);
  const int g = lane >> 4, r = lane & 15;
  const int x = 4 * (g >> 1) + (r >> 2);
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = 32 * db + ((g & 1) << 4) + 4 * (r & 3);
#pragma unroll
    for (int half = 0; half < 2; ++half) L.coff[db][half] = swz(x + 8 * half, d >> 3) + (d & 7) * 2;
  }
  return L;
}

__device__ __forceinline__ bf16x8 col_operand(const char *t, const TileLane &L, int db, int cs) {
  const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr16(t + L.coff[db][0] + cs * 16 * kRowBytes));
  const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr16(t + L.coff[db][1] + cs * 16 * kRowBytes));
  const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ bf16x8 row_operand(const char *t, const TileLane &L, int s, int rowblk) {
  return *(const bf16x8 *)(t + L.roff[s] + rowblk * 32 * kRowBytes);
}

// Operand of a 32x32x16 MFMA taken from a 32x32 fp32 accumulator block (rows =
// contraction index): step c2 (0 or 1) of the block uses rows {16c2 + 4h + k,
// 16c2 + 8 + 4h + k}, i.e. accumulator elements 8c2 + k and 8c2 + 4 + k of lane l.
__device__ __forceinline__ bf16x8 acc_to_operand(const f32x16 &acc, int c2) {
  const u32x4 w = {pack_bf16x2(acc[8 * c2 + 0], acc[8 * c2 + 1]), pack_bf16x2(acc[8 * c2 + 2], acc[8 * c2 + 3]),
                   pack_bf16x2(acc[8 * c2 + 4], acc[8 * c2 + 5]), pack_bf16x2(acc[8 * c2 + 6], acc[8 * c2 + 7])};
  return __builtin_bit_cast(bf16x8, w);
}

}  // namespace ncattn
