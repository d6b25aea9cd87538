// Device-side helpers shared by the gfx950 kernels: vector types for the MFMA
// builtins, bf16 <-> f32 conversion, lane exchange, and the launch-config
// helpers.  Nothing here encodes the attention method itself.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ncattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Two floats -> two bf16 (round to nearest even) packed in one dword, low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Lane exchange within the wave (ds_bpermute based).
__device__ __forceinline__ float shfl_xor(float x, int mask) { return __shfl_xor(x, mask, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// MFMA wrappers (gfx950).  32x32x16: A lane l holds row l%32, k = (l/32)*8 + [0,8);
// B lane l holds col l%32, same k; C lane l holds col l%32, rows 8i + 4(l/32) + j
// at element 4i + j.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS transposing read of four 16-bit elements.  Within each group of 16 lanes,
// the 16 source vectors (4 elements each, read at every lane's own address) form a
// 16 x 4 matrix M; lane i receives M[i/4 + 4k][i%4] for k = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const void *lds_ptr) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(lds_ptr));
}

template <typename T>
__device__ __forceinline__ T ldg(const T *p) { return __builtin_nontemporal_load(p); }

}  // namespace ncattn

namespace ncattn {

// Sum over each row of 16 lanes with DPP moves (every lane of the row receives
// the total): xor-1 and xor-2 quad permutes, then half-row and row mirrors.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, true));  // row_mirror
  return x;
}

}  // namespace ncattn
