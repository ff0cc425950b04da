// Matrix-core building blocks shared by the decode kernel and the row-state kernels: the
// 16x16x32 MFMA on 16-bit operands, the swizzled LDS layouts of key rows (read back as score
// operands) and value rows (read back transposed), and the split of fp32 probabilities into
// two 16-bit operands.
#pragma once

#include "device_common.h"

namespace pkv {

template <typename T>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (__is_same(T, bf16_t)) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Swizzle of the 32-byte pieces of value row t in the LDS tile (D / 16 pieces per row): the 16
// rows one transposed read touches (t = 8q + 4h + 0..3, q = 0..3) land on distinct piece
// positions in every 256-byte bank window.
template <int D>
__device__ __forceinline__ int piece_swizzle(int t) {
  if constexpr (D == 128) return (t & 3) | (((t >> 3) & 1) << 2);
  else return ((t >> 1) & 1) | (((t >> 3) & 1) << 1);
}

// Position of 16-byte piece c of key row t in an LDS key tile: pieces XOR-swizzled per row so
// that the 16 rows one score-operand read touches (t = 8q + 4a + 0..3, q = 0..3) fall on
// distinct banks, and the 16 pieces of one row written by 16 lanes stay distinct.
template <int D>
__device__ __forceinline__ int key_piece(int t, int c) {
  if constexpr (D == 128) return c ^ ((t & 3) | (((t >> 3) & 3) << 2));
  else return c ^ (((t >> 1) & 1) | (((t >> 3) & 3) << 1));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Four 16-bit elements, transposed across each 16-lane group (ds_read_b64_tr_b16).
__device__ __forceinline__ uint2 lds_read_tr16(const char* lds_byte_addr) {
  const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)(__attribute__((address_space(3))) char*)lds_byte_addr);
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Split two fp32 probabilities into packed 16-bit high parts and remainders.
template <typename T>
__device__ __forceinline__ void split_pair(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  uint16_t h0 = Elem<T>::from_f32(p0), h1 = Elem<T>::from_f32(p1);
  float r0 = p0 - Elem<T>::to_f32(h0), r1 = p1 - Elem<T>::to_f32(h1);
  hi = (uint32_t)h0 | ((uint32_t)h1 << 16);
  lo = (uint32_t)Elem<T>::from_f32(r0) | ((uint32_t)Elem<T>::from_f32(r1) << 16);
}

}  // namespace pkv
