// Matrix-core helpers for gfx950 (CDNA4).
//
// v_mfma_f32_16x16x32_bf16: D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).
// Operand layout used throughout (per 64-lane wave, lane = 16 * g + i):
//   A: lane holds 8 bf16 of row i, contraction slots 8g .. 8g+7;
//   B: lane holds 8 bf16 of column i, the same contraction slots 8g .. 8g+7;
//   D: lane holds D[4g + v][i], v = 0..3.
// Which physical contraction index a slot carries is up to the caller, as
// long as A and B agree, so the kernels may feed the 8 values of a lane in
// any fixed order.
#pragma once

#include "internal.h"

namespace qlora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// The same MFMA for either 16-bit compute type: bf16 (kF16 = false) or IEEE
// half (v_mfma_f32_16x16x32_f16), operand layout unchanged.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <bool kF16>
__device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
  if (kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  return mfma_16x16x32(a, b, c);
}

// Element 0 (low half) and 1 (high half) of a packed 16-bit pair as float32:
// exact for both types.
template <bool kF16>
__device__ __forceinline__ float lo16(uint32_t v) {
  if (kF16) return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v & 0xFFFFu)));
  return __uint_as_float(v << 16);
}
template <bool kF16>
__device__ __forceinline__ float hi16(uint32_t v) {
  if (kF16) return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(v >> 16)));
  return __uint_as_float(v & 0xFFFF0000u);
}
template <bool kF16>
__device__ __forceinline__ float to_f32(uint16_t v) {
  return lo16<kF16>(v);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// 8 bf16 from row_ptr[j0 .. j0+8) with zeros at and beyond `limit`; a 16-byte
// load when the run is whole and aligned.
__device__ __forceinline__ u32x4 ld8_bf16_guarded(const uint16_t* row_ptr, int j0, int limit, bool vec_ok) {
  if (j0 + 8 <= limit && vec_ok) return ld16(row_ptr + j0);
  uint32_t w[4] = {0, 0, 0, 0};
  for (int e = 0; e < 8; ++e) {
    if (j0 + e < limit) w[e >> 1] |= static_cast<uint32_t>(row_ptr[j0 + e]) << (16 * (e & 1));
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// 8 bf16 from row_ptr[j0 .. j0+8) where only indices in [0, limit) are read
// (the others are zeros); j0 may be negative. A 16-byte load when the run is
// whole and 16-byte aligned.
__device__ __forceinline__ u32x4 ld8_bf16_window(const uint16_t* row_ptr, int j0, int limit, bool row_aligned) {
  if (j0 >= 0 && j0 + 8 <= limit && row_aligned && (j0 & 7) == 0) return ld16(row_ptr + j0);
  uint32_t w[4] = {0, 0, 0, 0};
  for (int e = 0; e < 8; ++e) {
    const int j = j0 + e;
    if (j >= 0 && j < limit) w[e >> 1] |= static_cast<uint32_t>(row_ptr[j]) << (16 * (e & 1));
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// float32 -> the compute type, round to nearest even.
template <bool kF16>
__device__ __forceinline__ uint16_t to16(float f) {
  if (kF16) return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
  return f32_to_bf16_rne(f);
}

}  // namespace qlora
