// Register-resident NF4 -> bf16 lookup for one 64-weight block.
//
// For a block with decoded scale s, the 16 possible dequantized weights are
// T[c] = bf16_rne(fl32(L[c] * s)) (Ultralytics glossary "QLoRA", "Come
// funziona QLoRA": restore = level[code] * scale, taken to bfloat16 before the
// matmul). T is kept as two 16-byte tables -- low bytes and high bytes of the
// bf16 values -- and a code is looked up with the byte-permute instruction
// (v_perm_b32), which picks bytes out of an 8-byte register pair by 8-bit
// selectors: selector 0..7 returns that byte, any selector >= 13 returns 0xFF.
// A 16-entry table needs two such 8-byte halves; a code c < 8 selects byte c
// of the low half while the high-half selector is pushed to >= 24 (0xFF), and
// vice versa for c >= 8, so AND-ing the two results gives T[c]. Four codes are
// looked up per instruction, so 8 weights cost 25 VALU ops in decode order.
//
// The same functions compile for the host (with a byte-permute model) so the
// bit manipulation is unit-tested on the CPU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

__host__ __device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_perm(hi, lo, sel);
#else
  const uint64_t data = (uint64_t(hi) << 32) | lo;
  uint32_t out = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t s = (sel >> (8 * i)) & 0xFF;
    uint32_t byte;
    if (s >= 13) {
      byte = 0xFF;
    } else if (s == 12) {
      byte = 0x00;
    } else if (s >= 8) {
      byte = ((data >> (16 * (s - 8) + 15)) & 1) ? 0xFF : 0x00;  // sign of byte 1,3,5,7
    } else {
      byte = (data >> (8 * s)) & 0xFF;
    }
    out |= byte << (8 * i);
  }
  return out;
#endif
}

__host__ __device__ __forceinline__ uint32_t f32_bits(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __float_as_uint(f);
#else
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  return u;
#endif
}

// bf16 round-to-nearest-even of a finite float, returned in the HIGH half of
// a 32-bit word (low half is garbage).
__host__ __device__ __forceinline__ uint32_t bf16_rne_hi(float f) {
  const uint32_t u = f32_bits(f);
  return u + 0x7FFFu + ((u >> 16) & 1u);
}

// Pack two floats (RNE) into one dword of two bf16: lo element in bits 0..15.
__host__ __device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (bf16_rne_hi(lo) >> 16) | (bf16_rne_hi(hi) & 0xFFFF0000u);
}

// Same rounding through the gfx950 packed convert (v_cvt_pk_bf16_f32, round to
// nearest even). Used for the lookup tables of the matmul kernels; the
// bit-exact dequantize kernel keeps the integer form above.
__host__ __device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
#else
  return pack_bf16x2(lo, hi);
#endif
}

// The same pair conversion into either 16-bit compute type: bf16 (kF16 =
// false) or IEEE half (v_cvt_pk_f16_f32, round to nearest even). The host
// build models the bf16 form only.
template <bool kF16>
__host__ __device__ __forceinline__ uint32_t cvt_16x2(float lo, float hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (kF16) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const f2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
  }
#endif
  return cvt_bf16x2(lo, hi);
}

// fl32(k / 255) for an 8-bit scale code k, the double-quantization level
// (Ultralytics glossary "QLoRA", "Come funziona QLoRA": the block scales are
// themselves stored as 8-bit codes). One multiply by fl32(1/255) and one FMA
// correction with the exact residual k - 255 q0 give the correctly rounded
// quotient for every k in 0..255 (checked exhaustively on the host), at 3
// instructions instead of a full IEEE division.
__host__ __device__ __forceinline__ float u8_unit(uint32_t k) {
  const float kf = static_cast<float>(k);
  const float c = 1.0f / 255.0f;
  const float q0 = kf * c;
  const float r = fmaf(-q0, 255.0f, kf);
  return fmaf(r, c, q0);
}

// t = 16 fl32(v / m) for |v| <= m, m in [2^-60, 2^60], |v| >= 2^-100 (the
// quantizer's x = w / absmax, scaled for the bucket lookup), from y16 =
// fl32(16 / m) = 16 fl32(1 / m) and m16 = m / 16, both exact scalings of
// per-block values. q = v y is within one unit in the last place of v / m,
// the residual v - q m is exact in an FMA, and one correction q + r y rounds
// to the correctly rounded quotient (Markstein's theorem on division with a
// correctly rounded reciprocal); all three steps carry the factor 16
// exactly. Checked on the host against float32 division on 1.6e10 random
// pairs and on every significand of m. For |v| < 2^-100 the result stays
// within 2^-35 of 16 v / m, far from every switch point of the codebooks.
__host__ __device__ __forceinline__ float quotient16(float v, float y16, float m16) {
  const float q16 = v * y16;
  const float r = fmaf(-q16, m16, v);
  return fmaf(r, y16, q16);
}

// Code of x from t = 16 x (|t| <= 16) with the bucket table of the codebook
// (EncodeTable in internal.h): thr16 and base of bucket floor(t) + 16.
__host__ __device__ __forceinline__ int encode_bucket(float t16) {
  int b = static_cast<int>(floorf(t16)) + 16;
  b = b < 0 ? 0 : b;
  return b > 32 ? 32 : b;
}

// E_c of the float-like 8-bit scale code (double_quant = 2): c = 16 e + m,
// E = m 2^-18 for e = 0 and (16 + m) 2^(e - 19) = (1 + m/16) 2^(e - 15)
// otherwise, built exactly from its float32 bits (exponent field e + 112,
// top mantissa bits m). Code 240 is exactly 1.
__host__ __device__ __forceinline__ float e4m4_unit(uint32_t c) {
  const uint32_t e = c >> 4, m = c & 15u;
  const uint32_t bits = ((e + 112u) << 23) | (m << 19);
  float nrm;
#if defined(__HIP_DEVICE_COMPILE__)
  nrm = __uint_as_float(bits);
#else
  __builtin_memcpy(&nrm, &bits, 4);
#endif
  return e == 0 ? static_cast<float>(m) * 3.814697265625e-06f : nrm;  // 2^-18
}

// The scale unit of a double-quantization mode: 2 the float-like code,
// otherwise (1) the linear k / 255.
__host__ __device__ __forceinline__ float dq_unit(uint32_t c, int mode) {
  return mode == 2 ? e4m4_unit(c) : u8_unit(c);
}

struct BlockLut {
  uint32_t tl[4];  // low bytes of T[0..15], 4 per dword
  uint32_t th[4];  // high bytes of T[0..15]
};

// Build the tables for scale s. L holds the 16 float32 levels. kF16 selects
// half-precision entries (fp16 compute) instead of bf16; the lookup below
// only moves bytes, so it serves both.
template <bool kF16 = false>
__host__ __device__ __forceinline__ BlockLut make_block_lut(const float* L, float s) {
  uint32_t p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = cvt_16x2<kF16>(L[2 * j] * s, L[2 * j + 1] * s);
  BlockLut t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t.tl[q] = byte_perm(p[2 * q + 1], p[2 * q], 0x06040200u);
    t.th[q] = byte_perm(p[2 * q + 1], p[2 * q], 0x07050301u);
  }
  return t;
}

// Look up 8 codes held in one dword (element 2i in the low nibble of byte i,
// element 2i+1 in the high nibble). Returns four dwords of bf16 pairs in
// decode order: (e0,e2), (e4,e6), (e1,e3), (e5,e7).
__host__ __device__ __forceinline__ void lut8_decode_order(const BlockLut& t, uint32_t c, uint32_t out[4]) {
  const uint32_t se = (c & 0x0F0F0F0Fu) | ((c << 1) & 0x10101010u);
  const uint32_t so = ((c >> 4) & 0x0F0F0F0Fu) | ((c >> 3) & 0x10101010u);
  const uint32_t se2 = se ^ 0x18181818u, so2 = so ^ 0x18181818u;
  const uint32_t le = byte_perm(t.tl[1], t.tl[0], se) & byte_perm(t.tl[3], t.tl[2], se2);
  const uint32_t he = byte_perm(t.th[1], t.th[0], se) & byte_perm(t.th[3], t.th[2], se2);
  const uint32_t lo = byte_perm(t.tl[1], t.tl[0], so) & byte_perm(t.tl[3], t.tl[2], so2);
  const uint32_t ho = byte_perm(t.th[1], t.th[0], so) & byte_perm(t.th[3], t.th[2], so2);
  out[0] = byte_perm(he, le, 0x05010400u);
  out[1] = byte_perm(he, le, 0x07030602u);
  out[2] = byte_perm(ho, lo, 0x05010400u);
  out[3] = byte_perm(ho, lo, 0x07030602u);
}

// Same lookup, natural order: (e0,e1), (e2,e3), (e4,e5), (e6,e7). The
// nibbles are first spread into selector bytes in element order (bytes i and
// i + 1 of c interleaved with those of c >> 4, low nibble of each byte taken),
// so the pairs come out without a second reordering pass: 27 operations per
// 8 weights against 29 for the decode-order lookup plus 4 byte permutes.
__host__ __device__ __forceinline__ void lut8_natural_order(const BlockLut& t, uint32_t c, uint32_t out[4]) {
  const uint32_t c4 = c >> 4;
  const uint32_t n0 = byte_perm(c4, c, 0x05010400u);  // e0 e1 e2 e3 in the low nibbles
  const uint32_t n1 = byte_perm(c4, c, 0x07030602u);  // e4 e5 e6 e7
  const uint32_t s0 = (n0 & 0x0F0F0F0Fu) | ((n0 << 1) & 0x10101010u);
  const uint32_t s1 = (n1 & 0x0F0F0F0Fu) | ((n1 << 1) & 0x10101010u);
  const uint32_t s0b = s0 ^ 0x18181818u, s1b = s1 ^ 0x18181818u;
  const uint32_t l0 = byte_perm(t.tl[1], t.tl[0], s0) & byte_perm(t.tl[3], t.tl[2], s0b);
  const uint32_t h0 = byte_perm(t.th[1], t.th[0], s0) & byte_perm(t.th[3], t.th[2], s0b);
  const uint32_t l1 = byte_perm(t.tl[1], t.tl[0], s1) & byte_perm(t.tl[3], t.tl[2], s1b);
  const uint32_t h1 = byte_perm(t.th[1], t.th[0], s1) & byte_perm(t.th[3], t.th[2], s1b);
  out[0] = byte_perm(h0, l0, 0x05010400u);
  out[1] = byte_perm(h0, l0, 0x07030602u);
  out[2] = byte_perm(h1, l1, 0x05010400u);
  out[3] = byte_perm(h1, l1, 0x07030602u);
}

// Decode order of 8 consecutive bf16 values held as 4 dwords (x0x1, x2x3,
// x4x5, x6x7) -> (x0x2, x4x6, x1x3, x5x7), to match lut8_decode_order.
__host__ __device__ __forceinline__ void to_decode_order(const uint32_t in[4], uint32_t out[4]) {
  out[0] = byte_perm(in[1], in[0], 0x05040100u);
  out[1] = byte_perm(in[3], in[2], 0x05040100u);
  out[2] = byte_perm(in[1], in[0], 0x07060302u);
  out[3] = byte_perm(in[3], in[2], 0x07060302u);
}

}  // namespace qlora
