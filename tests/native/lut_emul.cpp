// Host build of the kernels' register lookup (nf4_lut.h) and of the quantize
// kernel's per-weight encoding for CPU tests: the byte-permute instruction is
// replaced by its documented byte-select model. Built together with
// codebook.cpp (the level and bucket tables), without FMA contraction.
#include <math.h>
#include <stdint.h>

#include "internal.h"
#include "nf4_lut.h"

extern "C" int lut_emul(const float* levels, float scale, const uint32_t* words, int nwords, uint32_t* decode_out,
                        uint32_t* natural_out) {
  const qlora::BlockLut t = qlora::make_block_lut(levels, scale);
  for (int i = 0; i < nwords; ++i) {
    qlora::lut8_decode_order(t, words[i], decode_out + 4 * i);
    qlora::lut8_natural_order(t, words[i], natural_out + 4 * i);
  }
  return 0;
}

extern "C" int decode_order_emul(const uint32_t* in, int n, uint32_t* out) {
  for (int i = 0; i < n; ++i) qlora::to_decode_order(in + 4 * i, out + 4 * i);
  return 0;
}

extern "C" int u8_unit_emul(float* out) {
  for (uint32_t k = 0; k < 256; ++k) out[k] = qlora::u8_unit(k);
  return 256;
}

extern "C" int e4m4_unit_emul(float* out) {
  for (uint32_t c = 0; c < 256; ++c) out[c] = qlora::e4m4_unit(c);
  return 256;
}

// Host model of the quantize kernel's per-weight encoding (nf4_lut.h's
// quotient16 and encode_bucket with the bucket table of internal.h):
// absmax per block of 64, t = 16 w / absmax by the same path selection as the
// kernel, code from the table. Codes are written one per byte.
extern "C" int quant_codes_emul(const float* w, int64_t numel, int codebook, uint8_t* codes_out,
                                float* absmax_out) {
  const qlora::EncodeTable& E = qlora::encode_table(codebook);
  for (int64_t b0 = 0; b0 < numel; b0 += 64) {
    const int64_t n = numel - b0 < 64 ? numel - b0 : 64;
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) m = fmaxf(m, fabsf(w[b0 + i]));
    absmax_out[b0 / 64] = m;
    const bool fast = m >= 0x1p-60f && m <= 0x1p60f;
    const float y16 = fast ? 16.0f / m : 0.0f, m16 = m * 0.0625f;
    const float mm = m > 0.0f ? m : 1.0f;
    for (int64_t i = 0; i < n; ++i) {
      const float v = w[b0 + i];
      const float t = fast ? qlora::quotient16(v, y16, m16) : 16.0f * (v / mm);
      const int b = qlora::encode_bucket(t);
      codes_out[b0 + i] = static_cast<uint8_t>(E.base[b] + (t >= E.thr16[b] ? 1u : 0u));
    }
  }
  return 0;
}

// The bucket table itself, for checks of its construction.
extern "C" int encode_table_emul(int codebook, float* thr16_out, uint32_t* base_out) {
  const qlora::EncodeTable& E = qlora::encode_table(codebook);
  for (int b = 0; b < 33; ++b) {
    thr16_out[b] = E.thr16[b];
    base_out[b] = E.base[b];
  }
  return 33;
}

// quotient16 against 16 times the float32 quotient v / m: `samples` random
// pairs (m in [2^-60, 2^60], |v| <= m, |v| >= 2^-100, significands often all
// ones or all zeros) plus, for every significand of m in [1, 2), four
// numerators in [m / 2, m]. Returns the number of mismatches.
extern "C" int64_t quotient16_check(int64_t samples, uint64_t seed) {
  auto next = [&seed]() {
    uint64_t z = (seed += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  };
  auto mk = [](uint32_t bits) {
    float f;
    __builtin_memcpy(&f, &bits, 4);
    return f;
  };
  auto same = [](float a, float b) { return qlora::f32_bits(a) == qlora::f32_bits(b); };
  int64_t bad = 0;
  for (int64_t i = 0; i < samples; ++i) {
    const uint64_t a = next(), b = next();
    const int em = static_cast<int>(a % 121) - 60;
    uint32_t mm = static_cast<uint32_t>(a >> 8) & 0x7FFFFF;
    if ((a >> 40) % 16 == 0) mm = 0x7FFFFF;
    if ((a >> 44) % 16 == 1) mm = 0;
    const float m = mk((static_cast<uint32_t>(em + 127) << 23) | mm);
    const int ev = em - static_cast<int>((b >> 50) % 42);
    if (ev < -100) continue;
    uint32_t vm = static_cast<uint32_t>(b) & 0x7FFFFF;
    if ((b >> 24) % 16 == 0) vm = 0x7FFFFF;
    float v = mk((static_cast<uint32_t>(ev + 127) << 23) | vm);
    v = v > m ? m : v;
    v = (b >> 63) ? -v : v;
    if (!same(qlora::quotient16(v, 16.0f / m, m * 0.0625f), 16.0f * (v / m))) ++bad;
  }
  for (uint32_t mm = 0; mm < (1u << 23); ++mm) {
    const float m = mk((127u << 23) | mm);
    const float y16 = 16.0f / m, m16 = m * 0.0625f;
    for (uint32_t j = 0; j < 4; ++j) {
      const uint32_t vm = j == 0 ? 0x7FFFFFu : (j == 1 ? 0u : static_cast<uint32_t>(next()) & 0x7FFFFF);
      float v = mk(((j & 1) ? 126u << 23 : 127u << 23) | vm);
      v = v > m ? m : v;
      if (!same(qlora::quotient16(v, y16, m16), 16.0f * (v / m))) ++bad;
    }
  }
  return bad;
}
