// Host build of the kernels' register lookup (nf4_lut.h) for CPU tests: the
// byte-permute instruction is replaced by its documented byte-select model.
#include <stdint.h>

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
