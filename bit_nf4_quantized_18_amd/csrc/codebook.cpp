// NF4 level table, built once on the host.
//
// Ultralytics glossary "QLoRA", section "Come funziona QLoRA": 16 levels at
// quantiles of the standard normal with an exact zero, normalised to [-1, 1];
// the printed example takes 8 probabilities evenly spaced from 0.9677083 down
// to 0.5 (0.5 excluded) for the positive side, 7 for the negative side.
//
// The quantile is found by bisection on the normal CDF written with erfc in
// long double, independently of any published inverse-CDF approximation. The
// bracket is halved 200 times, far below the float64 resolution of the result;
// each level is divided by the largest in double and rounded once to float.
#include <cmath>
#include <cstring>
#include <limits>
#include <mutex>

#include "internal.h"

namespace qlora {
namespace {

long double normal_cdf(long double x) { return 0.5L * std::erfc(-x / std::sqrt(2.0L)); }

double normal_quantile_upper(double p) {  // p in [0.5, 1)
  long double lo = 0.0L, hi = 40.0L;
  for (int i = 0; i < 200; ++i) {
    const long double mid = 0.5L * (lo + hi);
    if (normal_cdf(mid) < static_cast<long double>(p)) {
      lo = mid;
    } else {
      hi = mid;
    }
  }
  return static_cast<double>(0.5L * (lo + hi));
}

Levels build_levels() {
  const double offset = 0.9677083;
  double v[16];
  int n = 0;
  // Evenly spaced probabilities from the offset to 0.5, endpoint dropped:
  // start + i * ((0.5 - start) / (count - 1)), as a float64 linspace does.
  const double step_pos = (0.5 - offset) / 8.0;
  const double step_neg = (0.5 - offset) / 7.0;
  for (int j = 0; j < 7; ++j) v[n++] = -normal_quantile_upper(static_cast<double>(j) * step_neg + offset);
  v[n++] = 0.0;
  for (int i = 0; i < 8; ++i) v[n++] = normal_quantile_upper(static_cast<double>(i) * step_pos + offset);
  // ascending: negatives were produced from most negative (j = 0) upward,
  // positives from largest (i = 0) downward; reverse the positive run.
  for (int a = 8, b = 15; a < b; ++a, --b) {
    const double t = v[a];
    v[a] = v[b];
    v[b] = t;
  }
  const double top = v[15];
  Levels L;
  for (int c = 0; c < 16; ++c) L.v[c] = static_cast<float>(v[c] / top);
  return L;
}

// numpy's float64 linspace(-1, 1, 16): k * (2 / 15) - 1, the last value
// exactly 1, each rounded once to float32.
Levels build_int4() {
  Levels L;
  const double step = 2.0 / 15.0;
  for (int c = 0; c < 15; ++c) L.v[c] = static_cast<float>(static_cast<double>(c) * step + -1.0);
  L.v[15] = 1.0f;
  return L;
}

}  // namespace

const Levels& codebook_table(int codebook) {
  if (codebook == QLORA_CODEBOOK_INT4) {
    static std::once_flag once;
    static Levels table;
    std::call_once(once, [] { table = build_int4(); });
    return table;
  }
  return nf4_table();
}

const Levels& nf4_table() {
  static std::once_flag once;
  static Levels table;
  std::call_once(once, [] { table = build_levels(); });
  return table;
}

namespace {

// Total order of floats as integers (-0 and +0 both map to 0).
int64_t float_key(float f) {
  uint32_t b;
  std::memcpy(&b, &f, 4);
  const int64_t mag = static_cast<int64_t>(b & 0x7FFFFFFFu);
  return (b & 0x80000000u) ? -mag : mag;
}

float key_float(int64_t key) {
  const uint32_t b = key < 0 ? (0x80000000u | static_cast<uint32_t>(-key)) : static_cast<uint32_t>(key);
  float f;
  std::memcpy(&f, &b, 4);
  return f;
}

// The nearest-level rule between lo < hi in float32: true when hi is nearer
// (ties keep lo). volatile keeps each difference a float32 result.
bool hi_nearer(float x, float lo, float hi) {
  volatile float d_lo = x - lo;
  volatile float d_hi = hi - x;
  return d_hi < d_lo;
}

// The smallest float x in (lo, hi] for which hi is nearer: the rule is false
// at lo and true at hi, and monotone in between, so bisection over the
// floats' order finds the switch point exactly.
float switch_point(float lo, float hi) {
  int64_t a = float_key(lo), b = float_key(hi);
  while (b - a > 1) {
    const int64_t mid = a + (b - a) / 2;
    if (hi_nearer(key_float(mid), lo, hi)) {
      b = mid;
    } else {
      a = mid;
    }
  }
  return key_float(b);
}

EncodeTable build_encode(const Levels& L) {
  float u16[15];
  for (int k = 0; k < 15; ++k) u16[k] = 16.0f * switch_point(L.v[k], L.v[k + 1]);  // exact scaling
  EncodeTable E;
  for (int b = 0; b <= 32; ++b) {
    const float lo = static_cast<float>(b - 16), hi = lo + 1.0f;
    uint32_t base = 0;
    float thr = std::numeric_limits<float>::infinity();
    for (int k = 0; k < 15; ++k) {
      if (u16[k] <= lo) {
        ++base;
      } else if (u16[k] < hi) {
        thr = u16[k];  // at most one per bucket (switch points are > 1 apart in t)
      }
    }
    E.thr16[b] = thr;
    E.base[b] = base;
  }
  return E;
}

}  // namespace

const EncodeTable& encode_table(int codebook) {
  if (codebook == QLORA_CODEBOOK_INT4) {
    static std::once_flag once;
    static EncodeTable table;
    std::call_once(once, [] { table = build_encode(codebook_table(QLORA_CODEBOOK_INT4)); });
    return table;
  }
  static std::once_flag once;
  static EncodeTable table;
  std::call_once(once, [] { table = build_encode(nf4_table()); });
  return table;
}

}  // namespace qlora

extern "C" int qlora_nf4_levels(float out16[16]) {
  if (out16 == nullptr) return QLORA_ERR_NULL;
  const qlora::Levels& L = qlora::nf4_table();
  for (int c = 0; c < 16; ++c) out16[c] = L.v[c];
  return 16;
}

extern "C" int qlora_codebook_levels(int codebook, float out16[16]) {
  if (out16 == nullptr) return QLORA_ERR_NULL;
  if (codebook != QLORA_CODEBOOK_NF4 && codebook != QLORA_CODEBOOK_INT4) return QLORA_ERR_UNSUPPORTED;
  const qlora::Levels& L = qlora::codebook_table(codebook);
  for (int c = 0; c < 16; ++c) out16[c] = L.v[c];
  return 16;
}
