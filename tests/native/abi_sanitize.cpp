// Host driver for the C ABI. api.cpp and codebook.cpp (all of the library's
// host logic) are built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host side and linked with the library's kernel objects.
//
// It walks every entry point's host logic: status strings, level tables,
// workspace sizes (including sizes whose products overflow 64 bits), argument
// validation, and then calls with valid arguments on real host buffers. It is
// run with no GPU visible, so those calls reach the first kernel launch, which
// fails, and the entry point must report QLORA_ERR_HIP. If a device is
// visible after all, that part is skipped: no kernel may run on host
// pointers. Prints "abi_sanitize: all checks passed" and exits 0, or names
// every failed check and exits 1.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "qlora_nf4.h"

static int g_failures = 0;

#define CHECK_EQ(expr, want)                                                                        \
  do {                                                                                              \
    const long long got_ = static_cast<long long>(expr);                                            \
    const long long want_ = static_cast<long long>(want);                                           \
    if (got_ != want_) {                                                                            \
      std::fprintf(stderr, "FAILED line %d: %s = %lld, expected %lld\n", __LINE__, #expr, got_, want_); \
      ++g_failures;                                                                                 \
    }                                                                                               \
  } while (0)

#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);         \
      ++g_failures;                                                          \
    }                                                                        \
  } while (0)

// 256-byte aligned, zero-filled host buffer, released at exit.
static std::vector<void*> g_bufs;
static void* buf(size_t bytes) {
  const size_t sz = ((bytes == 0 ? 1 : bytes) + 255) / 256 * 256;
  void* p = std::aligned_alloc(256, sz);
  std::memset(p, 0, sz);
  g_bufs.push_back(p);
  return p;
}

int main() {
  // --- status strings and level tables
  for (int st = 0; st >= -6; --st) CHECK(std::strlen(qlora_status_string(st)) > 0);
  CHECK(std::strlen(qlora_status_string(-77)) > 0);
  float lv[16];
  CHECK_EQ(qlora_nf4_levels(lv), 16);
  CHECK(lv[0] == -1.0f && lv[7] == 0.0f && lv[15] == 1.0f);
  for (int i = 1; i < 16; ++i) CHECK(lv[i - 1] < lv[i]);
  CHECK_EQ(qlora_codebook_levels(QLORA_CODEBOOK_INT4, lv), 16);
  CHECK(lv[0] == -1.0f && lv[15] == 1.0f);
  CHECK_EQ(qlora_codebook_levels(2, lv), QLORA_ERR_UNSUPPORTED);
  CHECK_EQ(qlora_nf4_levels(nullptr), QLORA_ERR_NULL);

  // --- workspace sizes: zero for no work or unsupported ranks, never a
  // wrapped-around value for huge sizes
  CHECK_EQ(qlora_linear_workspace_bytes(0, 4096, 4096, 16), 0);
  CHECK_EQ(qlora_linear_workspace_bytes(16, 4096, 4096, 200), 0);
  CHECK(qlora_linear_workspace_bytes(2048, 4096, 4096, 16) > 0);
  CHECK(qlora_linear_workspace_bytes(4096, 8192, 22016, 64) > qlora_linear_workspace_bytes(2048, 4096, 4096, 16));
  CHECK_EQ(qlora_linear_workspace_bytes(INT64_MAX, INT64_MAX, INT64_MAX, 64), 0);
  CHECK_EQ(qlora_linear_workspace_bytes(-1, 64, 64, 8), 0);
  CHECK_EQ(qlora_linear_dropout_workspace_bytes(INT64_MAX, 64, 64, 8), 0);
  CHECK_EQ(qlora_linear_grouped_workspace_bytes(64, 192, 128, 3, 8) > 0, 1);
  CHECK_EQ(qlora_linear_grouped_workspace_bytes(64, 192, 128, 9, 8), 0);
  CHECK_EQ(qlora_linear_grouped_workspace_bytes(INT64_MAX, 192, 128, 3, 8), 0);

  // --- one small layer on host buffers
  const int64_t m = 32, n = 512, k = 128;
  const int r = 16;
  const int64_t numel = n * k, nb = numel / QLORA_BLOCK, ng = (nb + QLORA_DQ_GROUP - 1) / QLORA_DQ_GROUP;
  float* w32 = static_cast<float*>(buf(numel * 4));
  uint8_t* codes = static_cast<uint8_t*>(buf(numel / 2));
  uint8_t* sc = static_cast<uint8_t*>(buf(nb));
  float* gs = static_cast<float*>(buf(ng * 4));
  float* am = static_cast<float*>(buf(nb * 4));
  uint16_t* x = static_cast<uint16_t*>(buf(m * k * 2));
  uint16_t* dy = static_cast<uint16_t*>(buf(m * n * 2));
  uint16_t* a = static_cast<uint16_t*>(buf(2 * r * k * 2));  // up to two stacked parts
  uint16_t* b = static_cast<uint16_t*>(buf(n * r * 2));
  uint16_t* y = static_cast<uint16_t*>(buf(m * n * 2));
  float* h = static_cast<float*>(buf(m * 2 * r * 4));
  uint16_t* dx = static_cast<uint16_t*>(buf(m * k * 2));
  float* da = static_cast<float*>(buf(2 * r * k * 4));
  float* db = static_cast<float*>(buf(n * r * 4));
  uint8_t* keep = static_cast<uint8_t*>(buf(m * k));
  float* merged = static_cast<float*>(buf(numel * 4));
  const size_t ws_bytes = qlora_linear_dropout_workspace_bytes(m, n, k, r) + qlora_linear_grouped_workspace_bytes(m, n, k, 2, r);
  void* ws = buf(ws_bytes);
  const qlora_nf4_weight w{n, k, codes, sc, gs, nullptr, 1, QLORA_CODEBOOK_NF4};
  const qlora_nf4_weight w_no_dq{n, k, codes, nullptr, nullptr, am, 0, QLORA_CODEBOOK_NF4};
  const int64_t parts2[2] = {256, 256};  // grouped parts: multiples of 256 rows
  hipStream_t s0 = nullptr;

  // --- validation before any launch
  CHECK_EQ(qlora_nf4_quantize(w32, numel, 3, codes, sc, gs, nullptr, s0), QLORA_ERR_UNSUPPORTED);
  CHECK_EQ(qlora_nf4_quantize(nullptr, numel, 1, codes, sc, gs, nullptr, s0), QLORA_ERR_NULL);
  CHECK_EQ(qlora_nf4_quantize(w32 + 1, numel, 1, codes, sc, gs, nullptr, s0), QLORA_ERR_ALIGN);
  CHECK_EQ(qlora_nf4_quantize(w32, -1, 1, codes, sc, gs, nullptr, s0), QLORA_ERR_SHAPE);
  CHECK_EQ(qlora_nf4_dequantize(&w, 9, y, s0), QLORA_ERR_UNSUPPORTED);
  CHECK_EQ(qlora_nf4_dequantize(nullptr, QLORA_BF16, y, s0), QLORA_ERR_NULL);
  CHECK_EQ(qlora_linear_fwd(&w, x, m, a, b, 200, 16.f, y, h, ws, ws_bytes, s0), QLORA_ERR_UNSUPPORTED);
  CHECK_EQ(qlora_linear_fwd(&w, x, m, a, b, r, 16.f, y, h, ws, 8, s0), QLORA_ERR_WORKSPACE);
  CHECK_EQ(qlora_linear_fwd(&w, x + 1, m, a, b, r, 16.f, y, h, ws, ws_bytes, s0), QLORA_ERR_ALIGN);
  CHECK_EQ(qlora_linear_fwd(&w, x, -m, a, b, r, 16.f, y, h, ws, ws_bytes, s0), QLORA_ERR_SHAPE);
  CHECK_EQ(qlora_linear_fwd(&w, x, 0, nullptr, nullptr, r, 16.f, nullptr, nullptr, nullptr, 0, s0), QLORA_OK);
  CHECK_EQ(qlora_linear_bwd(&w, x, nullptr, m, a, b, r, 16.f, h, dx, da, db, ws, ws_bytes, s0), QLORA_ERR_NULL);
  CHECK_EQ(qlora_linear_fwd_dropout(&w, x, m, a, b, r, 16.f, keep, 1.0f, y, h, ws, ws_bytes, s0),
           QLORA_ERR_UNSUPPORTED);
  CHECK_EQ(qlora_linear_fwd_dropout(&w, x, m, a, b, r, 16.f, keep, std::nanf(""), y, h, ws, ws_bytes, s0),
           QLORA_ERR_UNSUPPORTED);
  CHECK_EQ(qlora_dropout_mask(1, 8, 100, 0.1f, keep, s0), QLORA_ERR_SHAPE);
  const int64_t bad_parts[2] = {256, 128};
  CHECK_EQ(qlora_linear_fwd_grouped(&w, 2, bad_parts, x, m, a, b, r, 16.f, y, h, ws, ws_bytes, s0), QLORA_ERR_SHAPE);
  CHECK_EQ(qlora_linear_fwd_grouped(&w, 2, nullptr, x, m, a, b, r, 16.f, y, h, ws, ws_bytes, s0), QLORA_ERR_NULL);
  CHECK_EQ(qlora_linear_fwd_noalloc(&w, x, int64_t(1) << 40, a, b, r, 16.f, y, h, s0), QLORA_ERR_SHAPE);
  CHECK_EQ(qlora_unmerge(merged, QLORA_F32, n, k, a, b, r, 16.f, nullptr, s0), QLORA_ERR_NULL);

  // --- valid calls: the first launch fails, reported as QLORA_ERR_HIP
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    std::printf("abi_sanitize: %d device(s) visible, launch-failure checks skipped\n", ndev);
    for (void* p : g_bufs) std::free(p);
    if (g_failures != 0) {
      std::fprintf(stderr, "abi_sanitize: %d check(s) failed\n", g_failures);
      return 1;
    }
    std::printf("abi_sanitize: all checks passed\n");
    return 0;
  }
  CHECK_EQ(qlora_nf4_quantize(w32, numel, 1, codes, sc, gs, nullptr, s0), QLORA_ERR_HIP);
  CHECK_EQ(qlora_quantize_codebook(w32, numel, 0, QLORA_CODEBOOK_INT4, codes, nullptr, nullptr, am, s0),
           QLORA_ERR_HIP);
  CHECK_EQ(qlora_nf4_dequantize(&w, QLORA_BF16, y, s0), QLORA_ERR_HIP);
  CHECK_EQ(qlora_nf4_dequantize(&w_no_dq, QLORA_F32, merged, s0), QLORA_ERR_HIP);
  for (int64_t mm : {int64_t(1), int64_t(2), int64_t(5), m}) {
    CHECK_EQ(qlora_linear_fwd(&w, x, mm, a, b, r, 16.f, y, h, ws, ws_bytes, s0), QLORA_ERR_HIP);
    CHECK_EQ(qlora_linear_fwd_f16(&w, x, mm, a, b, r, 16.f, y, h, ws, ws_bytes, s0), QLORA_ERR_HIP);
    CHECK_EQ(qlora_linear_bwd(&w, x, dy, mm, a, b, r, 16.f, h, dx, da, db, ws, ws_bytes, s0), QLORA_ERR_HIP);
    CHECK_EQ(qlora_linear_bwd_f16(&w, x, dy, mm, a, b, r, 16.f, nullptr, dx, da, db, ws, ws_bytes, s0),
             QLORA_ERR_HIP);
  }
  CHECK_EQ(qlora_linear_fwd(&w, x, m, nullptr, nullptr, 0, 0.f, y, nullptr, ws, ws_bytes, s0), QLORA_ERR_HIP);
  CHECK_EQ(qlora_linear_fwd_noalloc(&w, x, m, a, b, r, 16.f, y, h, s0), QLORA_ERR_HIP);
  CHECK_EQ(qlora_linear_fwd_grouped(&w, 2, parts2, x, m, a, b, r, 16.f, y, h, ws, ws_bytes, s0), QLORA_ERR_HIP);
  CHECK_EQ(qlora_linear_bwd_grouped(&w, 2, parts2, x, dy, m, a, b, r, 16.f, h, dx, da, db, ws, ws_bytes, s0),
           QLORA_ERR_HIP);
  CHECK_EQ(qlora_linear_fwd_grouped(&w, 2, parts2, x, 1, a, b, r, 16.f, y, h, ws, ws_bytes, s0), QLORA_ERR_HIP);
  CHECK_EQ(qlora_dropout_mask(7, 0, m * k, 0.1f, keep, s0), QLORA_ERR_HIP);
  CHECK_EQ(qlora_linear_fwd_dropout(&w, x, m, a, b, r, 16.f, keep, 0.1f, y, h, ws, ws_bytes, s0), QLORA_ERR_HIP);
  CHECK_EQ(qlora_linear_bwd_dropout(&w, x, dy, m, a, b, r, 16.f, keep, 0.1f, h, dx, da, db, ws, ws_bytes, s0),
           QLORA_ERR_HIP);
  CHECK_EQ(qlora_merge(&w, a, b, r, 16.f, QLORA_BF16, y, s0), QLORA_ERR_HIP);
  CHECK_EQ(qlora_unmerge(merged, QLORA_F32, n, k, a, b, r, 16.f, merged, s0), QLORA_ERR_HIP);
  CHECK_EQ(qlora_requantize(&w, a, b, r, 16.f, 1, QLORA_CODEBOOK_NF4, merged, codes, sc, gs, nullptr, s0),
           QLORA_ERR_HIP);

  for (void* p : g_bufs) std::free(p);
  if (g_failures != 0) {
    std::fprintf(stderr, "abi_sanitize: %d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("abi_sanitize: all checks passed\n");
  return 0;
}
