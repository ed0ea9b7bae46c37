// C ABI: argument validation, workspace layout and kernel dispatch.
#include <stddef.h>
#include <stdint.h>

#include "internal.h"

namespace {

using qlora::PackedW;

constexpr int64_t kAlign = 256;  // workspace sub-buffer alignment (bytes)
constexpr int64_t kGemvMaxM = 16;

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }
int rank_pad(int r) { return r == 0 ? 0 : static_cast<int>(round_up(r, 32)); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workspace layout: consecutive 256-byte aligned sub-buffers.
struct Carve {
  int64_t off = 0;
  int64_t take(int64_t bytes) {
    const int64_t at = off;
    off += round_up(bytes, kAlign);
    return at;
  }
};

struct FwdLayout {
  int64_t h32, hs, part, total;
};
// gemm: the fused GEMM for every m (dropout calls)
FwdLayout fwd_layout(int64_t m, int64_t n, int64_t k, int r, bool gemm = false) {
  (void)n;
  Carve c;
  FwdLayout L{};
  if (m <= kGemvMaxM && !gemm) {
    // decode: H partial sums, unless the GEMV computes H itself (a grouped
    // call fuses whenever the ungrouped rule does)
    L.h32 = c.take(r == 0 || qlora::gemv_fuses_h(m, k, r, nullptr) ? 0 : qlora::skinny_splits(m, k) * m * r * 4);
    L.hs = c.take(0);
  } else {
    L.h32 = c.take(m * r * 4);
    L.hs = c.take(m * rank_pad(r) * 2);
    L.part = c.take(static_cast<int64_t>(qlora::skinny_prefill_splits(m, k, r)) * m * r * 4);
  }
  L.total = c.off;
  return L;
}

struct BwdLayout {
  int64_t h32, dh32, dhs, at, bt, part, spart, total;
};
// r: adapter slots in total (g rpart for grouped weights)
BwdLayout bwd_layout(int64_t m, int64_t n, int64_t k, int r, int rpart) {
  Carve c;
  BwdLayout L{};
  const int rp = rank_pad(r);
  const int splits = qlora::rank_reduce_splits(m, n, k, r);
  L.h32 = c.take(m * r * 4);
  L.dh32 = c.take(m * r * 4);
  L.dhs = c.take(m * rp * 2);
  L.at = c.take(k * rp * 2);
  L.bt = c.take(n * rp * 2);
  {
    const int sk = qlora::skinny_prefill_splits(m, k, r), sn = qlora::skinny_prefill_splits(m, n, r);
    L.spart = c.take(static_cast<int64_t>(sk > sn ? sk : sn) * m * r * 4);
  }
  if (r == 0) {
    L.part = c.take(0);
  } else if (qlora::rank_grads_fused(r) && qlora::rank_grads_fused(rpart)) {
    L.part = c.take(static_cast<int64_t>(qlora::rank_grad_splits(m, n, k, r, rpart)) * (r * k + rpart * n) * 4);
  } else {
    L.part = c.take(static_cast<int64_t>(splits) * r * (k > n ? k : n) * 4);
  }
  L.total = c.off;
  return L;
}

// Dropout calls: the masked copy of X first, then the forward's (GEMM path)
// or the backward's buffers.
int64_t drop_xm_bytes(int64_t m, int64_t k) { return round_up(m * k * 2, kAlign); }
int64_t drop_total(int64_t m, int64_t n, int64_t k, int r) {
  const int64_t f = fwd_layout(m, n, k, r, true).total;
  const int64_t b = bwd_layout(m, n, k, r, r).total;
  return drop_xm_bytes(m, k) + (f > b ? f : b);
}

// The sizes every linear entry point accepts (m <= 2^31, n and k <= 2^22):
// workspace queries beyond them return 0 instead of a size whose products
// overflow 64 bits.
bool linear_sizes_ok(int64_t m, int64_t n, int64_t k) {
  return m > 0 && n > 0 && k > 0 && m <= (INT64_C(1) << 31) && n <= (INT64_C(1) << 22) && k <= (INT64_C(1) << 22);
}

// Adapter dropout: keep mask (m x k bytes, non-zero = kept) and 1 / (1 - p).
struct DropArg {
  const uint8_t* keep;
  float inv_keep;
};

qlora_status check_weight(const qlora_nf4_weight* w, bool linear) {
  if (w == nullptr || w->codes == nullptr) return QLORA_ERR_NULL;
  if (w->double_quant < 0 || w->double_quant > 2) return QLORA_ERR_UNSUPPORTED;
  if (w->codebook != QLORA_CODEBOOK_NF4 && w->codebook != QLORA_CODEBOOK_INT4) return QLORA_ERR_UNSUPPORTED;
  if (w->double_quant) {
    if (w->scale_codes == nullptr || w->group_scale == nullptr) return QLORA_ERR_NULL;
    if (!aligned16(w->scale_codes) || !aligned16(w->group_scale)) return QLORA_ERR_ALIGN;
  } else {
    if (w->absmax == nullptr) return QLORA_ERR_NULL;
    if (!aligned16(w->absmax)) return QLORA_ERR_ALIGN;
  }
  if (!aligned16(w->codes)) return QLORA_ERR_ALIGN;
  if (w->n < 1 || w->k < 1) return QLORA_ERR_SHAPE;
  if (w->n > (INT64_C(1) << 40) / w->k) return QLORA_ERR_SHAPE;
  if (linear && ((w->k % QLORA_BLOCK) != 0 || (w->n % 16) != 0)) return QLORA_ERR_SHAPE;
  // the matmul kernels address a weight, and a 256-row tile of the
  // activations (m x k forward, m x n backward), with 32-bit offsets
  if (linear && w->n * w->k > (INT64_C(1) << 31)) return QLORA_ERR_SHAPE;
  if (linear && (w->n > (INT64_C(1) << 22) || w->k > (INT64_C(1) << 22))) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

PackedW view(const qlora_nf4_weight* w) {
  PackedW p;
  p.codes = w->codes;
  p.scale_codes = w->scale_codes;
  p.group_scale = w->group_scale;
  p.absmax = w->absmax;
  p.n = w->n;
  p.k = w->k;
  p.dq = w->double_quant;
  p.codebook = w->codebook;
  return p;
}

qlora_status hip_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP; }

// The fused GEMM numbers its 256 x 128 output tiles with 32-bit integers.
bool gemm_tiles_fit(int64_t m, int64_t p) { return ((m + 255) / 256) * ((p + 127) / 128) < (INT64_C(1) << 31); }

#define QLORA_TRY(expr)                       \
  do {                                        \
    const hipError_t e_ = (expr);             \
    if (e_ != hipSuccess) return QLORA_ERR_HIP; \
  } while (0)

}  // namespace

extern "C" {

const char* qlora_status_string(int status) {
  // an int, not the enum: callers pass values from other code, and a C++
  // enum object outside its enumerators' range is undefined behaviour
  switch (status) {
    case QLORA_OK:
      return "ok";
    case QLORA_ERR_NULL:
      return "a required pointer is NULL";
    case QLORA_ERR_SHAPE:
      return "invalid size (negative, zero, too large, k not a multiple of 64 or n not a multiple of 16)";
    case QLORA_ERR_ALIGN:
      return "a pointer is not 16-byte aligned";
    case QLORA_ERR_UNSUPPORTED:
      return "unsupported argument (rank above QLORA_MAX_RANK, dtype or flag)";
    case QLORA_ERR_WORKSPACE:
      return "workspace missing or too small";
    case QLORA_ERR_HIP:
      return "HIP kernel launch failed";
  }
  return "unknown status";
}

size_t qlora_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) {
  if (!linear_sizes_ok(m, n, k) || r < 0 || r > QLORA_MAX_RANK) return 0;
  const int64_t f = fwd_layout(m, n, k, r).total;
  const int64_t b = bwd_layout(m, n, k, r, r).total;
  return static_cast<size_t>(f > b ? f : b);
}

size_t qlora_linear_grouped_workspace_bytes(int64_t m, int64_t n, int64_t k, int g, int r) {
  if (!linear_sizes_ok(m, n, k) || g < 1 || g > QLORA_MAX_PARTS || r < 1 || g * r > QLORA_MAX_RANK) return 0;
  const int64_t f = fwd_layout(m, n, k, g * r).total;
  const int64_t b = bwd_layout(m, n, k, g * r, r).total;
  return static_cast<size_t>(f > b ? f : b);
}

qlora_status qlora_quantize_codebook(const float* w, int64_t numel, int double_quant, int codebook, uint8_t* codes,
                                uint8_t* scale_codes, float* group_scale, float* absmax, hipStream_t stream) {
  if (double_quant < 0 || double_quant > 2) return QLORA_ERR_UNSUPPORTED;
  if (codebook != QLORA_CODEBOOK_NF4 && codebook != QLORA_CODEBOOK_INT4) return QLORA_ERR_UNSUPPORTED;
  if (w == nullptr || codes == nullptr) return QLORA_ERR_NULL;
  if (double_quant && (scale_codes == nullptr || group_scale == nullptr)) return QLORA_ERR_NULL;
  if (!double_quant && absmax == nullptr) return QLORA_ERR_NULL;
  if (numel < 1 || numel > (INT64_C(1) << 40)) return QLORA_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(codes)) return QLORA_ERR_ALIGN;
  if (double_quant && (!aligned16(scale_codes) || !aligned16(group_scale))) return QLORA_ERR_ALIGN;
  if (absmax != nullptr && !aligned16(absmax)) return QLORA_ERR_ALIGN;
  return hip_status(qlora::launch_quantize(w, numel, double_quant, codebook, codes, double_quant ? scale_codes : nullptr,
                                           double_quant ? group_scale : nullptr, absmax, stream));
}

qlora_status qlora_nf4_quantize(const float* w, int64_t numel, int double_quant, uint8_t* codes,
                                uint8_t* scale_codes, float* group_scale, float* absmax, hipStream_t stream) {
  return qlora_quantize_codebook(w, numel, double_quant, QLORA_CODEBOOK_NF4, codes, scale_codes, group_scale, absmax,
                                 stream);
}

qlora_status qlora_nf4_dequantize(const qlora_nf4_weight* w, int out_dtype, void* out,
                                  hipStream_t stream) {
  const qlora_status st = check_weight(w, false);
  if (st != QLORA_OK) return st;
  if (out_dtype != QLORA_BF16 && out_dtype != QLORA_F32 && out_dtype != QLORA_F16) return QLORA_ERR_UNSUPPORTED;
  if (out == nullptr) return QLORA_ERR_NULL;
  if (!aligned16(out)) return QLORA_ERR_ALIGN;
  const int kind = out_dtype == QLORA_F32 ? 1 : (out_dtype == QLORA_F16 ? 2 : 0);
  return hip_status(qlora::launch_dequantize(view(w), kind, out, stream));
}

}  // extern "C"

namespace {

// Both linear calls in one form: a weight of grp->g parts (grp null: one
// part) with r adapter slots in total, rpart per part, s = alpha / rpart.
// The forward's checks of everything but the workspace.
qlora_status check_fwd_args(const qlora_nf4_weight* w, const uint16_t* x, int64_t m, const uint16_t* a,
                            const uint16_t* b, int r, const uint16_t* y, const float* h_out) {
  qlora_status st = check_weight(w, true);
  if (st != QLORA_OK) return st;
  if (m < 0 || m > (INT64_C(1) << 31)) return QLORA_ERR_SHAPE;
  if (r < 0) return QLORA_ERR_SHAPE;
  if (r > QLORA_MAX_RANK) return QLORA_ERR_UNSUPPORTED;
  if (!gemm_tiles_fit(m, w->n)) return QLORA_ERR_SHAPE;
  if (m == 0) return QLORA_OK;
  if (x == nullptr || y == nullptr) return QLORA_ERR_NULL;
  if (r > 0 && (a == nullptr || b == nullptr)) return QLORA_ERR_NULL;
  if (!aligned16(x) || !aligned16(y)) return QLORA_ERR_ALIGN;
  if (r > 0 && (!aligned16(a) || !aligned16(b))) return QLORA_ERR_ALIGN;
  if (h_out != nullptr && !aligned16(h_out)) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

qlora_status linear_fwd_impl(const qlora_nf4_weight* w, const qlora::LoraParts* grp, const uint16_t* x, int64_t m,
                             const uint16_t* a, const uint16_t* b, int r, int rpart, float alpha, uint16_t* y,
                             float* h_out, void* ws, size_t ws_bytes, hipStream_t stream,
                             const DropArg* drop = nullptr, bool f16 = false, bool fwd_sized_ws = false) {
  const qlora_status st = check_fwd_args(w, x, m, a, b, r, y, h_out);
  if (st != QLORA_OK || m == 0) return st;
  const int64_t n = w->n, k = w->k;
  const bool grouped = grp != nullptr;
  if (drop != nullptr && r == 0) drop = nullptr;  // no adapter, nothing to drop
  // the public calls size one workspace for both directions; a caller-owned
  // scratch area is checked against the forward's own layout
  const size_t need = fwd_sized_ws    ? static_cast<size_t>(fwd_layout(m, n, k, r).total)
                      : drop != nullptr ? static_cast<size_t>(drop_total(m, n, k, r))
                      : grouped         ? qlora_linear_grouped_workspace_bytes(m, n, k, grp->g, rpart)
                                        : qlora_linear_workspace_bytes(m, n, k, r);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (ws != nullptr && !aligned16(ws)) return QLORA_ERR_ALIGN;

  // with dropout: the GEMM path for every m, after the masked copy of X
  const bool gemm_path = drop != nullptr;
  const FwdLayout L = fwd_layout(m, n, k, r, gemm_path);
  char* base = static_cast<char*>(ws);
  const uint16_t* xa = x;  // the adapter's input
  if (drop != nullptr) {
    uint16_t* xm = reinterpret_cast<uint16_t*>(base);
    QLORA_TRY(qlora::launch_mask_input(x, drop->keep, m * k, xm, stream));
    xa = xm;
    base += drop_xm_bytes(m, k);
  }
  const float s = (rpart == 0) ? 0.0f : alpha / static_cast<float>(rpart);
  const int rp = rank_pad(r);
  const PackedW pw = view(w);

  if (m <= kGemvMaxM && !gemm_path) {
    // One launch when the GEMV computes H itself; otherwise H as per-split
    // partial sums in the workspace, which the GEMV sums.
    float* hpart = nullptr;
    const int splits = qlora::skinny_splits(m, k);
    if (r > 0 && !qlora::gemv_fuses_h(m, k, r, grp)) {
      hpart = reinterpret_cast<float*>(base + L.h32);
      QLORA_TRY(qlora::launch_skinny_decode(x, a, m, k, r, rp, hpart, splits, stream, f16));
    }
    QLORA_TRY(qlora::launch_gemv(pw, x, m, a, hpart, splits, b, r, s, y, h_out, stream, f16, grp));
  } else {
    float* h32 = (r == 0) ? nullptr : (h_out != nullptr ? h_out : reinterpret_cast<float*>(base + L.h32));
    uint16_t* hs = (r == 0) ? nullptr : reinterpret_cast<uint16_t*>(base + L.hs);
    // H of every part at once: the parts' A matrices are stacked (r x k)
    // H = D(X) A^T = (X * keep) A^T / (1 - p) under dropout
    const float hscale = drop != nullptr ? drop->inv_keep : 1.0f;
    if (r > 0)
      QLORA_TRY(qlora::launch_skinny_prefill(xa, a, m, k, r, rp, hscale, s, reinterpret_cast<float*>(base + L.part),
                                             h32, hs, stream, f16));
    qlora::LoraParts one;
    one.g = 1;
    one.rpart = rpart;
    one.end[0] = static_cast<int>(n);
    QLORA_TRY(qlora::launch_gemm_fwd(pw, x, m, hs, b, rpart, rp, grouped ? *grp : one, y, stream, f16));
  }
  return QLORA_OK;
}

qlora_status linear_bwd_impl(const qlora_nf4_weight* w, const qlora::LoraParts* grp, const uint16_t* x,
                             const uint16_t* dy, int64_t m, const uint16_t* a, const uint16_t* b, int r, int rpart,
                             float alpha, const float* h_saved, uint16_t* dx, float* da, float* db, void* ws,
                             size_t ws_bytes, hipStream_t stream, const DropArg* drop = nullptr,
                             bool f16 = false) {
  qlora_status st = check_weight(w, true);
  if (st != QLORA_OK) return st;
  if (m < 0 || m > (INT64_C(1) << 31)) return QLORA_ERR_SHAPE;
  if (r < 0) return QLORA_ERR_SHAPE;
  if (r > QLORA_MAX_RANK) return QLORA_ERR_UNSUPPORTED;
  const int64_t n = w->n, k = w->k;
  const bool grouped = grp != nullptr;
  if (!gemm_tiles_fit(m, k)) return QLORA_ERR_SHAPE;
  if (r > 0) {
    if (a == nullptr || b == nullptr || da == nullptr || db == nullptr) return QLORA_ERR_NULL;
    if (!aligned16(a) || !aligned16(b) || !aligned16(da) || !aligned16(db)) return QLORA_ERR_ALIGN;
  }
  if (m == 0) {
    if (r > 0) {
      QLORA_TRY(qlora::launch_fill_zero(da, static_cast<int64_t>(r) * k, stream));
      QLORA_TRY(qlora::launch_fill_zero(db, n * rpart, stream));
    }
    return QLORA_OK;
  }
  if (dy == nullptr) return QLORA_ERR_NULL;
  if (r > 0 && x == nullptr) return QLORA_ERR_NULL;
  if (dx == nullptr && r == 0) return QLORA_OK;  // nothing requested
  if (!aligned16(dy) || (x != nullptr && !aligned16(x)) || (dx != nullptr && !aligned16(dx))) return QLORA_ERR_ALIGN;
  if (h_saved != nullptr && !aligned16(h_saved)) return QLORA_ERR_ALIGN;
  if (drop != nullptr && r == 0) drop = nullptr;  // no adapter, nothing to drop
  const size_t need = drop != nullptr ? static_cast<size_t>(drop_total(m, n, k, r))
                      : grouped       ? qlora_linear_grouped_workspace_bytes(m, n, k, grp->g, rpart)
                                      : qlora_linear_workspace_bytes(m, n, k, r);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return QLORA_ERR_WORKSPACE;
  if (ws != nullptr && !aligned16(ws)) return QLORA_ERR_ALIGN;

  const BwdLayout L = bwd_layout(m, n, k, r, rpart);
  char* base = static_cast<char*>(ws);
  const uint16_t* xa = x;  // the adapter's input
  if (drop != nullptr) {
    uint16_t* xm = reinterpret_cast<uint16_t*>(base);
    QLORA_TRY(qlora::launch_mask_input(x, drop->keep, m * k, xm, stream));
    xa = xm;
    base += drop_xm_bytes(m, k);
  }
  const float s = (rpart == 0) ? 0.0f : alpha / static_cast<float>(rpart);
  const int rp = rank_pad(r);
  const PackedW pw = view(w);
  uint16_t* dhs = nullptr;
  uint16_t* at = nullptr;

  if (r > 0) {
    uint16_t* bt = reinterpret_cast<uint16_t*>(base + L.bt);
    at = reinterpret_cast<uint16_t*>(base + L.at);
    float* dh32 = reinterpret_cast<float*>(base + L.dh32);
    dhs = reinterpret_cast<uint16_t*>(base + L.dhs);
    float* part = reinterpret_cast<float*>(base + L.part);
    float* spart = reinterpret_cast<float*>(base + L.spart);
    const float* h = h_saved;
    const float inv_keep = drop != nullptr ? drop->inv_keep : 1.0f;
    if (h == nullptr) {
      float* h32 = reinterpret_cast<float*>(base + L.h32);
      QLORA_TRY(qlora::launch_skinny_prefill(xa, a, m, k, r, rp, inv_keep, 1.0f, spart, h32, nullptr, stream, f16));
      h = h32;
    }
    // A^T, and B^T (block diagonal for grouped weights: part l's slots see
    // only its own output columns)
    QLORA_TRY(qlora::launch_lora_transpose(a, b, n, k, r, rp, at, bt, stream, grp));
    // dH = s dY B  (contraction over n, with B^T as the r x n operand).
    // Under dropout dh32 holds dH / (1 - p), the factor both dA and the
    // masked dX update need; the frozen-weight GEMM then runs without
    // adapter slots.
    if (drop != nullptr) dhs = nullptr;
    QLORA_TRY(qlora::launch_skinny_prefill(dy, bt, m, n, r, rp, drop != nullptr ? s * inv_keep : s, 1.0f, spart, dh32,
                                           dhs, stream, f16));
    if (qlora::rank_grads_fused(r) && qlora::rank_grads_fused(rpart)) {
      // dA = dH^T X (r x k) and dB = s dY^T H (n x rpart) in one pass each
      QLORA_TRY(qlora::launch_rank_grads(dh32, xa, k, h, dy, n, m, r, grp, s,
                                         qlora::rank_grad_splits(m, n, k, r, rpart), part, da, db, stream, f16));
    } else {
      if (grouped) return QLORA_ERR_UNSUPPORTED;  // checked by the caller
      const int splits = qlora::rank_reduce_splits(m, n, k, r);
      // dA = dH^T X  (r x k)
      QLORA_TRY(qlora::launch_rank_reduce(dh32, xa, m, k, r, 1.0f, splits, part, da, 0, stream, f16));
      // dB = s dY^T H  (n x r)
      QLORA_TRY(qlora::launch_rank_reduce(h, dy, m, n, r, s, splits, part, db, 1, stream, f16));
    }
  }
  if (dx != nullptr) {
    if (drop != nullptr) {
      // dX = dY W16, then + (dH A) / (1 - p) where the input was kept
      QLORA_TRY(qlora::launch_gemm_dx(pw, dy, m, nullptr, nullptr, 0, dx, stream, f16));
      QLORA_TRY(qlora::launch_masked_lora_add(dx, drop->keep, reinterpret_cast<const float*>(base + L.dh32), a, m, k,
                                              r, stream, f16));
    } else {
      QLORA_TRY(qlora::launch_gemm_dx(pw, dy, m, dhs, at, rp, dx, stream, f16));
    }
  }
  return QLORA_OK;
}

// Parts of a grouped weight: 1..QLORA_MAX_PARTS row counts, each a positive
// multiple of 256, summing to w->n; rank r >= 1 per part, g r <= QLORA_MAX_RANK.
qlora_status group_parts(const qlora_nf4_weight* w, int g, const int64_t* parts, int r, qlora::LoraParts* out) {
  if (w == nullptr || parts == nullptr) return QLORA_ERR_NULL;
  if (g < 1 || g > QLORA_MAX_PARTS || r < 1) return QLORA_ERR_SHAPE;
  if (g * r > QLORA_MAX_RANK) return QLORA_ERR_UNSUPPORTED;
  int64_t end = 0;
  out->g = g;
  out->rpart = r;
  for (int l = 0; l < g; ++l) {
    if (parts[l] <= 0 || parts[l] % 256 != 0) return QLORA_ERR_SHAPE;
    end += parts[l];
    if (end > w->n) return QLORA_ERR_SHAPE;
    out->end[l] = static_cast<int>(end);
  }
  if (end != w->n) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

}  // namespace

extern "C" {

qlora_status qlora_linear_fwd(const qlora_nf4_weight* w, const uint16_t* x, int64_t m, const uint16_t* a,
                              const uint16_t* b, int r, float alpha, uint16_t* y, float* h_out, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  return linear_fwd_impl(w, nullptr, x, m, a, b, r, r, alpha, y, h_out, ws, ws_bytes, stream);
}

}  // extern "C"

namespace qlora {

qlora_status linear_fwd_check(const qlora_nf4_weight* w, const uint16_t* x, int64_t m, const uint16_t* a,
                              const uint16_t* b, int r, const uint16_t* y, const float* h_out) {
  return check_fwd_args(w, x, m, a, b, r, y, h_out);
}

size_t linear_fwd_scratch_bytes(int64_t m, int64_t n, int64_t k, int r) {
  // sizes the forward rejects: 0, and the forward itself reports the error
  if (!linear_sizes_ok(m, n, k) || r < 0 || r > QLORA_MAX_RANK) return 0;
  return static_cast<size_t>(fwd_layout(m, n, k, r).total);
}

qlora_status linear_fwd_scratch(const qlora_nf4_weight* w, const uint16_t* x, int64_t m, const uint16_t* a,
                                const uint16_t* b, int r, float alpha, uint16_t* y, float* h_out, void* scratch,
                                size_t scratch_bytes, hipStream_t stream) {
  return linear_fwd_impl(w, nullptr, x, m, a, b, r, r, alpha, y, h_out, scratch, scratch_bytes, stream, nullptr, false,
                         true);
}

}  // namespace qlora

extern "C" {

qlora_status qlora_linear_bwd(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy, int64_t m,
                              const uint16_t* a, const uint16_t* b, int r, float alpha, const float* h_saved,
                              uint16_t* dx, float* da, float* db, void* ws, size_t ws_bytes, hipStream_t stream) {
  return linear_bwd_impl(w, nullptr, x, dy, m, a, b, r, r, alpha, h_saved, dx, da, db, ws, ws_bytes, stream);
}

qlora_status qlora_linear_fwd_grouped(const qlora_nf4_weight* w, int g, const int64_t* parts, const uint16_t* x,
                                      int64_t m, const uint16_t* a, const uint16_t* b, int r, float alpha,
                                      uint16_t* y, float* h_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  qlora::LoraParts lp;
  const qlora_status st = group_parts(w, g, parts, r, &lp);
  if (st != QLORA_OK) return st;
  return linear_fwd_impl(w, &lp, x, m, a, b, g * r, r, alpha, y, h_out, ws, ws_bytes, stream);
}

qlora_status qlora_linear_fwd_grouped_f16(const qlora_nf4_weight* w, int g, const int64_t* parts, const uint16_t* x,
                                          int64_t m, const uint16_t* a, const uint16_t* b, int r, float alpha,
                                          uint16_t* y, float* h_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  qlora::LoraParts lp;
  const qlora_status st = group_parts(w, g, parts, r, &lp);
  if (st != QLORA_OK) return st;
  return linear_fwd_impl(w, &lp, x, m, a, b, g * r, r, alpha, y, h_out, ws, ws_bytes, stream, nullptr, true);
}

qlora_status qlora_linear_bwd_grouped(const qlora_nf4_weight* w, int g, const int64_t* parts, const uint16_t* x,
                                      const uint16_t* dy, int64_t m, const uint16_t* a, const uint16_t* b, int r,
                                      float alpha, const float* h_saved, uint16_t* dx, float* da, float* db, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  qlora::LoraParts lp;
  const qlora_status st = group_parts(w, g, parts, r, &lp);
  if (st != QLORA_OK) return st;
  if (r % 16 != 0) return QLORA_ERR_UNSUPPORTED;
  return linear_bwd_impl(w, &lp, x, dy, m, a, b, g * r, r, alpha, h_saved, dx, da, db, ws, ws_bytes, stream);
}

qlora_status qlora_linear_bwd_grouped_f16(const qlora_nf4_weight* w, int g, const int64_t* parts, const uint16_t* x,
                                          const uint16_t* dy, int64_t m, const uint16_t* a, const uint16_t* b, int r,
                                          float alpha, const float* h_saved, uint16_t* dx, float* da, float* db,
                                          void* ws, size_t ws_bytes, hipStream_t stream) {
  qlora::LoraParts lp;
  const qlora_status st = group_parts(w, g, parts, r, &lp);
  if (st != QLORA_OK) return st;
  if (r % 16 != 0) return QLORA_ERR_UNSUPPORTED;
  return linear_bwd_impl(w, &lp, x, dy, m, a, b, g * r, r, alpha, h_saved, dx, da, db, ws, ws_bytes, stream, nullptr,
                         true);
}


// Adapter arguments of the merge calls: r in 0..QLORA_MAX_RANK; for r > 0,
// a (r x k) and b (n x r) are required and 16-byte aligned.
static qlora_status check_adapter(const uint16_t* a, const uint16_t* b, int r) {
  if (r < 0) return QLORA_ERR_SHAPE;
  if (r > QLORA_MAX_RANK) return QLORA_ERR_UNSUPPORTED;
  if (r > 0 && (a == nullptr || b == nullptr)) return QLORA_ERR_NULL;
  if (r > 0 && (!aligned16(a) || !aligned16(b))) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

qlora_status qlora_merge(const qlora_nf4_weight* w, const uint16_t* a, const uint16_t* b, int r, float alpha,
                         int out_dtype, void* out, hipStream_t stream) {
  qlora_status st = check_weight(w, false);
  if (st != QLORA_OK) return st;
  if (w->k % QLORA_BLOCK != 0) return QLORA_ERR_SHAPE;
  if (out_dtype != QLORA_BF16 && out_dtype != QLORA_F32) return QLORA_ERR_UNSUPPORTED;
  if ((st = check_adapter(a, b, r)) != QLORA_OK) return st;
  if (out == nullptr) return QLORA_ERR_NULL;
  if (!aligned16(out)) return QLORA_ERR_ALIGN;
  const float s = (r == 0) ? 0.0f : alpha / static_cast<float>(r);
  return hip_status(qlora::launch_merge(view(w), a, b, r, s, out_dtype == QLORA_F32, out, stream));
}

qlora_status qlora_unmerge(const void* merged, int dtype, int64_t n, int64_t k, const uint16_t* a,
                           const uint16_t* b, int r, float alpha, void* out, hipStream_t stream) {
  if (dtype != QLORA_BF16 && dtype != QLORA_F32) return QLORA_ERR_UNSUPPORTED;
  if (n < 1 || k < 1 || k % 8 != 0 || n > (INT64_C(1) << 40) / k) return QLORA_ERR_SHAPE;
  qlora_status st = check_adapter(a, b, r);
  if (st != QLORA_OK) return st;
  if (merged == nullptr || out == nullptr) return QLORA_ERR_NULL;
  if (!aligned16(merged) || !aligned16(out)) return QLORA_ERR_ALIGN;
  const float s = (r == 0) ? 0.0f : alpha / static_cast<float>(r);
  return hip_status(qlora::launch_unmerge(merged, dtype == QLORA_F32, n, k, a, b, r, s, out, stream));
}

qlora_status qlora_requantize(const qlora_nf4_weight* w, const uint16_t* a, const uint16_t* b, int r, float alpha,
                              int double_quant, int codebook, float* merged, uint8_t* codes, uint8_t* scale_codes,
                              float* group_scale, float* absmax, hipStream_t stream) {
  qlora_status st = check_weight(w, false);
  if (st != QLORA_OK) return st;
  if (w->k % QLORA_BLOCK != 0) return QLORA_ERR_SHAPE;
  if ((st = check_adapter(a, b, r)) != QLORA_OK) return st;
  if (double_quant < 0 || double_quant > 2) return QLORA_ERR_UNSUPPORTED;
  if (codebook != QLORA_CODEBOOK_NF4 && codebook != QLORA_CODEBOOK_INT4) return QLORA_ERR_UNSUPPORTED;
  if (merged == nullptr || codes == nullptr) return QLORA_ERR_NULL;
  if (double_quant && (scale_codes == nullptr || group_scale == nullptr)) return QLORA_ERR_NULL;
  if (!double_quant && absmax == nullptr) return QLORA_ERR_NULL;
  if (!aligned16(merged) || !aligned16(codes)) return QLORA_ERR_ALIGN;
  if (double_quant && (!aligned16(scale_codes) || !aligned16(group_scale))) return QLORA_ERR_ALIGN;
  if (absmax != nullptr && !aligned16(absmax)) return QLORA_ERR_ALIGN;
  const float s = (r == 0) ? 0.0f : alpha / static_cast<float>(r);
  QLORA_TRY(qlora::launch_merge(view(w), a, b, r, s, 1, merged, stream));
  return hip_status(qlora::launch_quantize(merged, w->n * w->k, double_quant, codebook, codes,
                                           double_quant ? scale_codes : nullptr, double_quant ? group_scale : nullptr,
                                           absmax, stream));
}

// Dropout probability p in [0, 1) (NaN fails the test) and the keep mask.
static qlora_status make_drop(const uint8_t* keep, float p, DropArg* out) {
  if (!(p >= 0.0f && p < 1.0f)) return QLORA_ERR_UNSUPPORTED;
  if (keep == nullptr) return QLORA_ERR_NULL;
  if (!aligned16(keep)) return QLORA_ERR_ALIGN;
  out->keep = keep;
  out->inv_keep = static_cast<float>(1.0 / (1.0 - static_cast<double>(p)));
  return QLORA_OK;
}

size_t qlora_linear_dropout_workspace_bytes(int64_t m, int64_t n, int64_t k, int r) {
  if (!linear_sizes_ok(m, n, k) || r < 0 || r > QLORA_MAX_RANK) return 0;
  if (r == 0) return qlora_linear_workspace_bytes(m, n, k, r);
  return static_cast<size_t>(drop_total(m, n, k, r));
}

qlora_status qlora_linear_fwd_dropout(const qlora_nf4_weight* w, const uint16_t* x, int64_t m, const uint16_t* a,
                                      const uint16_t* b, int r, float alpha, const uint8_t* keep, float p,
                                      uint16_t* y, float* h_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (m == 0) return linear_fwd_impl(w, nullptr, x, m, a, b, r, r, alpha, y, h_out, ws, ws_bytes, stream);
  DropArg d{};
  const qlora_status st = make_drop(keep, p, &d);
  if (st != QLORA_OK) return st;
  return linear_fwd_impl(w, nullptr, x, m, a, b, r, r, alpha, y, h_out, ws, ws_bytes, stream, &d);
}

qlora_status qlora_linear_bwd_dropout(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy, int64_t m,
                                      const uint16_t* a, const uint16_t* b, int r, float alpha, const uint8_t* keep,
                                      float p, const float* h_saved, uint16_t* dx, float* da, float* db, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
  if (m == 0)
    return linear_bwd_impl(w, nullptr, x, dy, m, a, b, r, r, alpha, h_saved, dx, da, db, ws, ws_bytes, stream);
  DropArg d{};
  const qlora_status st = make_drop(keep, p, &d);
  if (st != QLORA_OK) return st;
  return linear_bwd_impl(w, nullptr, x, dy, m, a, b, r, r, alpha, h_saved, dx, da, db, ws, ws_bytes, stream, &d);
}

qlora_status qlora_linear_fwd_dropout_f16(const qlora_nf4_weight* w, const uint16_t* x, int64_t m, const uint16_t* a,
                                          const uint16_t* b, int r, float alpha, const uint8_t* keep, float p,
                                          uint16_t* y, float* h_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (m == 0)
    return linear_fwd_impl(w, nullptr, x, m, a, b, r, r, alpha, y, h_out, ws, ws_bytes, stream, nullptr, true);
  DropArg d{};
  const qlora_status st = make_drop(keep, p, &d);
  if (st != QLORA_OK) return st;
  return linear_fwd_impl(w, nullptr, x, m, a, b, r, r, alpha, y, h_out, ws, ws_bytes, stream, &d, true);
}

qlora_status qlora_linear_bwd_dropout_f16(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy,
                                          int64_t m, const uint16_t* a, const uint16_t* b, int r, float alpha,
                                          const uint8_t* keep, float p, const float* h_saved, uint16_t* dx, float* da,
                                          float* db, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (m == 0)
    return linear_bwd_impl(w, nullptr, x, dy, m, a, b, r, r, alpha, h_saved, dx, da, db, ws, ws_bytes, stream,
                           nullptr, true);
  DropArg d{};
  const qlora_status st = make_drop(keep, p, &d);
  if (st != QLORA_OK) return st;
  return linear_bwd_impl(w, nullptr, x, dy, m, a, b, r, r, alpha, h_saved, dx, da, db, ws, ws_bytes, stream, &d,
                         true);
}

qlora_status qlora_dropout_mask(uint64_t seed, uint64_t offset, int64_t count, float p, uint8_t* keep,
                                hipStream_t stream) {
  if (!(p >= 0.0f && p < 1.0f)) return QLORA_ERR_UNSUPPORTED;
  if (count < 1 || count > (INT64_C(1) << 40) || offset % 16 != 0) return QLORA_ERR_SHAPE;
  if (keep == nullptr) return QLORA_ERR_NULL;
  if (!aligned16(keep)) return QLORA_ERR_ALIGN;
  return hip_status(qlora::launch_dropout_mask(seed, offset / 16, count, p * 65536.0f, keep, stream));
}

qlora_status qlora_linear_fwd_f16(const qlora_nf4_weight* w, const uint16_t* x, int64_t m, const uint16_t* a,
                                  const uint16_t* b, int r, float alpha, uint16_t* y, float* h_out, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  return linear_fwd_impl(w, nullptr, x, m, a, b, r, r, alpha, y, h_out, ws, ws_bytes, stream, nullptr, true);
}

qlora_status qlora_linear_bwd_f16(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy, int64_t m,
                                  const uint16_t* a, const uint16_t* b, int r, float alpha, const float* h_saved,
                                  uint16_t* dx, float* da, float* db, void* ws, size_t ws_bytes, hipStream_t stream) {
  return linear_bwd_impl(w, nullptr, x, dy, m, a, b, r, r, alpha, h_saved, dx, da, db, ws, ws_bytes, stream, nullptr,
                         true);
}

}  // extern "C"
