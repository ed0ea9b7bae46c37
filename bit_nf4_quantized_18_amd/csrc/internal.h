// Internal declarations shared by the host library and the kernels.
//
// Every launcher that reads or writes 16-bit activations takes `f16`: false
// for bfloat16 (the default), true for IEEE half; the data layout is the same.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlora_nf4.h"

namespace qlora {

// Native vector types (for 16-byte loads/stores and MFMA operands).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The 16 NF4 levels as float32, passed to kernels by value (kernarg -> SGPRs).
struct Levels {
  float v[16];
};

// Host-side level table, built once (thread-safe) from the standard-normal
// quantile function.
const Levels& nf4_table();
// The table of a codebook: QLORA_CODEBOOK_NF4 or QLORA_CODEBOOK_INT4 (16
// evenly spaced levels on [-1, 1]); any other value gives the NF4 table.
const Levels& codebook_table(int codebook);

// Nearest-level encoding of x in [-1, 1] for the quantize kernel, by
// buckets of t = 16 x. Between adjacent levels L_k < L_k+1 the rule "code
// k + 1 when fl32(L_k+1 - x) < fl32(x - L_k), else k" switches once, at a
// float U_k (both distances are monotone in x), so the code of x is the
// number of switch points U_k <= x. Bucket b = floor(t) + 16 (0 .. 32)
// covers t in [b - 16, b - 15); base[b] counts the switch points at or
// below its start and thr16[b] is 16 U_k of the one switch point inside it
// (+inf if none: adjacent switch points are more than 1/16 apart for both
// codebooks). Built once per codebook on the host from the level table.
struct EncodeTable {
  float thr16[33];
  uint32_t base[33];
};
const EncodeTable& encode_table(int codebook);

// ---------------------------------------------------------------------------
// Launchers (each enqueues on `s` and returns hipGetLastError()).
// ---------------------------------------------------------------------------
hipError_t launch_quantize(const float* w, int64_t numel, int dq, int codebook, uint8_t* codes, uint8_t* scale_codes,
                           float* group_scale, float* absmax, hipStream_t s);

// Packed weight view used by all kernels that read NF4 weights.
struct PackedW {
  const uint8_t* codes;
  const uint8_t* scale_codes;  // dq
  const float* group_scale;    // dq
  const float* absmax;         // !dq
  int64_t n, k;
  int dq;
  int codebook;  // QLORA_CODEBOOK_*
};

// out_kind: 0 bf16, 1 float32, 2 IEEE half.
hipError_t launch_dequantize(const PackedW& w, int out_kind, void* out, hipStream_t s);

// H-like skinny projection: out[m][j] = scale * sum_q P[m][q] * Q[j][q] for j < r,
// P bf16 m x qn (row stride qn, qn % 8 == 0), Q bf16 r x qn. With one
// contraction split (m > 16) it writes out_f32 (m x r, may be null) and
// out_bf16 (m x rpad, zero-padded for j >= r, may be null) holding
// bf16(scale2 * scale * sum). With several splits (m <= 16, see
// skinny_splits, decode path only) it writes raw partial sums to out_f32 as splits x m x r.
hipError_t launch_skinny(const uint16_t* P, const uint16_t* Q, int64_t m, int64_t qn, int r, int rpad,
                         float scale, float scale2, float* out_f32, uint16_t* out_bf16, int splits, hipStream_t s,
                         bool f16 = false);
int skinny_splits(int64_t m, int64_t qn);
// Decode (m <= 16) partial sums of the same projection with scale 1: part is
// splits x m x r float32, splits = skinny_splits(m, qn); rpad / 16 in
// {2, 4, 6, 8} (the GEMV computes H itself for r <= 16).
hipError_t launch_skinny_decode(const uint16_t* P, const uint16_t* Q, int64_t m, int64_t qn, int r, int rpad,
                                float* part, int splits, hipStream_t s, bool f16 = false);

// Prefill (m > 16) form of the same projection, split over the contraction
// for parallelism: raw partials in part (skinny_prefill_splits(m, qn, r) x m x r
// float32), then out_f32 (m x r, may be null) = scale * sum and out_bf16
// (m x rpad, may be null) = bf16(scale2 * scale * sum), zero-padded. For
// r <= 16 the partials come from a streaming kernel (LDS ring, MFMA).
int skinny_prefill_splits(int64_t m, int64_t qn, int r);
hipError_t launch_skinny_prefill(const uint16_t* P, const uint16_t* Q, int64_t m, int64_t qn, int r, int rpad,
                                 float scale, float scale2, float* part, float* out_f32, uint16_t* out_bf16,
                                 hipStream_t st, bool f16 = false);

// A weight made of g row blocks (grouped linears sharing their input): part
// l covers output rows end[l-1] .. end[l]-1 (end[-1] = 0) and owns adapter
// slots l rpart .. (l+1) rpart - 1. g = 1 (the default): one part.
struct LoraParts {
  int g = 1;
  int rpart = 0;
  int end[4] = {0, 0, 0, 0};
};

// Decode GEMV, m <= 16: y = x W16^T + s * h B^T in one launch when
// gemv_fuses_h(n, k, r, parts) (H = x A^T computed in the kernel from a);
// otherwise hpart holds hsplits partial sums of H (hsplits x m x r float32,
// from launch_skinny_decode). r = 0: base only. h_out (m x r, may be null)
// receives H. Grouped weights (parts != null): r = g rpart slots of H (a is
// r x k), b is n x rpart and row p of part l takes H's slots l rpart ..
// (l+1) rpart - 1. H is fused for 3..16 tokens, or k > 12288, when r <= 16;
// for one or two tokens at k <= 4096 when r <= 32 (one part) or rpart <= 16
// (grouped); never for one or two tokens at 4096 < k <= 12288.
// A call with parts fuses whenever the same call without them would.
bool gemv_fuses_h(int64_t m, int64_t k, int r, const LoraParts* parts);
int device_cus();
hipError_t launch_gemv(const PackedW& w, const uint16_t* x, int64_t m, const uint16_t* a, const float* hpart,
                       int hsplits, const uint16_t* b, int r, float s, uint16_t* y, float* h_out, hipStream_t st,
                       bool f16 = false, const LoraParts* parts = nullptr);
// The matrix-core form (3..16 tokens, or k > 4096); same arguments as launch_gemv.
hipError_t launch_gemv_mfma(const PackedW& w, const uint16_t* x, int64_t m, const uint16_t* a, const float* hpart,
                            int hsplits, const uint16_t* b, int r, float s, uint16_t* y, float* h_out, hipStream_t st,
                            bool f16, const LoraParts* parts);

// Fused dequant-GEMM, forward: y = x W16^T + the LoRA term where hs is bf16
// m x rpad (already scaled by s) and b is n x r bf16 (r = slots per part);
// output column p of part l adds sum_j hs[.][l r + j] b[p][j].
hipError_t launch_gemm_fwd(const PackedW& w, const uint16_t* x, int64_t m, const uint16_t* hs,
                           const uint16_t* b, int r, int rpad, const LoraParts& parts, uint16_t* y, hipStream_t st,
                           bool f16 = false);

// Fused dequant-GEMM, backward data: dx = dy W16 + dhs At where dhs is bf16
// m x rpad and at is bf16 k x rpad (A transposed, zero padded).
hipError_t launch_gemm_dx(const PackedW& w, const uint16_t* dy, int64_t m, const uint16_t* dhs,
                          const uint16_t* at, int rpad, uint16_t* dx, hipStream_t st, bool f16 = false);

// Transposes with zero padding: bt (rpad x n) from b (n x r); at (k x rpad) from a (r x k).
// Grouped weights (parts != null, r = g rpart): b is n x rpart (the parts' B
// stacked) and bt is block diagonal: slot j of part l is zero outside part l's columns.
hipError_t launch_lora_transpose(const uint16_t* a, const uint16_t* b, int64_t n, int64_t k, int r, int rpad,
                                 uint16_t* at, uint16_t* bt, hipStream_t st, const LoraParts* parts = nullptr);

// out(j, c) = scale * sum_m U[m][j] * V[m][c], U float32 m x r, V bf16 m x cn.
// Deterministic: `splits` partial sums over m-ranges into part (splits x r x cn),
// then a fixed-order reduce. c_major=0 writes out[j*cn + c], 1 writes out[c*r + j].
hipError_t launch_rank_reduce(const float* U, const uint16_t* V, int64_t m, int64_t cn, int r, float scale,
                              int splits, float* part, float* out, int c_major, hipStream_t st, bool f16 = false);

hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t st);

// Merge: out (w.n x w.k, float32 if out_f32 else bf16) = w16 + t with
// t = fl32(s d), d the float32 sum over ascending j of b[p][j] a[j][q]
// (a r x k, b n x r bf16). Unmerge: out = merged - t for a dense merged
// weight (float32 if src_f32, else bf16; out of the same type, may alias).
// k % 64 == 0 for merge, k % 8 == 0 for unmerge; r = 0 gives t = 0.
hipError_t launch_merge(const PackedW& w, const uint16_t* a, const uint16_t* b, int r, float s, int out_f32,
                        void* out, hipStream_t st);
// Adapter dropout: xm = x where keep != 0, else +0 (count = m k, a multiple
// of 8); dx += keep ? dh a : 0 per element, dh float32 m x r, a bf16 r x k,
// k % 64 == 0, dx rounded to bf16 once.
hipError_t launch_mask_input(const uint16_t* x, const uint8_t* keep, int64_t count, uint16_t* xm, hipStream_t st);
// keep[i] for i < count from Philox4x64-10 block block0 + i / 16 under the
// key (seed, 0): 16-bit chunk i % 16, dropped when float(chunk) < thr.
hipError_t launch_dropout_mask(uint64_t seed, uint64_t block0, int64_t count, float thr, uint8_t* keep,
                               hipStream_t st);
hipError_t launch_masked_lora_add(uint16_t* dx, const uint8_t* keep, const float* dh, const uint16_t* a, int64_t m,
                                  int64_t k, int r, hipStream_t st, bool f16 = false);

hipError_t launch_unmerge(const void* merged, int src_f32, int64_t n, int64_t k, const uint16_t* a,
                          const uint16_t* b, int r, float s, void* out, hipStream_t st);

int rank_reduce_splits(int64_t m, int64_t n, int64_t k, int r);

// Both adapter gradients in two launches when rank_grads_fused(r)
// (r % 16 == 0): da (r x k) = dh^T x and db (n x r) = scale * dy^T h, with
// dh, h float32 m x r and x, dy bf16. part holds splits x r x (k + n)
// float32 partial sums (splits = rank_grad_splits), reduced in a fixed order.
// Grouped weights (parts != null): dh and h are m x r0 with r0 = g rpart,
// da is r0 x k and db is n x rpart, row p of db (part l) from h columns
// l rpart .. (l+1) rpart - 1; part holds splits x (r0 k + rpart n) float32.
bool rank_grads_fused(int r);
int rank_grad_splits(int64_t m, int64_t n, int64_t k, int r0, int r1);
hipError_t launch_rank_grads(const float* dh, const uint16_t* x, int64_t k, const float* h, const uint16_t* dy,
                             int64_t n, int64_t m, int r0, const LoraParts* parts, float scale, int splits, float* part,
                             float* da, float* db, hipStream_t st, bool f16 = false);

// The plain forward (qlora_linear_fwd) on a scratch area the caller
// provides, checked against the forward's own workspace layout
// (linear_fwd_scratch_bytes) rather than the two-direction size of the
// public calls; QLORA_ERR_WORKSPACE if it is too small. linear_fwd_check
// runs the forward's argument checks alone (no device use);
// linear_fwd_scratch_bytes is 0 for sizes those checks reject.
qlora_status linear_fwd_check(const qlora_nf4_weight* w, const uint16_t* x, int64_t m, const uint16_t* a,
                              const uint16_t* b, int r, const uint16_t* y, const float* h_out);
size_t linear_fwd_scratch_bytes(int64_t m, int64_t n, int64_t k, int r);
qlora_status linear_fwd_scratch(const qlora_nf4_weight* w, const uint16_t* x, int64_t m, const uint16_t* a,
                                const uint16_t* b, int r, float alpha, uint16_t* y, float* h_out, void* scratch,
                                size_t scratch_bytes, hipStream_t stream);

}  // namespace qlora
