/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) QLoRA NF4 linear layer.
 *
 * What the library computes (pages cited by title and section):
 *   - Ultralytics glossary "QLoRA", section "Come funziona QLoRA":
 *       NF4 bullet: each weight is a 4-bit code pointing at one of 16 levels
 *       placed at normal quantiles; every block of 64 weights has one absmax
 *       scale. Double-quantization bullet: the per-block scales are themselves
 *       quantized to 8 bit in blocks of 256 (0.5 -> ~0.127 bit/param).
 *       Forward/backward paragraph: every frozen layer dequantizes its NF4
 *       weights to bfloat16 right before the matmul and adds the LoRA path;
 *       the backward goes through the dequantized weights but only the two
 *       LoRA matrices receive gradients.
 *   - "LoRA y QLoRA en Profundidad", sections "La Idea Central" and "Alpha":
 *       W is d_out x d_in, A is r x d_in, B is d_out x r, and the adapter
 *       contributes (alpha / r) * B @ A.
 *   - "Modulo 4: QLoRA", section 4.3 b): the weights are quantized to 4 bit,
 *       then the scale constants to 8 bit.
 *
 * Numeric conventions (the readings taken where the pages are silent):
 *   - levels: 16 float32 values, ascending, level 7 is +0.0, levels 0 and 15
 *     are -1 and +1 (see qlora_nf4_levels). The same page's NF4-vs-INT4
 *     example also names the evenly spaced 4-bit code; a weight may use it
 *     instead (codebook QLORA_CODEBOOK_INT4: level k = fl32(-1 + 2k/15), no
 *     exact zero level), with every other convention unchanged;
 *   - block b covers elements [64 b, 64 b + 64) of the row-major flattening
 *     (the last block may be partial); group g covers blocks [256 g, 256 g + 256);
 *   - a_b = max |w| over block b; x = w / a_b (correctly rounded float32);
 *     code = argmin_k fl32(|x - L_k|), lowest k on ties; an all-zero block
 *     has code 7 everywhere;
 *   - packing: byte i holds element 2i in bits 0..3 and element 2i+1 in bits
 *     4..7; an odd element count leaves the last high nibble 0;
 *   - double quantization: M_g = max a_b over group g; c2_b = argmin_k
 *     fl32(|a_b / M_g - U_k|) with U_k = fl32(k / 255), lowest k on ties
 *     (c2_b = 0 when M_g = 0); decoded scale s_b = fl32(U[c2_b] * M_g);
 *     without double quantization s_b = a_b stored as float32. double_quant
 *     = 2 selects a float-like 8-bit code instead of k/255: E_c, c = 16 e +
 *     m, is m 2^-18 for e = 0 and (16 + m) 2^(e - 19) otherwise (E_240 = 1;
 *     codes above 240 exceed 1 and are never chosen), with the same nearest
 *     rule; s_b = fl32(E[c2_b] * M_g). Its relative scale error stays below
 *     1/32 down to a_b / M_g = 2^-14, where k/255 degrades for small ratios;
 *   - dequantized weight: w32 = fl32(L[code] * s_b); w16 = bf16 round-to-
 *     nearest-even of w32. Codes, c2, M_g, w32 and w16 are bit-exact with the
 *     CPU oracle;
 *   - linear: s = fl32(alpha / r); Y = X W16^T + s (X A^T) B^T; bf16 inputs,
 *     float32 accumulation, bf16 Y and dX, float32 H, dA and dB.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, 16-byte aligned, row-major,
 *     owned by the caller. The library never allocates or frees caller memory
 *     and keeps no state besides a constant level table built once on the host.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream). No
 *     host synchronisation happens inside a call. Results are valid once the
 *     stream reaches that point.
 *   - Argument errors are detected on the host, before anything is enqueued,
 *     and returned as a negative status; QLORA_ERR_HIP reports a failed
 *     launch (hipGetLastError). Nothing is thrown across the ABI. Calls are
 *     thread-safe; calls that write the same buffers must be ordered by the
 *     caller.
 *   - Weights must be finite; non-finite weights give undefined codes. X, dY,
 *     A and B must be finite as well: the matmul kernels may multiply
 *     elements past a ragged edge of X or dY by exact zeros, so a non-finite
 *     value there could reach a neighbouring output.
 */
#ifndef QLORA_NF4_H_
#define QLORA_NF4_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = -1,        /* a required pointer is NULL                     */
  QLORA_ERR_SHAPE = -2,       /* a size is negative / zero where not allowed,   */
                              /* or, for the linear entry points, k % 64 != 0   */
                              /* or n % 16 != 0                                 */
  QLORA_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned               */
  QLORA_ERR_UNSUPPORTED = -4, /* r > QLORA_MAX_RANK, unknown dtype or flag      */
  QLORA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required        */
  QLORA_ERR_HIP = -6          /* a kernel launch failed                         */
} qlora_status;

/* Element types; the calls take them as plain int (any other value is
 * rejected with QLORA_ERR_UNSUPPORTED). */
typedef enum { QLORA_BF16 = 0, QLORA_F32 = 1, QLORA_F16 = 2 } qlora_dtype;

#define QLORA_BLOCK 64     /* weights per absmax block              */
#define QLORA_DQ_GROUP 256 /* blocks per double-quantization group  */
#define QLORA_MAX_RANK 128 /* largest LoRA rank r the kernels take  */
#define QLORA_MAX_PARTS 4  /* most linears in one grouped call      */

#define QLORA_DQ_NONE 0    /* fp32 absmax per block                 */
#define QLORA_DQ_LINEAR8 1 /* 8-bit scale codes k / 255 (default)   */
#define QLORA_DQ_FLOAT8 2  /* 8-bit float-like scale codes E_c      */

#define QLORA_CODEBOOK_NF4 0  /* normal-quantile levels (the default)  */
#define QLORA_CODEBOOK_INT4 1 /* 16 evenly spaced levels on [-1, 1]    */

/* A packed NF4 weight W (n x k, row-major, numel = n * k). Device pointers.
 *   codes        : ceil(numel / 2) bytes, packing as above.
 *   scale_codes  : double_quant = 1 or 2: ceil(numel / 64) uint8 codes c2_b.
 *   group_scale  : double_quant = 1 or 2: ceil(ceil(numel / 64) / 256) float M_g.
 *   absmax       : double_quant = 0: ceil(numel / 64) float a_b.
 *   codebook     : QLORA_CODEBOOK_NF4 or QLORA_CODEBOOK_INT4, the level table
 *                  the codes index (a zero-initialised struct selects NF4).
 * Pointers not used by the selected mode may be NULL. */
typedef struct {
  int64_t n, k;
  const uint8_t* codes;
  const uint8_t* scale_codes;
  const float* group_scale;
  const float* absmax;
  int32_t double_quant;
  int32_t codebook;
} qlora_nf4_weight;

/* Quantize `numel` float32 weights `w` (any numel >= 1; partial last block and
 * group allowed). Ultralytics glossary "QLoRA", "Come funziona QLoRA" (NF4 and
 * double-quantization bullets); "Modulo 4: QLoRA" 4.3 b) for the order
 * (weights with their exact absmax first, then the scales).
 * Outputs (caller-allocated device buffers):
 *   codes       : ceil(numel/2) bytes.
 *   double_quant = 1: scale_codes (ceil(numel/64) bytes) and group_scale
 *     (ceil(ceil(numel/64)/256) floats) are required; absmax may be NULL, and
 *     if given receives the exact float a_b.
 *   double_quant = 0: absmax (ceil(numel/64) floats) is required;
 *     scale_codes and group_scale are ignored.
 * double_quant = 2 is the same with the float-like scale code (QLORA_DQ_FLOAT8).
 * Errors: NULL / ALIGN / SHAPE (numel < 1) / UNSUPPORTED (flag not 0, 1 or 2) / HIP. */
qlora_status qlora_nf4_quantize(const float* w, int64_t numel, int double_quant, uint8_t* codes,
                                uint8_t* scale_codes, float* group_scale, float* absmax,
                                hipStream_t stream);

/* qlora_nf4_quantize with the level table chosen by `codebook`
 * (QLORA_CODEBOOK_NF4 gives exactly qlora_nf4_quantize; QLORA_CODEBOOK_INT4
 * the evenly spaced levels of the NF4-vs-INT4 example in Ultralytics glossary
 * "QLoRA", "Come funziona QLoRA"). The nearest-level rule, ties, packing,
 * blocks and double quantization are the same; an all-zero block gets code 7
 * in either table. A weight quantized this way is used with its
 * qlora_nf4_weight.codebook set to the same value.
 * Errors: as qlora_nf4_quantize, and UNSUPPORTED for an unknown codebook. */
qlora_status qlora_quantize_codebook(const float* w, int64_t numel, int double_quant, int codebook,
                                     uint8_t* codes, uint8_t* scale_codes, float* group_scale,
                                     float* absmax, hipStream_t stream);

/* Dequantize a packed weight to bf16 (w16) or float32 (w32), n*k elements,
 * row-major, into `out`; QLORA_F16 gives the IEEE-half rounding (nearest
 * even) of w32 instead, the weight of the fp16 compute calls. Ultralytics glossary "QLoRA", "Come funziona QLoRA"
 * (restore = level[code] * scale; dequantize to bfloat16 before the matmul).
 * Any n, k >= 1 (k need not be a multiple of 64 here).
 * Errors: NULL / ALIGN / SHAPE / UNSUPPORTED (dtype) / HIP. */
qlora_status qlora_nf4_dequantize(const qlora_nf4_weight* w, int out_dtype, void* out,
                                  hipStream_t stream);

/* Forward: Y = X W16^T + s (X A^T) B^T with s = fl32(alpha / r).
 * Ultralytics glossary "QLoRA", "Come funziona QLoRA" (forward paragraph);
 * "LoRA y QLoRA en Profundidad", "La Idea Central" / "Alpha".
 *   w     : packed NF4 weight, n x k, k % 64 == 0, n % 16 == 0, n * k <= 2^31,
 *           n <= 2^22 and k <= 2^22.
 *   x     : bf16 (uint16 bit patterns) m x k, m <= 2^31.
 *   a     : bf16 r x k; b : bf16 n x r. r = 0 (a, b NULL) means base only.
 *   y     : bf16 m x n output.
 *   h_out : optional float32 m x r output of H = X A^T (pass it to the
 *           backward to skip recomputing H); may be NULL.
 *   ws    : device workspace of at least qlora_linear_workspace_bytes(m,n,k,r)
 *           bytes (may be NULL when that is 0). Contents are scratch.
 * m = 0 is a no-op. m <= 16 takes the decode (GEMV) kernels, larger m the
 * fused dequant-GEMM. Y does not depend on which path runs beyond float32
 * accumulation order.
 * Errors: NULL / ALIGN / SHAPE / UNSUPPORTED (r > QLORA_MAX_RANK) / WORKSPACE / HIP. */
qlora_status qlora_linear_fwd(const qlora_nf4_weight* w, const uint16_t* x, int64_t m,
                              const uint16_t* a, const uint16_t* b, int r, float alpha,
                              uint16_t* y, float* h_out, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* Backward of the forward above for L with dL/dY = dy (bf16 m x n).
 * Ultralytics glossary "QLoRA", "Come funziona QLoRA": gradients flow through
 * the dequantized frozen weight; only A and B get gradients (no dW).
 *   dX = dY W16 + dH A   (bf16 m x k; dx may be NULL to skip it)
 *   dA = dH^T X          (float32 r x k, overwritten)
 *   dB = s dY^T H        (float32 n x r, overwritten)
 * with H = X A^T and dH = s dY B. h_saved (float32 m x r, from the forward's
 * h_out) may be NULL, in which case H is recomputed. With r = 0, only dX is
 * produced (a, b, da, db ignored). m = 0 writes zeros to dA and dB.
 * dA and dB are computed in a fixed order: results are run-to-run identical.
 * Errors: NULL / ALIGN / SHAPE / UNSUPPORTED / WORKSPACE / HIP. */
qlora_status qlora_linear_bwd(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy,
                              int64_t m, const uint16_t* a, const uint16_t* b, int r, float alpha,
                              const float* h_saved, uint16_t* dx, float* da, float* db, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* The same two calls with IEEE half as the 16-bit compute type ("Modulo 4:
 * QLoRA", section "QLoRA combina tres componentes clave": the LoRA weights
 * stay in full 16-bit precision, BF16 or FP16): X, A, B, dY, Y and dX are
 * fp16 (uint16_t bit patterns), the weight is dequantized to fp16
 * (round-to-nearest-even of w32) inside the matmuls, and the f16 matrix-core
 * instructions accumulate in float32. H, dA and dB stay float32. Arguments,
 * layouts, limits, workspace (qlora_linear_workspace_bytes) and errors are
 * those of qlora_linear_fwd / qlora_linear_bwd. */
qlora_status qlora_linear_fwd_f16(const qlora_nf4_weight* w, const uint16_t* x, int64_t m,
                                  const uint16_t* a, const uint16_t* b, int r, float alpha,
                                  uint16_t* y, float* h_out, void* ws, size_t ws_bytes,
                                  hipStream_t stream);
qlora_status qlora_linear_bwd_f16(const qlora_nf4_weight* w, const uint16_t* x, const uint16_t* dy,
                                  int64_t m, const uint16_t* a, const uint16_t* b, int r,
                                  float alpha, const float* h_saved, uint16_t* dx, float* da,
                                  float* db, void* ws, size_t ws_bytes, hipStream_t stream);

/* Forward and backward with dropout on the adapter path ("LoRA y QLoRA en
 * Profundidad", "Dropout (lora_dropout)": the LoRA layers randomly zero
 * elements during training). The adapter's input is dropped, the frozen
 * path is not:
 *   D(X) = X * keep / (1 - p),   H = D(X) A^T,   Y = X W16^T + s H B^T;
 *   dH = s dY B,   dX = dY W16 + (dH A) * keep / (1 - p),
 *   dA = dH^T D(X),   dB = s dY^T H.
 *   keep : m x k bytes, row-major, 16-byte aligned; non-zero = element kept.
 *          The caller draws it (Bernoulli(1 - p) per element) and passes
 *          the same mask to both calls of a step.
 *   p    : drop probability, 0 <= p < 1 (the factor is fl32(1 / (1 - p))).
 *   h_out / h_saved : H from the dropped input, as above.
 *   ws   : at least qlora_linear_dropout_workspace_bytes(m, n, k, r).
 * Every other argument, layout and limit is as in qlora_linear_fwd /
 * qlora_linear_bwd; every m takes the matmul path. r = 0 is the plain call.
 * Errors: as those calls, plus NULL (keep), ALIGN (keep) and UNSUPPORTED
 * (p outside [0, 1)). */
size_t qlora_linear_dropout_workspace_bytes(int64_t m, int64_t n, int64_t k, int r);

/* Draw a keep mask on the device with a counter-based generator, Philox4x64
 * with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011), so that the mask for the dropout calls above
 * is reproducible from (seed, offset) alone.
 *   Element i (0 <= i < count) is element g = offset + i of one stream. Block
 *   b = g / 16 gives the four 64-bit words Philox4x64-10(counter (b, 0, 0, 0),
 *   key (seed, 0)); chunk j = g % 16 is bits 16 (j % 4) .. 16 (j % 4) + 15 of
 *   word j / 4, and keep[i] = 0 when float(chunk) < 65536 p, else 1. The
 *   drop probability is ceil(65536 p) / 65536.
 *   offset % 16 == 0 (distinct layers and steps take disjoint windows);
 *   1 <= count <= 2^40; 0 <= p < 1; keep: count bytes, device, 16-byte
 *   aligned. Bit-exact with the CPU oracle.
 * Errors: NULL / ALIGN / SHAPE / UNSUPPORTED (p) / HIP. */
qlora_status qlora_dropout_mask(uint64_t seed, uint64_t offset, int64_t count, float p, uint8_t* keep,
                                hipStream_t stream);
qlora_status qlora_linear_fwd_dropout(const qlora_nf4_weight* w, const uint16_t* x, int64_t m,
                                      const uint16_t* a, const uint16_t* b, int r, float alpha,
                                      const uint8_t* keep, float p, uint16_t* y, float* h_out,
                                      void* ws, size_t ws_bytes, hipStream_t stream);
qlora_status qlora_linear_bwd_dropout(const qlora_nf4_weight* w, const uint16_t* x,
                                      const uint16_t* dy, int64_t m, const uint16_t* a,
                                      const uint16_t* b, int r, float alpha, const uint8_t* keep,
                                      float p, const float* h_saved, uint16_t* dx, float* da,
                                      float* db, void* ws, size_t ws_bytes, hipStream_t stream);

/* The two dropout calls with IEEE half as the compute type (X, A, B, dY,
 * Y and dX fp16), as qlora_linear_fwd_f16 / qlora_linear_bwd_f16 are to the
 * plain calls. Arguments, workspace and errors as the bf16 dropout calls. */
qlora_status qlora_linear_fwd_dropout_f16(const qlora_nf4_weight* w, const uint16_t* x, int64_t m,
                                          const uint16_t* a, const uint16_t* b, int r, float alpha,
                                          const uint8_t* keep, float p, uint16_t* y, float* h_out,
                                          void* ws, size_t ws_bytes, hipStream_t stream);
qlora_status qlora_linear_bwd_dropout_f16(const qlora_nf4_weight* w, const uint16_t* x,
                                          const uint16_t* dy, int64_t m, const uint16_t* a,
                                          const uint16_t* b, int r, float alpha,
                                          const uint8_t* keep, float p, const float* h_saved,
                                          uint16_t* dx, float* da, float* db, void* ws,
                                          size_t ws_bytes, hipStream_t stream);

/* Bytes of device workspace that qlora_linear_fwd and qlora_linear_bwd need
 * for these sizes (the larger of the two); 0 if none, and 0 for sizes the
 * calls reject (m <= 0 or m > 2^31, n or k outside 1 .. 2^22, r outside
 * 0 .. QLORA_MAX_RANK). Host only, no GPU use. */
size_t qlora_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, int r);

/* Largest scratch area qlora_linear_fwd_noalloc uses (16 MiB per device). */
#define QLORA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* qlora_linear_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The call itself allocates nothing
 * (no hipMalloc, hipFree or allocating library routine). The forward's
 * scratch (split partial sums of H and the padded bf16 s H of the matmul
 * path; partial sums of H on the decode path when r > 16) lives in a
 * library-owned device array of QLORA_NOALLOC_SCRATCH_BYTES, one per
 * device, held until the process ends; its device address is looked up on
 * the first call on each device.
 *   Arguments, layouts, limits and results are those of qlora_linear_fwd
 *   (the same kernels: outputs are bit-identical to qlora_linear_fwd's on the
 *   same inputs). The caller still allocates x, a, b, y and h_out.
 *   Every call on one device shares that device's array, and the array keeps
 *   the last call's contents (nothing in it needs to start at zero): calls
 *   that overlap on one device (different streams or threads without
 *   ordering) race and give undefined results. Order them on one stream.
 * Errors: as qlora_linear_fwd; QLORA_ERR_WORKSPACE when these sizes need
 * more than QLORA_NOALLOC_SCRATCH_BYTES (checked on the host before
 * anything is enqueued); QLORA_ERR_HIP if the array's address cannot be
 * found on the current device. */
qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_weight* w, const uint16_t* x, int64_t m,
                                      const uint16_t* a, const uint16_t* b, int r, float alpha,
                                      uint16_t* y, float* h_out, hipStream_t stream);

/* Grouped linears that read the same input: the adapted projections of one
 * block ("LoRA y QLoRA en Profundidad", "Modulos Objetivo": q/k/v of the
 * attention, gate/up of the MLP), run as one call over their stacked weights.
 *   w     : the g weights W_1..W_g stacked by rows (n = sum of parts) and
 *           quantized as one matrix. With k % 64 == 0 and every part a
 *           multiple of 256 rows, no block or double-quantization group spans
 *           two parts, so the codes, scale codes and group scales are those
 *           of the parts quantized separately, laid end to end.
 *   g     : number of parts, 1 .. QLORA_MAX_PARTS.
 *   parts : host array of the g row counts (each a positive multiple of 256,
 *           summing to w->n).
 *   a     : bf16 (g r) x k, the parts' A matrices stacked (part l: rows l r ..).
 *   b     : bf16 n x r, the parts' B matrices stacked (part l: its rows of W).
 *   r     : rank of every part (1 <= r, g r <= QLORA_MAX_RANK); s = fl32(alpha / r).
 * Forward: y (bf16 m x n) holds, in the columns of part l,
 *   X W_l^T + s (X A_l^T) B_l^T;
 * h_out (float32 m x (g r), may be NULL) = [X A_1^T | ... | X A_g^T].
 * Backward for dL/dY = dy (bf16 m x n, part l in its columns):
 *   dx (bf16 m x k, may be NULL) = sum over l of dY_l W_l + dH_l A_l,
 *   da (float32 (g r) x k) = the dA_l stacked, db (float32 n x r) = the dB_l
 *   stacked, with dH_l = s dY_l B_l, dA_l = dH_l^T X, dB_l = s dY_l^T H_l;
 *   h_saved (float32 m x (g r), from h_out) may be NULL. The backward needs
 *   r % 16 == 0 (QLORA_ERR_UNSUPPORTED otherwise).
 * The forward takes the decode (GEMV) kernels for m <= 16 and the fused
 * dequant-GEMM above; the backward takes the GEMM for every m. ws must hold
 * qlora_linear_grouped_workspace_bytes(m, n, k, g, r) bytes.
 * Errors as for the single-linear calls; SHAPE also for bad parts. */
qlora_status qlora_linear_fwd_grouped(const qlora_nf4_weight* w, int g, const int64_t* parts,
                                      const uint16_t* x, int64_t m, const uint16_t* a,
                                      const uint16_t* b, int r, float alpha, uint16_t* y,
                                      float* h_out, void* ws, size_t ws_bytes, hipStream_t stream);
qlora_status qlora_linear_bwd_grouped(const qlora_nf4_weight* w, int g, const int64_t* parts,
                                      const uint16_t* x, const uint16_t* dy, int64_t m,
                                      const uint16_t* a, const uint16_t* b, int r, float alpha,
                                      const float* h_saved, uint16_t* dx, float* da, float* db,
                                      void* ws, size_t ws_bytes, hipStream_t stream);

/* The two grouped calls with IEEE half as the compute type (X, A, B, dY, Y
 * and dX fp16), as qlora_linear_fwd_f16 / qlora_linear_bwd_f16 are to the
 * plain calls. Arguments, workspace and errors as the bf16 grouped calls. */
qlora_status qlora_linear_fwd_grouped_f16(const qlora_nf4_weight* w, int g, const int64_t* parts,
                                          const uint16_t* x, int64_t m, const uint16_t* a,
                                          const uint16_t* b, int r, float alpha, uint16_t* y,
                                          float* h_out, void* ws, size_t ws_bytes,
                                          hipStream_t stream);
qlora_status qlora_linear_bwd_grouped_f16(const qlora_nf4_weight* w, int g, const int64_t* parts,
                                          const uint16_t* x, const uint16_t* dy, int64_t m,
                                          const uint16_t* a, const uint16_t* b, int r, float alpha,
                                          const float* h_saved, uint16_t* dx, float* da, float* db,
                                          void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for the grouped calls (n = sum of parts); 0 for invalid
 * sizes. Host only, no GPU use. */
size_t qlora_linear_grouped_workspace_bytes(int64_t m, int64_t n, int64_t k, int g, int r);

/* Merge a trained adapter into the weight: out (n x k, row-major) =
 * fl32(W16 + t), where W16 is the bf16 dequantized weight (as
 * qlora_nf4_dequantize), t = fl32(s d), s = fl32(alpha / r), and d is the
 * float32 sum of b[p][j] a[j][q] over j = 0 .. r-1 in that order (each step
 * one float32 addition; bf16 products are exact). "LoRA y QLoRA en
 * Profundidad", "La Idea Central" (W + (alpha/r) B A for inference);
 * Ultralytics glossary "QLoRA", "Compromessi" (merging starts from the
 * weight dequantized to 16 bit).
 *   w         : packed weight, k % 64 == 0 (any codebook, DQ on or off).
 *   a, b      : bf16 A (r x k) and B (n x r); may be NULL when r = 0.
 *   r         : 0 .. QLORA_MAX_RANK; r = 0 gives out = W16.
 *   out_dtype : QLORA_F32 writes the float32 value, QLORA_BF16 its
 *               round-to-nearest-even bf16 (the 16-bit model).
 *   out       : n x k, caller-allocated.
 * Bit-exact with the CPU oracle. Errors: NULL / ALIGN / SHAPE (k % 64 != 0,
 * r < 0) / UNSUPPORTED (r > QLORA_MAX_RANK, dtype, codebook, flag) / HIP. */
qlora_status qlora_merge(const qlora_nf4_weight* w, const uint16_t* a, const uint16_t* b, int r,
                         float alpha, int out_dtype, void* out, hipStream_t stream);

/* Take an adapter back out of a merged weight (adapters are stored and
 * swapped per task: Ultralytics glossary "QLoRA", "Compromessi"):
 * out = fl32(W' - t) with t as in qlora_merge.
 *   merged : W', n x k, bf16 (dtype QLORA_BF16) or float32 (QLORA_F32).
 *   out    : n x k of the same dtype (bf16: round-to-nearest-even); may be
 *            `merged` itself (in place).
 *   n >= 1, k % 8 == 0. a, b, r, alpha as in qlora_merge.
 * Errors: NULL / ALIGN / SHAPE / UNSUPPORTED / HIP. */
qlora_status qlora_unmerge(const void* merged, int dtype, int64_t n, int64_t k,
                           const uint16_t* a, const uint16_t* b, int r, float alpha, void* out,
                           hipStream_t stream);

/* Re-quantize a merged model for distribution (Ultralytics glossary
 * "QLoRA", "QLoRA e metodi correlati": the merged 16-bit weights are
 * quantized again). Two launches on `stream`: `merged` (n x k float32,
 * caller-allocated) receives qlora_merge's float32 output, then the packed
 * outputs receive qlora_quantize_codebook(merged, n k, double_quant,
 * codebook, ...), with the same buffer sizes and NULL rules. The new weight
 * may use another codebook or DQ mode than `w`.
 * Errors: as qlora_merge and qlora_quantize_codebook. */
qlora_status qlora_requantize(const qlora_nf4_weight* w, const uint16_t* a, const uint16_t* b, int r,
                              float alpha, int double_quant, int codebook, float* merged,
                              uint8_t* codes, uint8_t* scale_codes, float* group_scale,
                              float* absmax, hipStream_t stream);

/* Static, NUL-terminated description of a status (any int: values that are
 * no qlora_status get a generic text). Host only. */
const char* qlora_status_string(int status);

/* Copy the 16 float32 NF4 levels the kernels use into out16 (host memory).
 * The table is built on the host from the standard-normal quantile at the
 * offset 0.9677083 (Ultralytics glossary "QLoRA", the NF4-vs-INT4 example).
 * Returns 16, or QLORA_ERR_NULL. Host only, no GPU use. */
int qlora_nf4_levels(float out16[16]);

/* Copy the 16 float32 levels of `codebook` into out16 (host memory):
 * QLORA_CODEBOOK_NF4 as qlora_nf4_levels, QLORA_CODEBOOK_INT4 level k =
 * fl32(-1 + 2k/15) (correctly rounded; the last is exactly +1).
 * Returns 16, QLORA_ERR_NULL or QLORA_ERR_UNSUPPORTED. Host only. */
int qlora_codebook_levels(int codebook, float out16[16]);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H_ */
