// Decode path (m <= 16 tokens): Y = X W16^T + s H B^T with W read straight
// from its packed NF4 form.
//
// Ultralytics glossary "QLoRA", section "Come funziona QLoRA": each frozen
// layer dequantizes its NF4 weights to bfloat16 right before the matmul and
// adds the LoRA path output. At a handful of tokens the layer is bound by the
// HBM stream of the packed weight (0.5 B of codes + 1/64 B of scale codes per
// weight), so the kernel is built around that stream:
//   * a workgroup owns 16 weight rows; its WAVES x 4 lane groups split the
//     row's 64-blocks round-robin, so every lane loads whole blocks (32 B of
//     codes, two 16-byte loads); all loads of a pass are issued
//     unconditionally (clamped addresses; an out-of-range block gets a zero
//     scale) before the first is used, so a pass costs one memory round
//     trip -- a guarded load would make the compiler wait for every
//     outstanding load at the guard;
//   * per block a lane decodes the scale, builds a 16-entry bf16 table in
//     registers (nf4_lut.h) and looks up 8 weights per table access;
//   * the dot products run on the matrix cores (16x16x32 bf16 MFMA with the
//     tokens padded to 16 rows), so the vector ALU only unpacks;
//   * X is pre-arranged by the LoRA-down kernel in the lookup's output order,
//     and partial sums of the waves are reduced in a fixed order in LDS.
#include "internal.h"
#include "mfma.h"
#include "nf4_lut.h"

namespace qlora {
namespace {

constexpr int kGroup = 256;

template <int WAVES, bool kDQ>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(PackedW w, const uint16_t* __restrict__ xp, int M,
                                                          const float* __restrict__ hpart, int hsplits,
                                                          const uint16_t* __restrict__ b, int r, float s,
                                                          uint16_t* __restrict__ y, float* __restrict__ h_out,
                                                          Levels L) {
  constexpr int kLaneGroups = WAVES * 4;
  __shared__ f32x4 red[WAVES][64];
  __shared__ float h_lds[16 * QLORA_MAX_RANK];
  __shared__ uint16_t b_lds[16 * QLORA_MAX_RANK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int G = wave * 4 + g;
  // 32-bit offsets: the host guarantees n * k <= 2^31
  const int K = static_cast<int>(w.k), N = static_cast<int>(w.n);
  const int nbk = K / 64;
  const int n0 = blockIdx.x * 16;
  const int n = n0 + i;
  const int n_c = n < N ? n : N - 1;     // clamped: every load is unconditional
  const int xrow = i < M ? i : M - 1;    // rows past M feed outputs that are never stored

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  // One block per lane group per pass. All loads of a pass (codes, scale,
  // X) are issued unconditionally from clamped addresses before any is used;
  // a block past the row or past K gets a zero scale, so its weights are 0.
  for (int base = 0; base < nbk; base += kLaneGroups) {
    const int kb = base + G;
    const int kb_c = kb < nbk ? kb : nbk - 1;
    const u32x4* cp = reinterpret_cast<const u32x4*>(w.codes + (n_c * (K / 2) + kb_c * 32));
    const u32x4 c0 = __builtin_nontemporal_load(cp);
    const u32x4 c1 = __builtin_nontemporal_load(cp + 1);
    const int bi = n_c * nbk + kb_c;
    uint32_t scode = 0;
    float gsc;
    if (kDQ) {
      scode = w.scale_codes[bi];
      gsc = w.group_scale[bi / kGroup];
    } else {
      gsc = w.absmax[bi];
    }
    u32x4 xa[8];
    const uint16_t* xr = xp + xrow * K + kb_c * 64;
#pragma unroll
    for (int j = 0; j < 8; ++j) xa[j] = ld16(xr + 8 * j);
    if (base == 0) {
      // Epilogue operands, fetched while the weight loads are in flight: H =
      // sum of the LoRA-down partials (fixed order) and this workgroup's 16
      // rows of B (contiguous in memory).
      const int mr = M * r;
      for (int idx = tid; idx < mr; idx += WAVES * 64) {
        float hv = 0.0f;
        for (int sp = 0; sp < hsplits; ++sp) hv += hpart[sp * mr + idx];
        h_lds[idx] = hv;
        if (h_out != nullptr && blockIdx.x == 0) h_out[idx] = hv;
      }
      const int blast = N * r - 1;
      for (int idx = tid; idx < 16 * r; idx += WAVES * 64) {
        const int e = n0 * r + idx;
        b_lds[idx] = b[e < blast ? e : blast];  // rows past N are never stored
      }
    }
    // wave-uniform: skip a pass slot no lane group of this wave uses
    if (base + wave * 4 < nbk) {
      const bool ok = (n < N) && (kb < nbk);
      const float sc = kDQ ? u8_unit(scode) * gsc : gsc;
      const BlockLut lut = make_block_lut(L.v, ok ? sc : 0.0f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t cw = (j < 4) ? c0[j] : c1[j - 4];
        uint32_t wv[4];
        lut8_decode_order(lut, cw, wv);
        acc = mfma_16x16x32(xa[j], u32x4{wv[0], wv[1], wv[2], wv[3]}, acc);
      }
    }
  }

  red[wave][lane] = acc;
  __syncthreads();
  if (tid >= 256) return;
  const int l2 = tid & 63, v = tid >> 6;
  const int mo = 4 * (l2 >> 4) + v;
  const int no = n0 + (l2 & 15);
  if (mo >= M || no >= N) return;
  float sum = 0.0f;
#pragma unroll
  for (int wv = 0; wv < WAVES; ++wv) sum += red[wv][l2][v];
  if (r > 0) {
    float lo = 0.0f;
    const uint16_t* brow = b_lds + (l2 & 15) * r;
    const float* hrow = h_lds + mo * r;
    for (int j = 0; j < r; ++j) lo = fmaf(hrow[j], __uint_as_float(static_cast<uint32_t>(brow[j]) << 16), lo);
    sum = fmaf(s, lo, sum);
  }
  y[mo * N + no] = f32_to_bf16_rne(sum);
}

}  // namespace

hipError_t launch_gemv(const PackedW& w, const uint16_t* xp, int64_t m, const float* hpart, int hsplits,
                       const uint16_t* b, int r, float s, uint16_t* y, float* h_out, hipStream_t st) {
  constexpr int kWaves = 16;
  const unsigned grid = static_cast<unsigned>((w.n + 15) / 16);
  auto kern = w.dq ? gemv_kernel<kWaves, true> : gemv_kernel<kWaves, false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kWaves * 64), 0, st, w, xp, static_cast<int>(m), hpart, hsplits, b, r, s,
                     y, h_out, nf4_table());
  return hipGetLastError();
}

}  // namespace qlora
