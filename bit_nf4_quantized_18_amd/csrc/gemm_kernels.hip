// Fused dequant-GEMMs over the packed NF4 weight (prefill / training shapes).
//
// Ultralytics glossary "QLoRA", section "Come funziona QLoRA": each frozen
// layer dequantizes its NF4 weights to bfloat16 right before the matmul, adds
// the LoRA path, and the backward computes gradients through the dequantized
// weights. Here the dequantization happens inside the K-loop of the GEMM:
// packed codes are read from HBM, turned into bf16 tiles in registers and
// staged in LDS for the matrix cores; the bf16 copy of W never exists in HBM.
//
//   forward  (kTransW = false): Y[m][n]  = sum_k X[m][k]  W[n][k] + sum_j Hs[m][j] B[n][j]
//   backward (kTransW = true):  dX[m][k] = sum_n dY[m][n] W[n][k] + sum_j dHs[m][j] At[k][j]
//
// Workgroup tile: 256 token rows x 128 output columns x 64 contraction (one
// NF4 block per weight row and step), 4 waves as 2 x 2, each wave 128 x 64 =
// 8 x 4 tiles of the 16x16x32 bf16 MFMA. The token tile is tall so that the
// per-weight unpacking cost (table build + byte-permute lookups) is shared by
// 256 rows. LDS holds two stages (A and dequantized W), rows padded to 144 B
// so that 16 lanes reading 16 B each hit 64 distinct banks. One barrier per
// step: the next stage is unpacked into the other buffer while the current
// one feeds the MFMAs, and its global loads were issued a step earlier.
// The rank-r LoRA term is one more pass of MFMAs over the r-wide operands.
#include "internal.h"
#include "mfma.h"
#include "nf4_lut.h"

namespace qlora {
namespace {

constexpr int kBM = 256, kBP = 128, kBQ = 64;
constexpr int kPitch = kBQ + 8;  // bf16 elements per LDS row (144 B)
constexpr int kGroup = 256;

struct Stage {
  u32x4 a[8];   // 8 x 16 B of the A tile
  u32x4 codes;  // 32 codes of one weight row (half a block)
  float scale;
};

template <bool kTransW>
__global__ __launch_bounds__(256) void nf4_gemm_kernel(PackedW w, const uint16_t* __restrict__ A, int64_t M,
                                                       int64_t P, int64_t Qn, const uint16_t* __restrict__ ep_a,
                                                       const uint16_t* __restrict__ ep_b, int64_t ep_ld, int ep_lim,
                                                       int rpad, uint16_t* __restrict__ out, Levels L) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBP * kPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wp = wave & 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kBP;
  const int64_t K = w.k;
  const int64_t nbk = K / 64;
  const int64_t nk = (Qn + kBQ - 1) / kBQ;

  // --- per-thread roles in the tile loads ---------------------------------
  // A tile: chunks t + 256 u -> row t/8 + 32 u, 16-byte column t % 8.
  const int a_row = tid >> 3, a_col = (tid & 7) * 8;
  // W tile. Forward: weight row p0 + tid/2, k-half tid%2 of the step.
  // Backward: weight row q0 + tid%64, k-quarter tid/64 of the output tile.
  const int w_r = kTransW ? (tid & 63) : (tid >> 1);
  const int w_c = kTransW ? (tid >> 6) * 32 : (tid & 1) * 32;

  auto load_stage = [&](int64_t kt, Stage& st) {
    const int64_t q0 = kt * kBQ;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t m = m0 + a_row + 32 * u;
      const int64_t q = q0 + a_col;
      st.a[u] = u32x4{0, 0, 0, 0};
      if (m < M && q < Qn) st.a[u] = ld16(A + m * Qn + q);
    }
    int64_t wrow, wk;
    if (kTransW) {
      wrow = q0 + w_r;
      wk = p0 + w_c;
    } else {
      wrow = p0 + w_r;
      wk = q0 + w_c;
    }
    st.codes = u32x4{0, 0, 0, 0};
    st.scale = 0.0f;
    if (wrow < w.n && wk < K) {
      st.codes = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w.codes + (wrow * K + wk) / 2));
      const int64_t bi = wrow * nbk + wk / 64;
      st.scale = w.dq ? (static_cast<float>(w.scale_codes[bi]) / 255.0f) * w.group_scale[bi / kGroup] : w.absmax[bi];
    }
  };

  auto store_stage = [&](int buf, const Stage& st) {
    uint16_t* as = As[buf];
#pragma unroll
    for (int u = 0; u < 8; ++u) st16(as + (a_row + 32 * u) * kPitch + a_col, st.a[u]);
    const BlockLut lut = make_block_lut(L.v, st.scale);
    uint16_t* bs = Bs[buf];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t wv[4];
      lut8_natural_order(lut, st.codes[j], wv);
      if (kTransW) {
        // element (n = w_r, k = w_c + 8 j + e) goes to Bs[k][n]
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t word = wv[e >> 1];
          bs[(w_c + 8 * j + e) * kPitch + w_r] = static_cast<uint16_t>((e & 1) ? (word >> 16) : word);
        }
      } else {
        st16(bs + w_r * kPitch + w_c + 8 * j, u32x4{wv[0], wv[1], wv[2], wv[3]});
      }
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    const uint16_t* as = As[buf] + (wm * 128 + i) * kPitch + 8 * g;
    const uint16_t* bs = Bs[buf] + (wp * 64 + i) * kPitch + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 fa[8], fb[4];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) fa[mt] = ld16(as + 16 * mt * kPitch + 32 * ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) fb[nt] = ld16(bs + 16 * nt * kPitch + 32 * ks);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_16x16x32(fa[mt], fb[nt], acc[mt][nt]);
    }
  };

  Stage st;
  load_stage(0, st);
  store_stage(0, st);
  if (nk > 1) load_stage(1, st);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int buf = static_cast<int>(kt & 1);
    compute(buf);
    if (kt + 1 < nk) store_stage(buf ^ 1, st);
    if (kt + 2 < nk) load_stage(kt + 2, st);
    __syncthreads();
  }

  // LoRA term: rpad more contraction slots.
  for (int ks = 0; ks < rpad / 32; ++ks) {
    u32x4 fa[8], fb[4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int64_t m = m0 + wm * 128 + 16 * mt + i;
      fa[mt] = (m < M) ? ld16(ep_a + m * rpad + 32 * ks + 8 * g) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t p = p0 + wp * 64 + 16 * nt + i;
      fb[nt] = (p < P) ? ld8_bf16_guarded(ep_b + p * ep_ld, 32 * ks + 8 * g, ep_lim, (ep_ld % 8) == 0)
                       : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_16x16x32(fa[mt], fb[nt], acc[mt][nt]);
  }

#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t p = p0 + wp * 64 + 16 * nt + i;
      if (p >= P) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = m0 + wm * 128 + 16 * mt + 4 * g + v;
        if (m < M) out[m * P + p] = f32_to_bf16_rne(acc[mt][nt][v]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_fwd(const PackedW& w, const uint16_t* x, int64_t m, const uint16_t* hs, const uint16_t* b,
                           int r, int rpad, uint16_t* y, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((w.n + kBP - 1) / kBP), static_cast<unsigned>((m + kBM - 1) / kBM));
  hipLaunchKernelGGL(nf4_gemm_kernel<false>, grid, dim3(256), 0, st, w, x, m, w.n, w.k, hs, b,
                     static_cast<int64_t>(r), r, rpad, y, nf4_table());
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const PackedW& w, const uint16_t* dy, int64_t m, const uint16_t* dhs, const uint16_t* at,
                          int rpad, uint16_t* dx, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((w.k + kBP - 1) / kBP), static_cast<unsigned>((m + kBM - 1) / kBM));
  hipLaunchKernelGGL(nf4_gemm_kernel<true>, grid, dim3(256), 0, st, w, dy, m, w.k, w.n, dhs, at,
                     static_cast<int64_t>(rpad), rpad, rpad, dx, nf4_table());
  return hipGetLastError();
}

}  // namespace qlora
