// Rank-r side kernels of the LoRA path.
//
// "LoRA y QLoRA en Profundidad", section "La Idea Central": the adapter adds
// (alpha / r) * B @ A with A r x d_in and B d_out x r. With H = X A^T the
// forward adds s H B^T; the backward (Ultralytics glossary "QLoRA", "Come
// funziona QLoRA": gradients only for the two LoRA matrices) needs
// dH = s dY B, dA = dH^T X and dB = s dY^T H.
//
// These are thin (r <= 128 columns) and are bounded by one pass over X or dY.
#include "internal.h"
#include "mfma.h"
#include "nf4_lut.h"

namespace qlora {
namespace {

// out[m][j] = scale * sum_q P[m][q] Q[j][q]. One workgroup (WAVES waves) per
// 16 rows of P and one contraction split; waves take interleaved 32-wide
// chunks of q and are summed in a fixed order through LDS. RT = rpad / 16
// output column tiles (0: only the reordered copy of P is produced). Narrow
// ranks get more waves per row block, so that each wave makes only one or
// two trips to memory.
template <int RT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void skinny_kernel(const uint16_t* __restrict__ P, const uint16_t* __restrict__ Q,
                                                     int64_t M, int64_t qn, int r, int rpad, float scale,
                                                     float scale2, float* __restrict__ out_f32,
                                                     uint16_t* __restrict__ out_bf16, int splits) {
  constexpr int kRT = RT > 0 ? RT : 1;
  __shared__ f32x4 red[WAVES][kRT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, i = lane & 15, g = lane >> 4;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int split = blockIdx.y;
  const int64_t m = m0 + i;
  const int64_t nchunks = (qn + 31) / 32;
  const int64_t per = (nchunks + splits - 1) / splits;
  const int64_t c_begin = split * per;
  const int64_t c_end = (c_begin + per < nchunks) ? c_begin + per : nchunks;

  f32x4 acc[kRT];
#pragma unroll
  for (int t = 0; t < kRT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // U chunks per wave per trip. Loads are unconditional from clamped
  // addresses (a guarded load makes the compiler wait for all outstanding
  // loads); chunks past the split and ranks past r are zeroed at the operand.
  constexpr int U = (RT <= 2) ? 4 : (RT <= 4 ? 8 : 4);
  const int64_t m_c = m < M ? m : M - 1;
  for (int64_t c0 = c_begin + wave; c0 < c_end; c0 += WAVES * U) {
    u32x4 a[U], b[U][kRT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t q = (c0 + WAVES * u) * 32 + 8 * g;
      const int64_t q_c = q < qn - 8 ? q : qn - 8;
      a[u] = ld16(P + m_c * qn + q_c);
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int j = 16 * t + i;
        b[u][t] = ld16(Q + static_cast<int64_t>(j < r ? j : r - 1) * qn + q_c);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t q = (c0 + WAVES * u) * 32 + 8 * g;
      const bool qvalid = (c0 + WAVES * u < c_end) && q < qn;  // qn % 8 == 0: a valid run is whole
      const u32x4 av = qvalid ? a[u] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        const int j = 16 * t + i;
        acc[t] = mfma_16x16x32(av, j < r ? b[u][t] : u32x4{0, 0, 0, 0}, acc[t]);
      }
    }
  }
  if (RT == 0) return;

#pragma unroll
  for (int t = 0; t < RT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (tid >= 256) return;
  const int l2 = tid & 63, v = tid >> 6;
  const int64_t mo = m0 + 4 * (l2 >> 4) + v;
  if (mo >= M) return;
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int j = 16 * t + (l2 & 15);
    float sum = 0.0f;
#pragma unroll
    for (int wv = 0; wv < WAVES; ++wv) sum += red[wv][t][l2][v];
    if (splits > 1) {
      if (j < r) out_f32[(split * M + mo) * r + j] = sum;
    } else {
      const float val = scale * sum;
      if (out_f32 != nullptr && j < r) out_f32[mo * r + j] = val;
      if (out_bf16 != nullptr && j < rpad) out_bf16[mo * rpad + j] = f32_to_bf16_rne(scale2 * val);
    }
  }
}

// Second half of the split prefill projection: out_f32 = scale * sum of the
// split partials (summed in split order), out_bf16 = bf16(scale2 * that),
// zero-padded from r to rpad columns.
__global__ void skinny_final_kernel(const float* __restrict__ part, int64_t M, int r, int rpad, int splits,
                                    float scale, float scale2, float* __restrict__ out_f32,
                                    uint16_t* __restrict__ out_bf16) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= M * rpad) return;
  const int64_t mo = idx / rpad;
  const int j = static_cast<int>(idx % rpad);
  float sum = 0.0f;
  if (j < r)
    for (int sp = 0; sp < splits; ++sp) sum += part[(static_cast<int64_t>(sp) * M + mo) * r + j];
  const float val = scale * sum;
  if (out_f32 != nullptr && j < r) out_f32[mo * r + j] = val;
  if (out_bf16 != nullptr) out_bf16[idx] = f32_to_bf16_rne(scale2 * val);
}

// at (k x rpad) = A^T zero-padded; bt (rpad x n) = B^T zero-padded.
__global__ void lora_transpose_kernel(const uint16_t* __restrict__ a, const uint16_t* __restrict__ b, int64_t n,
                                      int64_t k, int r, int rpad, uint16_t* __restrict__ at,
                                      uint16_t* __restrict__ bt) {
  int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t na = k * rpad;
  if (idx < na) {
    const int64_t kk = idx / rpad;
    const int j = static_cast<int>(idx % rpad);
    at[idx] = (j < r) ? a[static_cast<int64_t>(j) * k + kk] : uint16_t(0);
    return;
  }
  idx -= na;
  if (idx < static_cast<int64_t>(rpad) * n) {
    const int j = static_cast<int>(idx / n);
    const int64_t nn = idx % n;
    bt[idx] = (j < r) ? b[nn * r + j] : uint16_t(0);
  }
}

// part[s][j][c] = sum over rows m of split s of U[m][j] * V[m][c] (float32
// U, bf16 V). A workgroup (16 waves) owns 128 columns (two per lane) and 16
// ranks; its waves take interleaved rows of the split, 8 rows per trip with
// all V loads issued first, and are summed in LDS in a fixed order. The
// 16-rank slice of a U row is the same for every lane, so it is fetched with
// scalar loads. kFull: r is a multiple of 16 (no rank tail).
template <bool kFull>
__global__ __launch_bounds__(1024) void rank_partial_kernel(const float* __restrict__ U, const uint16_t* __restrict__ V,
                                                            int64_t M, int64_t cn, int r, int splits,
                                                            float* __restrict__ part) {
  constexpr int kWaves = 16, kRows = kFull ? 8 : 2;
  __shared__ float red[kWaves][16][128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 128 + 2 * lane;
  const int j0 = blockIdx.y * 16;
  const int s = blockIdx.z;
  const int64_t per = (M + splits - 1) / splits;
  const int64_t mb = s * per;
  const int64_t me = (mb + per < M) ? mb + per : M;
  const bool cvalid = c < cn;
  float acc[16][2];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) acc[jj][0] = acc[jj][1] = 0.0f;
  const int64_t c_c = cvalid ? c : cn - 2;  // columns past cn are computed but never stored
  for (int64_t m0 = mb + wave; m0 < me; m0 += kWaves * kRows) {
    uint32_t v2[kRows];
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int64_t m = m0 + kWaves * u;
      v2[u] = *reinterpret_cast<const uint32_t*>(V + (m < me ? m : me - 1) * cn + c_c);
    }
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int64_t m = m0 + kWaves * u;
      if (m >= me) break;  // uniform across the wave
      const float v0 = __uint_as_float(v2[u] << 16), v1 = __uint_as_float(v2[u] & 0xFFFF0000u);
      float uu[16];
      if (kFull) {
        const f32x4* up = reinterpret_cast<const f32x4*>(U + __builtin_amdgcn_readfirstlane(static_cast<int>(m)) *
                                                                 static_cast<int64_t>(r) + j0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 t = up[q];
          uu[4 * q] = t[0];
          uu[4 * q + 1] = t[1];
          uu[4 * q + 2] = t[2];
          uu[4 * q + 3] = t[3];
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) uu[jj] = U[m * r + ((j0 + jj < r) ? j0 + jj : r - 1)];  // tail never stored
      }
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        acc[jj][0] = fmaf(uu[jj], v0, acc[jj][0]);
        acc[jj][1] = fmaf(uu[jj], v1, acc[jj][1]);
      }
    }
  }
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    red[wave][jj][2 * lane] = acc[jj][0];
    red[wave][jj][2 * lane + 1] = acc[jj][1];
  }
  __syncthreads();
  for (int idx = tid; idx < 16 * 128; idx += kWaves * 64) {
    const int jj = idx >> 7, cc = idx & 127;
    const int64_t col = static_cast<int64_t>(blockIdx.x) * 128 + cc;
    if (j0 + jj < r && col < cn) {
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < kWaves; ++wv) sum += red[wv][jj][cc];
      part[(static_cast<int64_t>(s) * r + j0 + jj) * cn + col] = sum;
    }
  }
}

// out = scale * sum_s part[s], summed in split order.
__global__ void rank_final_kernel(const float* __restrict__ part, int64_t cn, int r, int splits, float scale,
                                  float* __restrict__ out, int c_major) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(r) * cn) return;
  int64_t j, c;
  if (c_major) {
    c = idx / r;
    j = idx % r;
  } else {
    j = idx / cn;
    c = idx % cn;
  }
  float sum = 0.0f;
  for (int s = 0; s < splits; ++s) sum += part[(static_cast<int64_t>(s) * r + j) * cn + c];
  out[idx] = scale * sum;
}

template <int RT>
void launch_skinny_rt(dim3 grid, hipStream_t st, const uint16_t* P, const uint16_t* Q, int64_t m, int64_t qn, int r,
                      int rpad, float scale, float scale2, float* out_f32, uint16_t* out_bf16, int splits) {
  constexpr int kWaves = (RT <= 2) ? 16 : (RT <= 4 ? 8 : 4);
  hipLaunchKernelGGL((skinny_kernel<RT, kWaves>), grid, dim3(kWaves * 64), 0, st, P, Q, m, qn, r, rpad, scale, scale2,
                     out_f32, out_bf16, splits);
}

}  // namespace

int rank_reduce_splits(int64_t m, int64_t n, int64_t k, int r) {
  // enough workgroups for two per CU on the narrower of the two reductions
  // (dA over k columns, dB over n columns), with at least 64 rows per split
  const int64_t cn = n < k ? n : k;
  const int64_t wg = ((cn + 127) / 128) * ((r + 15) / 16);
  if (wg <= 0) return 1;  // r = 0: no reduction
  int64_t s = (512 + wg - 1) / wg;
  const int64_t by_rows = m / 64;
  if (s > by_rows) s = by_rows;
  if (s > 32) s = 32;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

int skinny_prefill_splits(int64_t m, int64_t qn) {
  // about two workgroups per CU, at least 256 contraction elements per split
  const int64_t tiles = (m + 15) / 16;
  int64_t s = (512 + tiles - 1) / tiles;
  if (s > qn / 256) s = qn / 256;
  if (s > 8) s = 8;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

hipError_t launch_skinny_prefill(const uint16_t* P, const uint16_t* Q, int64_t m, int64_t qn, int r, int rpad,
                                 float scale, float scale2, float* part, float* out_f32, uint16_t* out_bf16,
                                 hipStream_t st) {
  const int splits = skinny_prefill_splits(m, qn);
  hipError_t e = launch_skinny(P, Q, m, qn, r, rpad, 1.0f, 1.0f, part, nullptr, splits, st);
  if (e != hipSuccess) return e;
  const int64_t total = m * rpad;
  hipLaunchKernelGGL(skinny_final_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st, part, m,
                     r, rpad, splits, scale, scale2, out_f32, out_bf16);
  return hipGetLastError();
}

int skinny_splits(int64_t m, int64_t qn) {
  if (m > 16) return 1;
  const int64_t s = (qn + 511) / 512;  // ~512 contraction elements per workgroup
  return static_cast<int>(s < 1 ? 1 : (s > 64 ? 64 : s));
}

hipError_t launch_skinny(const uint16_t* P, const uint16_t* Q, int64_t m, int64_t qn, int r, int rpad, float scale,
                         float scale2, float* out_f32, uint16_t* out_bf16, int splits, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((m + 15) / 16), static_cast<unsigned>(splits));
  switch (rpad / 16) {
    case 0: launch_skinny_rt<0>(grid, s, P, Q, m, qn, r, rpad, scale, scale2, out_f32, out_bf16, splits); break;
    case 2: launch_skinny_rt<2>(grid, s, P, Q, m, qn, r, rpad, scale, scale2, out_f32, out_bf16, splits); break;
    case 4: launch_skinny_rt<4>(grid, s, P, Q, m, qn, r, rpad, scale, scale2, out_f32, out_bf16, splits); break;
    case 6: launch_skinny_rt<6>(grid, s, P, Q, m, qn, r, rpad, scale, scale2, out_f32, out_bf16, splits); break;
    case 8: launch_skinny_rt<8>(grid, s, P, Q, m, qn, r, rpad, scale, scale2, out_f32, out_bf16, splits); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lora_transpose(const uint16_t* a, const uint16_t* b, int64_t n, int64_t k, int r, int rpad,
                                 uint16_t* at, uint16_t* bt, hipStream_t st) {
  const int64_t total = (k + n) * rpad;
  hipLaunchKernelGGL(lora_transpose_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st, a, b,
                     n, k, r, rpad, at, bt);
  return hipGetLastError();
}

hipError_t launch_rank_reduce(const float* U, const uint16_t* V, int64_t m, int64_t cn, int r, float scale,
                              int splits, float* part, float* out, int c_major, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((cn + 127) / 128), static_cast<unsigned>((r + 15) / 16),
                  static_cast<unsigned>(splits));
  if (r % 16 == 0) {
    hipLaunchKernelGGL(rank_partial_kernel<true>, grid, dim3(1024), 0, st, U, V, m, cn, r, splits, part);
  } else {
    hipLaunchKernelGGL(rank_partial_kernel<false>, grid, dim3(1024), 0, st, U, V, m, cn, r, splits, part);
  }
  const int64_t total = static_cast<int64_t>(r) * cn;
  hipLaunchKernelGGL(rank_final_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st, part, cn,
                     r, splits, scale, out, c_major);
  return hipGetLastError();
}

}  // namespace qlora
