// Dropout on the adapter input with an explicit keep mask.
//
// "LoRA y QLoRA en Profundidad", section "Dropout (lora_dropout)": during
// training the LoRA path randomly zeroes elements. The layer drops the
// adapter's input, H = D(X) A^T with D(X) = X * keep / (1 - p), and leaves
// the frozen path X W^T alone; by the chain rule the backward adds the
// adapter's share of dX only where the input was kept.
//
// Two elementwise kernels, both bound by HBM: the masked copy of X (the
// 1 / (1 - p) factor goes into the projection's scale, so the copy is exact)
// and the masked rank-r update of dX after the frozen-weight GEMM. A third
// draws keep masks with the counter-based generator Philox4x64-10 (J. K.
// Salmon, M. A. Moraes, R. O. Dror and D. E. Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC 2011), so a mask can be made on the device and
// reproduced anywhere from (seed, offset).
#include "internal.h"
#include "mfma.h"
#include "nf4_lut.h"

namespace qlora {
namespace {

constexpr int kRows = 16;   // rows per workgroup of the dX update: 4 per wave
constexpr int kCols = 512;  // columns per workgroup: 8 per lane

// Ten Philox rounds on the counter c under the key (k0, k1): each round takes
// the two 64 x 64 -> 128-bit products of the paper's multipliers with c0 and
// c2, mixes their high halves with c1, c3 and the key, and advances the key
// by the paper's two Weyl constants. Integer arithmetic only.
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t hi0 = __umul64hi(kM0, c[0]), lo0 = kM0 * c[0];
    const uint64_t hi1 = __umul64hi(kM1, c[2]), lo1 = kM1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += kW0;
    k1 += kW1;
  }
}

// keep[16 t + j] for thread t: block block0 + t under the key (seed, 0);
// chunk j is bits 16 (j % 4) .. of word j / 4, dropped when float(chunk) <
// thr = 65536 p. One 16-byte store per block (byte stores for the tail).
__global__ __launch_bounds__(256) void dropout_mask_kernel(uint64_t seed, uint64_t block0, int64_t count, float thr,
                                                           uint8_t* __restrict__ keep) {
  const int64_t nblocks = (count + 15) / 16;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; t < nblocks; t += stride) {
    uint64_t c[4] = {block0 + static_cast<uint64_t>(t), 0, 0, 0};
    philox4x64_10(c, seed, 0);
    uint32_t out[4];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      uint32_t v = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float u = static_cast<float>(static_cast<uint32_t>((c[wd] >> (16 * q)) & 0xFFFFu));
        v |= (u < thr ? 0u : 1u) << (8 * q);
      }
      out[wd] = v;
    }
    const int64_t e0 = 16 * t;
    if (e0 + 16 <= count) {
      *reinterpret_cast<u32x4*>(keep + e0) = u32x4{out[0], out[1], out[2], out[3]};
    } else {
      for (int j = 0; e0 + j < count; ++j) keep[e0 + j] = static_cast<uint8_t>(out[j >> 2] >> (8 * (j & 3)));
    }
  }
}

// 0xFFFF for each of the two bf16 halves whose keep byte is non-zero.
__device__ __forceinline__ uint32_t keep_halves(uint32_t word, int pair) {
  const uint32_t b0 = (word >> (16 * pair)) & 0xFFu, b1 = (word >> (16 * pair + 8)) & 0xFFu;
  return (b0 ? 0x0000FFFFu : 0u) | (b1 ? 0xFFFF0000u : 0u);
}

// xm = x where keep != 0, else +0. Eight elements per lane and step (16 bytes
// of x, 8 bytes of keep); count8 = m k / 8.
__global__ __launch_bounds__(256) void mask_input_kernel(const uint16_t* __restrict__ x,
                                                         const uint8_t* __restrict__ keep, int64_t count8,
                                                         uint16_t* __restrict__ xm) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < count8; i += stride) {
    const u32x4 v = reinterpret_cast<const u32x4*>(x)[i];
    const u32x2 kb = reinterpret_cast<const u32x2*>(keep)[i];
    const u32x4 o = {v[0] & keep_halves(kb[0], 0), v[1] & keep_halves(kb[0], 1), v[2] & keep_halves(kb[1], 0),
                     v[3] & keep_halves(kb[1], 1)};
    reinterpret_cast<u32x4*>(xm)[i] = o;
  }
}

// dx[i][q] = bf16(dx[i][q] + (keep[i][q] ? sum_j dh[i][j] a[j][q] : 0)) for a
// 16 x 512 tile: dh's 16 rows in LDS, each lane 8 columns of 4 rows, A rows
// read from L2 (16 bytes per rank step). k % 64 == 0, so a lane's 8 columns
// are all inside the row or all past its end.
template <bool kF16>
__global__ __launch_bounds__(256) void masked_lora_add_kernel(uint16_t* __restrict__ dx,
                                                              const uint8_t* __restrict__ keep,
                                                              const float* __restrict__ dh,
                                                              const uint16_t* __restrict__ a, int64_t m, int64_t k,
                                                              int r) {
  __shared__ float hs[kRows][QLORA_MAX_RANK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tiles_c = (k + kCols - 1) / kCols;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) / tiles_c) * kRows;
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) % tiles_c) * kCols;
  for (int i = tid; i < kRows * r; i += 256) {
    const int rr = i / r, j = i - rr * r;
    hs[rr][j] = (row0 + rr < m) ? dh[(row0 + rr) * r + j] : 0.0f;
  }
  __syncthreads();
  const int64_t q0 = col0 + 8 * lane;
  if (q0 >= k) return;  // no barrier follows

  // this lane's dX and keep bytes of its 4 rows, loaded before the rank
  // loop so that their trip to memory overlaps it (rows past m: not loaded)
  u32x4 gx[4];
  u32x2 kx[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int64_t i = row0 + 4 * wave + rr;
    gx[rr] = u32x4{0, 0, 0, 0};
    kx[rr] = u32x2{0, 0};
    if (i < m) {
      const int64_t e0 = i * k + q0;
      gx[rr] = *reinterpret_cast<const u32x4*>(dx + e0);
      kx[rr] = *reinterpret_cast<const u32x2*>(keep + e0);
    }
  }

  float d[4][8];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
#pragma unroll
    for (int c = 0; c < 8; ++c) d[rr][c] = 0.0f;
  const uint16_t* acol = a + q0;
#pragma unroll 4
  for (int j = 0; j < r; ++j) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(acol + static_cast<int64_t>(j) * k);
    float av[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      av[2 * c] = lo16<kF16>(v[c]);
      av[2 * c + 1] = hi16<kF16>(v[c]);
    }
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float hj = hs[4 * wave + rr][j];
#pragma unroll
      for (int c = 0; c < 8; ++c) d[rr][c] = fmaf(hj, av[c], d[rr][c]);
    }
  }
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int64_t i = row0 + 4 * wave + rr;
    if (i >= m) break;
    const int64_t e0 = i * k + q0;
    u32x4* dst = reinterpret_cast<u32x4*>(dx + e0);
    const u32x4 g = gx[rr];
    const u32x2 kb = kx[rr];
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t kw = kb[c >> 1] >> (16 * (c & 1));
      const float lo = lo16<kF16>(g[c]) + ((kw & 0xFFu) ? d[rr][2 * c] : 0.0f);
      const float hi = hi16<kF16>(g[c]) + ((kw & 0xFF00u) ? d[rr][2 * c + 1] : 0.0f);
      o[c] = cvt_16x2<kF16>(lo, hi);
    }
    *dst = o;
  }
}

}  // namespace

hipError_t launch_mask_input(const uint16_t* x, const uint8_t* keep, int64_t count, uint16_t* xm, hipStream_t st) {
  const int64_t count8 = count / 8;
  int64_t blocks = (count8 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(mask_input_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, x, keep, count8, xm);
  return hipGetLastError();
}

hipError_t launch_dropout_mask(uint64_t seed, uint64_t block0, int64_t count, float thr, uint8_t* keep,
                               hipStream_t st) {
  int64_t blocks = ((count + 15) / 16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, seed, block0, count,
                     thr, keep);
  return hipGetLastError();
}

hipError_t launch_masked_lora_add(uint16_t* dx, const uint8_t* keep, const float* dh, const uint16_t* a, int64_t m,
                                  int64_t k, int r, hipStream_t st, bool f16) {
  const int64_t tiles = ((m + kRows - 1) / kRows) * ((k + kCols - 1) / kCols);
  if (f16) {
    hipLaunchKernelGGL(masked_lora_add_kernel<true>, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, st, dx, keep,
                       dh, a, m, k, r);
  } else {
    hipLaunchKernelGGL(masked_lora_add_kernel<false>, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, st, dx, keep,
                       dh, a, m, k, r);
  }
  return hipGetLastError();
}

}  // namespace qlora
