// NF4 quantize (with double quantization of the scales) and dequantize.
//
// Ultralytics glossary "QLoRA", section "Come funziona QLoRA": every weight is
// a 4-bit code into 16 normal-quantile levels with one absmax scale per block
// of 64; the per-block scales are in turn quantized to 8 bit in blocks of 256.
// "Modulo 4: QLoRA", 4.3 b): weights first, then the scale constants.
//
// Both kernels stream HBM once and are bandwidth bound. This translation unit
// is built with -ffp-contract=off and IEEE float32 division and denormals,
// because codes, scale codes and dequantized values are bit-exact outputs.
#include "internal.h"
#include "nf4_lut.h"

namespace qlora {
namespace {

constexpr int kBlock = 64;
constexpr int kGroup = 256;

// U_k = fl32(k / 255): correctly rounded float32 division.
__device__ __forceinline__ float u8_level(uint32_t k) { return static_cast<float>(k) / 255.0f; }

// Nearest U_k to x2 in [0, 1], lowest k on ties. The fp32 argmin lies within
// one step of rint(255 x2), so three candidates suffice.
__device__ __forceinline__ uint32_t nearest_u8(float x2) {
  int k0 = static_cast<int>(rintf(x2 * 255.0f));
  k0 = min(max(k0, 0), 255);
  const int lo = max(k0 - 1, 0), hi = min(k0 + 1, 255);
  uint32_t best = lo;
  float bd = fabsf(x2 - u8_level(lo));
  for (int k = lo + 1; k <= hi; ++k) {
    const float d = fabsf(x2 - u8_level(k));
    if (d < bd) {
      bd = d;
      best = k;
    }
  }
  return best;
}

// Nearest E_c (the float-like code, nf4_lut.h) to x2 in [0, 1], lowest c on
// ties. c0, the largest code with E_c0 <= x2, comes from x2's bits: below
// 2^-14 it is floor(x2 2^18) (exact scaling), above it the exponent and the
// top 4 mantissa bits; the nearest is c0 or c0 + 1 (farther codes are at
// least one spacing away, about x2 / 16). x2 = 1 gives c0 = 240, E = 1.
__device__ __forceinline__ uint32_t nearest_e4m4(float x2) {
  uint32_t c0;
  if (x2 < 6.103515625e-05f) {  // 2^-14
    c0 = static_cast<uint32_t>(x2 * 262144.0f);
  } else {
    const uint32_t b = __float_as_uint(x2);
    c0 = (((b >> 23) - 112u) << 4) | ((b >> 19) & 15u);
  }
  if (c0 >= 240u) return 240u;
  const float d_lo = x2 - e4m4_unit(c0);
  const float d_hi = e4m4_unit(c0 + 1) - x2;
  return (d_hi < d_lo) ? c0 + 1 : c0;
}

// One workgroup (512 threads) per double-quantization group of 256 blocks.
// Wave w owns blocks [32w, 32w + 32) of the group, 8 at a time: 8 lanes per
// block, 8 consecutive elements per lane (two 16-byte loads), so a wave reads
// 2 KB contiguous per step. (512 threads measured 2-10% faster than 256 or
// 1024 at the 7B shapes.) The block absmax is an 8-lane max-reduction; the
// codes of a lane's 8 elements form one 32-bit store. Block maxima go to LDS
// and the group maximum M_g is a workgroup reduction.
//
// Per weight, x = fl32(w / a_b) (correctly rounded) is formed as t = 16 x by
// quotient16 from the block's fl32(16 / a_b), and its code is read from the
// bucket table (EncodeTable) in LDS: one 8-byte read of (16 U, base) and one
// compare. Blocks whose absmax lies outside [2^-60, 2^60] take the IEEE
// division instead (same result, more instructions).
constexpr int kQThreads = 512;
constexpr int kQWaves = kQThreads / 64;
constexpr int kQSteps = kGroup / kQWaves / 8;  // 8-block steps per wave

__global__ __launch_bounds__(kQThreads) void nf4_quantize_kernel(const float* __restrict__ w, int64_t numel, int dq,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scale_codes,
                                                           float* __restrict__ group_scale,
                                                           float* __restrict__ absmax_out, EncodeTable E) {
  __shared__ u32x2 enc[33];
  __shared__ float blk_max[kGroup];
  __shared__ float wave_max[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 33) enc[tid] = u32x2{__float_as_uint(E.thr16[tid]), E.base[tid]};
  __syncthreads();

  const int64_t nblocks = (numel + kBlock - 1) / kBlock;
  const int64_t g = blockIdx.x;
  const int sub = lane >> 3, part = lane & 7;

  // Vector loads are unconditional from clamped addresses (a guarded load
  // makes the compiler wait for all outstanding loads); only the lanes that
  // straddle the end of the array redo theirs with element loads. Plain
  // loads: with the nontemporal hint the kernel ran 4-7% slower.
  float v[kQSteps][8];
  const int64_t last8 = numel >= 8 ? numel - 8 : 0;
#pragma unroll
  for (int it = 0; it < kQSteps; ++it) {
    const int64_t b = g * kGroup + wave * (8 * kQSteps) + it * 8 + sub;
    const int64_t e0 = b * kBlock + part * 8;
    if (numel >= 8) {
      const f32x4* p = reinterpret_cast<const f32x4*>(w + (e0 < last8 ? e0 : (last8 & ~INT64_C(3))));
      const f32x4 a = p[0];
      const f32x4 c = p[1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[it][j] = a[j];
        v[it][4 + j] = c[j];
      }
    }
  }
#pragma unroll
  for (int it = 0; it < kQSteps; ++it) {
    const int64_t b = g * kGroup + wave * (8 * kQSteps) + it * 8 + sub;
    const int64_t e0 = b * kBlock + part * 8;
    if (e0 + 8 > numel) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[it][j] = (e0 + j < numel) ? w[e0 + j] : 0.0f;
    }
  }

#pragma unroll
  for (int it = 0; it < kQSteps; ++it) {
    const int bl = wave * (8 * kQSteps) + it * 8 + sub;
    const int64_t b = g * kGroup + bl;
    const int64_t e0 = b * kBlock + part * 8;
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[it][j]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    // t = 16 x for the lane's 8 weights (an all-zero block: every x = 0)
    float t[8];
    if (m >= 0x1p-60f && m <= 0x1p60f) {
      const float y16 = 16.0f / m, m16 = m * 0.0625f;
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = quotient16(v[it][j], y16, m16);
    } else {
      const float mm = m > 0.0f ? m : 1.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = 16.0f * (v[it][j] / mm);
    }
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x2 e = enc[encode_bucket(t[j])];
      packed |= (e[1] + (t[j] >= __uint_as_float(e[0]) ? 1u : 0u)) << (4 * j);
    }
    if (e0 + 8 <= numel) {
      *reinterpret_cast<uint32_t*>(codes + e0 / 2) = packed;
    } else if (e0 < numel) {
      const int64_t nvalid = numel - e0;  // 1..7 elements
      const int nbytes = static_cast<int>((nvalid + 1) / 2);
      const uint32_t keep = (nvalid >= 8) ? 0xFFFFFFFFu : ((1u << (4 * nvalid)) - 1u);
      packed &= keep;  // an odd count leaves the last high nibble 0
      for (int i = 0; i < nbytes; ++i) codes[e0 / 2 + i] = static_cast<uint8_t>(packed >> (8 * i));
    }
    if (part == 0) blk_max[bl] = (b < nblocks) ? m : 0.0f;
  }
  __syncthreads();

  // the group's 256 block maxima: threads 0..255, one each (waves 0..3)
  const int tq = tid & (kGroup - 1);
  const int64_t b = g * kGroup + tq;
  const float a = blk_max[tq];
  float mg = a;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mg = fmaxf(mg, __shfl_xor(mg, off));
  if (lane == 0 && wave < 4) wave_max[wave] = mg;
  __syncthreads();
  mg = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));

  if (tid < kGroup && b < nblocks) {
    if (absmax_out != nullptr) absmax_out[b] = a;
    if (dq) {
      const float x2 = (mg > 0.0f) ? a / mg : 0.0f;
      scale_codes[b] = static_cast<uint8_t>(dq == 2 ? nearest_e4m4(x2) : nearest_u8(x2));
    }
  }
  if (dq && tid == 0) group_scale[g] = mg;
}

// Dequantize: each lane turns one 32-bit word of codes (8 weights) into 8
// outputs per step; a wave covers 256 contiguous code bytes -> 1 KB of bf16
// (or 2 KB of fp32) contiguous. Four steps per lane, all loads first.
// kOut: 0 = bf16, 1 = float32, 2 = IEEE half (both 16-bit forms round the
// float32 value to nearest even).
template <int kOut, bool kDQ>
__global__ __launch_bounds__(256) void nf4_dequantize_kernel(PackedW w, void* __restrict__ out, Levels L) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = L.v[threadIdx.x];
  __syncthreads();
  const int64_t numel = w.n * w.k;
  const int64_t nwords = (numel + 7) / 8;  // 8 codes per 32-bit word
  const int64_t nbytes_total = (numel + 1) / 2;
  const int64_t nfull = nbytes_total / 4;  // words lying wholly inside the buffer
  const int64_t base = static_cast<int64_t>(blockIdx.x) * 1024 + threadIdx.x;
  // Whole words: unconditional loads from clamped addresses (a guarded load
  // makes the compiler wait for all outstanding loads). The one partial
  // word at the end is assembled from bytes by the lane that owns it.
  uint32_t cw[4] = {0, 0, 0, 0};
  if (nfull > 0) {  // uniform
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t q = base + j * 256;
      cw[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(w.codes) + (q < nfull - 1 ? q : nfull - 1));
    }
  }
  // per-word block scales, also unconditional (clamped block index)
  const int64_t nb = (numel + kBlock - 1) / kBlock;
  uint32_t sc8[4];
  float sc32[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t bq = (base + j * 256) * 8 / kBlock;
    const int64_t bc = bq < nb - 1 ? bq : nb - 1;
    if (kDQ) {
      sc8[j] = w.scale_codes[bc];
      sc32[j] = w.group_scale[bc / kGroup];
    } else {
      sc8[j] = 0;
      sc32[j] = w.absmax[bc];
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t q = base + j * 256;
    if (q >= nfull && q < nwords) {
      uint32_t word = 0;
      for (int i = 0; i < 4; ++i)
        if (q * 4 + i < nbytes_total) word |= static_cast<uint32_t>(w.codes[q * 4 + i]) << (8 * i);
      cw[j] = word;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t q = base + j * 256;
    if (q >= nwords) continue;
    const int64_t e0 = q * 8;
    const float s = kDQ ? (w.dq == 2 ? e4m4_unit(sc8[j]) : u8_level(sc8[j])) * sc32[j] : sc32[j];
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = lv[(cw[j] >> (4 * i)) & 0xF] * s;
    if (e0 + 8 <= numel) {
      if (kOut == 1) {
        f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(out) + e0);
        __builtin_nontemporal_store(f32x4{f[0], f[1], f[2], f[3]}, o);
        __builtin_nontemporal_store(f32x4{f[4], f[5], f[6], f[7]}, o + 1);
      } else if (kOut == 2) {
        const u32x4 o = {cvt_16x2<true>(f[0], f[1]), cvt_16x2<true>(f[2], f[3]), cvt_16x2<true>(f[4], f[5]),
                         cvt_16x2<true>(f[6], f[7])};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + e0));
      } else {
        const u32x4 o = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                         pack_bf16x2(f[6], f[7])};
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + e0));
      }
    } else {
      for (int i = 0; i < 8; ++i) {
        if (e0 + i >= numel) break;
        if (kOut == 1) {
          static_cast<float*>(out)[e0 + i] = f[i];
        } else if (kOut == 2) {
          static_cast<uint16_t*>(out)[e0 + i] = static_cast<uint16_t>(cvt_16x2<true>(f[i], 0.0f) & 0xFFFFu);
        } else {
          static_cast<uint16_t*>(out)[e0 + i] = static_cast<uint16_t>(bf16_rne_hi(f[i]) >> 16);
        }
      }
    }
  }
}

__global__ void fill_zero_kernel(float* p, int64_t count) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0.0f;
}

}  // namespace

hipError_t launch_quantize(const float* w, int64_t numel, int dq, int codebook, uint8_t* codes, uint8_t* scale_codes,
                           float* group_scale, float* absmax, hipStream_t s) {
  const int64_t nblocks = (numel + kBlock - 1) / kBlock;
  const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
  hipLaunchKernelGGL(nf4_quantize_kernel, dim3(static_cast<unsigned>(ngroups)), dim3(kQThreads), 0, s, w, numel, dq,
                     codes, scale_codes, group_scale, absmax, encode_table(codebook));
  return hipGetLastError();
}

hipError_t launch_dequantize(const PackedW& w, int out_kind, void* out, hipStream_t s) {
  const int64_t numel = w.n * w.k;
  const int64_t nwords = (numel + 7) / 8;
  const unsigned grid = static_cast<unsigned>((nwords + 1023) / 1024);
  auto kern = out_kind == 1   ? (w.dq ? nf4_dequantize_kernel<1, true> : nf4_dequantize_kernel<1, false>)
              : out_kind == 2 ? (w.dq ? nf4_dequantize_kernel<2, true> : nf4_dequantize_kernel<2, false>)
                              : (w.dq ? nf4_dequantize_kernel<0, true> : nf4_dequantize_kernel<0, false>);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, w, out, codebook_table(w.codebook));
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t st) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256), 0, st, p,
                     count);
  return hipGetLastError();
}

}  // namespace qlora
