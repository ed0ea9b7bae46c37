// Merging a trained adapter into the weight, taking it back out, and
// re-quantizing the merged weight.
//
// "LoRA y QLoRA en Profundidad", "La Idea Central: Descomposicion de Bajo
// Rango": for inference the adapter is folded into the weight, W + (alpha/r)
// B A. Ultralytics glossary "QLoRA", "QLoRA e metodi correlati" and
// "Compromessi": the merge happens on the weight dequantized to 16 bit, and
// the merged model is quantized again for distribution.
//
// Element (p, q) of the update is t = fl32(s d) with d the float32 sum of
// b_pj a_jq over j = 0 .. r-1 in ascending order (bf16 products are exact in
// float32); the merged value is fl32(w16 + t) and the unmerged one fl32(W' - t).
// That order is part of the contract (the results are bit-exact), so this
// unit is built without floating-point contraction. The work is an
// elementwise pass with a rank-r inner product per element: bound by HBM
// (packed codes in, 2 or 4 bytes per element out) for the ranks the layer
// uses, by vector fp32 issue only near r = 128.
#include "internal.h"
#include "nf4_lut.h"

namespace qlora {
namespace {

constexpr int kRows = 16;   // rows per workgroup: 4 per wave
constexpr int kCols = 512;  // columns per workgroup: 8 per lane
constexpr int kBlock = 64;
constexpr int kGroup = 256;

enum SrcKind { kPacked = 0, kDenseBf16 = 1, kDenseF32 = 2 };

struct MergeArgs {
  PackedW w;           // kPacked: the NF4 weight
  const void* dense;   // kDense*: n x k values (may alias out)
  const uint16_t* a;   // r x k bf16
  const uint16_t* b;   // n x r bf16
  int64_t n, k;
  int r;
  float s;             // fl32(alpha / r); 0 when r = 0
  void* out;           // n x k, float32 or bf16
};

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// One workgroup per 16 x 512 tile. The tile's 16 B rows (float32) sit in LDS;
// each lane owns 8 consecutive columns of 4 rows and walks j upward, reading
// A[j][q0 .. q0+7] (16 bytes, from L2: A is at most 1 MB) and broadcasting
// B[p][j] from LDS. k % 8 == 0 (k % 64 == 0 for packed sources), so a lane's
// 8 columns are all inside the row or all past its end, and inside one
// 64-weight block.
template <int kSrc, bool kSub, bool kOutF32>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs g, Levels L) {
  __shared__ float lv[16];
  __shared__ float bs[kRows][QLORA_MAX_RANK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tiles_c = (g.k + kCols - 1) / kCols;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) / tiles_c) * kRows;
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) % tiles_c) * kCols;
  if (tid < 16) lv[tid] = L.v[tid];
  for (int i = tid; i < kRows * g.r; i += 256) {
    const int rr = i / g.r, j = i - rr * g.r;
    const int64_t p = row0 + rr;
    bs[rr][j] = (p < g.n) ? __uint_as_float(static_cast<uint32_t>(g.b[p * g.r + j]) << 16) : 0.0f;
  }
  __syncthreads();

  const int64_t q0 = col0 + 8 * lane;
  if (q0 >= g.k) return;  // no barrier follows
  float d[4][8];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr)
#pragma unroll
    for (int c = 0; c < 8; ++c) d[rr][c] = 0.0f;

  const uint16_t* arow = g.a + q0;
#pragma unroll 4
  for (int j = 0; j < g.r; ++j) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(arow + static_cast<int64_t>(j) * g.k);
    const float av[8] = {bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1]),
                         bf16_lo(v[2]), bf16_hi(v[2]), bf16_lo(v[3]), bf16_hi(v[3])};
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float bj = bs[4 * wave + rr][j];
#pragma unroll
      for (int c = 0; c < 8; ++c) d[rr][c] = d[rr][c] + bj * av[c];
    }
  }

#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int64_t p = row0 + 4 * wave + rr;
    if (p >= g.n) break;
    const int64_t e0 = p * g.k + q0;
    float base[8];
    if (kSrc == kPacked) {
      const uint32_t cw = *reinterpret_cast<const uint32_t*>(g.w.codes + e0 / 2);
      const int64_t blk = e0 / kBlock;
      const float sc =
          g.w.dq ? dq_unit(g.w.scale_codes[blk], g.w.dq) * g.w.group_scale[blk / kGroup] : g.w.absmax[blk];
#pragma unroll
      for (int c = 0; c < 8; ++c) base[c] = bf16_hi(bf16_rne_hi(lv[(cw >> (4 * c)) & 0xF] * sc));
    } else if (kSrc == kDenseBf16) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(g.dense) + e0);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        base[2 * c] = bf16_lo(v[c]);
        base[2 * c + 1] = bf16_hi(v[c]);
      }
    } else {
      const f32x4* src = reinterpret_cast<const f32x4*>(static_cast<const float*>(g.dense) + e0);
      const f32x4 u0 = src[0], u1 = src[1];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        base[c] = u0[c];
        base[4 + c] = u1[c];
      }
    }
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float t = g.s * d[rr][c];
      o[c] = kSub ? base[c] - t : base[c] + t;
    }
    if (kOutF32) {
      f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(g.out) + e0);
      dst[0] = f32x4{o[0], o[1], o[2], o[3]};
      dst[1] = f32x4{o[4], o[5], o[6], o[7]};
    } else {
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(g.out) + e0) =
          u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
    }
  }
}

template <int kSrc, bool kSub>
hipError_t launch_merge_t(const MergeArgs& g, bool out_f32, const Levels& L, hipStream_t st) {
  const int64_t tiles = ((g.n + kRows - 1) / kRows) * ((g.k + kCols - 1) / kCols);
  const dim3 grid(static_cast<unsigned>(tiles)), block(256);
  if (out_f32) {
    hipLaunchKernelGGL((merge_kernel<kSrc, kSub, true>), grid, block, 0, st, g, L);
  } else {
    hipLaunchKernelGGL((merge_kernel<kSrc, kSub, false>), grid, block, 0, st, g, L);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const PackedW& w, const uint16_t* a, const uint16_t* b, int r, float s, int out_f32,
                        void* out, hipStream_t st) {
  MergeArgs g{};
  g.w = w;
  g.a = a;
  g.b = b;
  g.n = w.n;
  g.k = w.k;
  g.r = r;
  g.s = r > 0 ? s : 0.0f;
  g.out = out;
  return launch_merge_t<kPacked, false>(g, out_f32 != 0, codebook_table(w.codebook), st);
}

hipError_t launch_unmerge(const void* merged, int src_f32, int64_t n, int64_t k, const uint16_t* a,
                          const uint16_t* b, int r, float s, void* out, hipStream_t st) {
  MergeArgs g{};
  g.dense = merged;
  g.a = a;
  g.b = b;
  g.n = n;
  g.k = k;
  g.r = r;
  g.s = r > 0 ? s : 0.0f;
  g.out = out;
  const Levels& L = nf4_table();  // unused by dense sources
  return src_f32 ? launch_merge_t<kDenseF32, true>(g, true, L, st) : launch_merge_t<kDenseBf16, true>(g, false, L, st);
}

}  // namespace qlora
