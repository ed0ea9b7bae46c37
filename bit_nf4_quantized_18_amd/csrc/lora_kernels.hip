// Rank-r side kernels of the LoRA path.
//
// "LoRA y QLoRA en Profundidad", section "La Idea Central": the adapter adds
// (alpha / r) * B @ A with A r x d_in and B d_out x r. With H = X A^T the
// forward adds s H B^T; the backward (Ultralytics glossary "QLoRA", "Come
// funziona QLoRA": gradients only for the two LoRA matrices) needs
// dH = s dY B, dA = dH^T X and dB = s dY^T H.
//
// These are thin (r <= 128 columns) and are bounded by one pass over X or dY.
#include "bufmem.h"
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
template <int RT, int WAVES, bool kF16, int kU = 0>
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

  // U chunks per wave per trip (kU if given). Loads are unconditional from
  // clamped addresses (a guarded load makes the compiler wait for all
  // outstanding loads); chunks past the split and ranks past r are zeroed at
  // the operand.
  constexpr int U = kU > 0 ? kU : ((RT <= 2) ? 4 : (RT <= 4 ? 8 : 4));
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
        acc[t] = mma16<kF16>(av, j < r ? b[u][t] : u32x4{0, 0, 0, 0}, acc[t]);
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
      if (out_bf16 != nullptr && j < rpad) out_bf16[mo * rpad + j] = to16<kF16>(scale2 * val);
    }
  }
}

// Prefill projection for r <= 64 (RT = 1, 2 or 4 rank tiles of 16):
// part[s][m][j] = sum over the columns q of split s of P[m][q] Q[j][q], P bf16
// M x qn, Q bf16 r x qn. Workgroup: 64 rows of P and one split of the
// columns. Two copy waves stream chunks of 128 columns -- one the P tile
// (64 x 128), the other the Q tile (16 RT x 128), whole 256-byte row runs --
// into a ring of four LDS stages with global->LDS buffer loads, three chunks
// ahead. Four compute waves (16 rows each) read 16-byte fragments and run
// 16x16x32 bf16 MFMAs (Q as the first operand: a lane ends with 4 ranks of
// one row per rank tile). In LDS the 16-byte chunk c of row t is stored at
// chunk c ^ (t % 16), so the 16 lanes that read one chunk of 16 rows hit
// distinct banks. Rows past M and Q rows past r read as zeros, Q columns past
// the split's end too; a column of P past it meets one of those zeros.
constexpr int kPjRows = 64, kPjCols = 128, kPjStages = 4;
constexpr int kPjP = kPjRows * kPjCols;  // bf16 elements per stage

template <int RT, bool kF16>
__global__ __launch_bounds__(384) void proj_kernel(const uint16_t* __restrict__ P, const uint16_t* __restrict__ Q,
                                                   int64_t M, int64_t qn, int r, int splits, int64_t per,
                                                   float* __restrict__ part) {
  // bf16 elements per Q stage: 64 rows, so that every copy instruction has
  // rows of its own (those past 16 RT receive zeros and are never read)
  constexpr int kQ = kPjRows * kPjCols;
  __shared__ __attribute__((aligned(16))) uint16_t Ps[kPjStages * kPjP];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[kPjStages * kQ];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.y;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kPjRows;
  const int64_t qb = s * per;
  const int64_t qe = (qb + per < qn) ? qb + per : qn;
  const int nch = qe > qb ? static_cast<int>((qe - qb + kPjCols - 1) / kPjCols) : 0;

  if (wave >= 4) {
    // ======================= copy waves =======================
    // wave 4 moves P, wave 5 moves Q. Instruction u: rows 4u + lane / 16 of
    // the tile, the logical chunk that the swizzle stores at position lane % 16.
    const bool isq = wave == 5;
    const int64_t rows = (M - m0 < kPjRows) ? M - m0 : kPjRows;
    const int trow = lane >> 4;
    constexpr int kCopies = 16;  // per chunk and wave: 64 rows of 128 columns
    auto copy_chunk = [&](int c) {
      const int64_t qc = qb + static_cast<int64_t>(c) * kPjCols;
      const bool live = qc < qe;
      const int64_t qcl = live ? qc : 0;
      const __amdgpu_buffer_rsrc_t rs = isq ? make_rsrc(Q + qcl, live ? (r * qn - qcl) * 2 : 0)
                                            : make_rsrc(P + m0 * qn + qcl, live ? (rows * qn - qcl) * 2 : 0);
      uint16_t* dst = isq ? Qs + (c % kPjStages) * kQ : Ps + (c % kPjStages) * kPjP;
#pragma unroll
      for (int u = 0; u < kCopies; ++u) {
        const int row = 4 * u + trow;
        const int chunk = (lane & 15) ^ (row & 15);
        // Q: rows past 16 RT and columns past the split's end read zero
        // (offset out of range)
        const bool in = !isq || (row < 16 * RT && qc + 8 * chunk < qe);
        const int off = in ? static_cast<int>((row * qn + 8 * chunk) * 2) : 0x7FFFFFF0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + u * 512), 16, off, 0, 0, 0);
      }
    };
    copy_chunk(0);
    copy_chunk(1);
    copy_chunk(2);
    for (int c = 0; c < nch; ++c) {
      copy_chunk(c + 3);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<3 * kCopies>();  // chunk c has landed (loads complete in issue order)
      // bare barriers: a fenced one would wait for the copies still in flight
      __builtin_amdgcn_s_barrier();  // chunk c is in LDS
      __builtin_amdgcn_s_barrier();  // its slot has been read
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<0>();  // no copy may still be writing LDS when the wave ends
    return;
  }

  // ======================= compute waves =======================
  const int i = lane & 15, g = lane >> 4;
  const int prow = (16 * wave + i) * kPjCols, qrow = i * kPjCols;
  f32x4 acc[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nch; ++c) {
    __syncthreads();  // chunk c is in LDS
    const uint16_t* ps = Ps + (c % kPjStages) * kPjP + prow;
    const uint16_t* qs = Qs + (c % kPjStages) * kQ + qrow;
#pragma unroll
    for (int kk = 0; kk < kPjCols / 32; ++kk) {
      const int off = ((4 * kk + g) ^ i) * 8;  // rows 16 w + i and 16 t + i: the swizzle key is i
      const u32x4 pf = ld16(ps + off);
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t] = mma16<kF16>(ld16(qs + t * 16 * kPjCols + off), pf, acc[t]);
    }
    __syncthreads();  // the slot may be refilled
  }
  // acc[t][v] = sum for rank 16 t + 4g + v of row m0 + 16 wave + i
  const int64_t m = m0 + 16 * wave + i;
  if (m < M) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * t + 4 * g + v;
        if (j < r) part[(static_cast<int64_t>(s) * M + m) * r + j] = acc[t][v];
      }
  }
}

// p[0] + p[stride] + ... + p[(splits - 1) stride], added in that order from
// +0. The loads go out eight at a time ahead of their additions, so a thread
// waits for one memory round trip per eight splits, not one per split.
__device__ __forceinline__ float sum_splits(const float* __restrict__ p, int64_t stride, int splits) {
  constexpr int kAhead = 8;
  float sum = 0.0f;
  for (int s0 = 0; s0 < splits; s0 += kAhead) {
    float v[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) v[u] = (s0 + u < splits) ? p[static_cast<int64_t>(s0 + u) * stride] : 0.0f;
#pragma unroll
    for (int u = 0; u < kAhead; ++u)
      if (s0 + u < splits) sum += v[u];
  }
  return sum;
}

// Second half of the split prefill projection: out_f32 = scale * sum of the
// split partials (summed in split order), out_bf16 = bf16(scale2 * that),
// zero-padded from r to rpad columns.
template <bool kF16>
__global__ void skinny_final_kernel(const float* __restrict__ part, int64_t M, int r, int rpad, int splits,
                                    float scale, float scale2, float* __restrict__ out_f32,
                                    uint16_t* __restrict__ out_bf16) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= M * rpad) return;
  const int64_t mo = idx / rpad;
  const int j = static_cast<int>(idx % rpad);
  const float sum = j < r ? sum_splits(part + mo * r + j, M * r, splits) : 0.0f;
  const float val = scale * sum;
  if (out_f32 != nullptr && j < r) out_f32[mo * r + j] = val;
  if (out_bf16 != nullptr) out_bf16[idx] = to16<kF16>(scale2 * val);
}

// at (k x rpad) = A^T zero-padded; bt (rpad x n) = B^T zero-padded, both
// through LDS so that global reads and writes are whole 16-byte runs. The
// first k / 64 workgroups take 64 columns of A each, the rest 64 rows of B.
// Grouped weights: row j of B^T is slot j, owned by part j / rpart, and is
// zero outside that part's columns (b holds the parts' B stacked, rpart
// columns each). k % 64 == 0, n % 16 == 0, rpad % 32 == 0, rpart % 8 == 0
// or a single part.
constexpr int kTrCols = 64;
__global__ __launch_bounds__(256) void lora_transpose_kernel(const uint16_t* __restrict__ a,
                                                             const uint16_t* __restrict__ b, int64_t n, int64_t k,
                                                             int r, int rpad, LoraParts lp, uint16_t* __restrict__ at,
                                                             uint16_t* __restrict__ bt) {
  __shared__ uint16_t tile[QLORA_MAX_RANK * (kTrCols + 2)];
  constexpr int kLd = kTrCols + 2;  // odd word stride: column reads spread over the banks
  const int tid = threadIdx.x;
  const int64_t at_tiles = k / kTrCols;
  if (blockIdx.x < at_tiles) {
    const int64_t k0 = static_cast<int64_t>(blockIdx.x) * kTrCols;
    // rows j < rpad of A's 64-column slice (zeros for j >= r), 8 elements per item
    for (int it = tid; it < rpad * 8; it += 256) {
      const int j = it >> 3, c8 = (it & 7) * 8;
      const u32x4 v = (j < r) ? *reinterpret_cast<const u32x4*>(a + static_cast<int64_t>(j) * k + k0 + c8)
                              : u32x4{0, 0, 0, 0};
      uint32_t* dst = reinterpret_cast<uint32_t*>(tile + j * kLd + c8);  // 4-byte aligned: kLd and c8 are even
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = v[e];
    }
    __syncthreads();
    // at[k0 + kk][j .. j+7] for each output row kk of the slice
    for (int it = tid; it < kTrCols * (rpad / 8); it += 256) {
      const int kk = it / (rpad / 8), j8 = (it % (rpad / 8)) * 8;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = static_cast<uint32_t>(tile[(j8 + 2 * e) * kLd + kk]) |
               (static_cast<uint32_t>(tile[(j8 + 2 * e + 1) * kLd + kk]) << 16);
      *reinterpret_cast<u32x4*>(at + (k0 + kk) * rpad + j8) = u32x4{w[0], w[1], w[2], w[3]};
    }
    return;
  }
  const int64_t n0 = (static_cast<int64_t>(blockIdx.x) - at_tiles) * kTrCols;
  const int rp = lp.rpart;
  // B rows n0 .. n0+63 (rp slots each) into the tile as [slot][row]
  for (int it = tid; it < kTrCols * rp; it += 256) {
    const int row = it / rp, jj = it % rp;
    const int64_t nn = n0 + row;
    tile[jj * kLd + row] = (nn < n) ? b[nn * rp + jj] : uint16_t(0);
  }
  __syncthreads();
  // bt[j][n0 .. n0+63], 8 columns per item
  for (int it = tid; it < rpad * (kTrCols / 8); it += 256) {
    const int j = it / (kTrCols / 8), c8 = (it % (kTrCols / 8)) * 8;
    const int part = j / rp;
    const int64_t lo = part == 0 ? 0 : lp.end[part - 1 < 3 ? part - 1 : 3];
    const int64_t hi = part < lp.g ? lp.end[part] : 0;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t pair = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t nn = n0 + c8 + 2 * e + h;
        const uint16_t v = (j < r && nn >= lo && nn < hi) ? tile[(j - part * rp) * kLd + c8 + 2 * e + h] : 0;
        pair |= static_cast<uint32_t>(v) << (16 * h);
      }
      w[e] = pair;
    }
    if (n0 + c8 < n) *reinterpret_cast<u32x4*>(bt + static_cast<int64_t>(j) * n + n0 + c8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// part[s][j][c] = sum over rows m of split s of U[m][j] * V[m][c] (float32
// U, bf16 V). A workgroup (16 waves) owns 128 columns (two per lane) and 16
// ranks; its waves take interleaved rows of the split, 8 rows per trip with
// all V loads issued first, and are summed in LDS in a fixed order. The
// 16-rank slice of a U row is the same for every lane, so it is fetched with
// scalar loads. kFull: r is a multiple of 16 (no rank tail).
template <bool kFull, bool kF16>
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
      const float v0 = lo16<kF16>(v2[u]), v1 = hi16<kF16>(v2[u]);
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
  out[idx] = scale * sum_splits(part + j * cn + c, static_cast<int64_t>(r) * cn, splits);
}

// Both adapter gradients in one launch, for r % 16 == 0:
//   problem 0: part0[s][j][c] = sum over rows m of split s of U0[m][j] V0[m][c]
//              (dA: U0 = dH, V0 = X, c < k)
//   problem 1: the same with U1 = H, V1 = dY (dB before its scale, c < n).
// Workgroup: one 256-column block, one 16-rank tile and one row split. The
// split's rows stream through LDS in chunks of 32 rows: a copy wave moves
// the V tile (32 x 256 bf16, whole 512-byte row runs) and the U tile
// (32 x 16 float32) with global->LDS buffer loads, three chunks ahead in a
// ring of four, so each CU keeps tens of KB of reads in flight without
// spending registers on them. Eight compute waves only read LDS. With bf16
// V, each float32 U is split into two bf16 terms, hi (U with its low 16 bits
// dropped) and lo = bf16(U - hi), so U enters the product to 16 significant
// bits (relative error below 2^-16), and the bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16, float32 accumulation) run two MFMAs per 32 rows
// and 16 columns instead of eight float32 ones; the layout is described at
// the bf16 branch below. With fp16 V (whose range could not hold every U
// split this way), they run the float32 matrix-core product
// v_mfma_f32_16x16x4_f32 (D[16 ranks][16 cols]
// += U^T[16 ranks][4 rows] V[4 rows][16 cols], all in float32): wave w owns
// the 64 columns 64 (w % 4) .. +63 and every other group of 4 rows
// (w / 4); lane (g, i) reads row g of a group, U[row][j0 + i] and the 4
// bf16 at columns 4i .. 4i+3 of its 64, which feed 4 MFMAs (MFMA t covers
// columns 4i + t). The two waves of a column range are summed in a fixed
// order through LDS at the end. Rows past the split or past M and columns
// past cn read as zeros (buffer ranges); columns past cn are never stored.
struct RankGradProblem {
  const float* U;     // m x ldu float32
  const uint16_t* V;  // m x cn bf16
  int64_t cn;
  float* part;        // splits x r x cn float32
  int blocks;         // column blocks of 256
  int r;              // ranks of this problem (a multiple of 16)
  int ldu;            // row stride of U
  LoraParts lp;       // grouped dB: the column block of part l reads U columns l rpart ..
};

constexpr int kRgCols = 256, kRgRows = 32, kRgStages = 4;
constexpr int kRgV = kRgRows * kRgCols;  // bf16 elements per stage
constexpr int kRgU = kRgRows * 16;       // float32 per stage
constexpr int kRgWaves = 8;              // compute waves; one more wave copies

__device__ __forceinline__ f32x4 mfma_16x16x4_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// bf16 V tile: the 16-byte chunk c of row r is stored at chunk c ^ rg_swz(r),
// so that each 32-lane half of a transposing read (16 rows x 8 bytes: rows
// 4 s + const over s and two adjacent rows) covers every bank once.
__device__ __forceinline__ int rg_swz(int r) { return (2 * ((r >> 2) & 3)) | (8 * (r & 1)); }

// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4 p + e receives element
// e of the 8-byte rows addressed by lanes p, p + 4, p + 8 and p + 12.
__device__ __forceinline__ u32x2 rg_ld_tr(const uint16_t* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

template <bool kF16>
__global__ __launch_bounds__((kRgWaves + 1) * 64) void rank_grad_kernel(RankGradProblem p0, RankGradProblem p1,
                                                                        int64_t M, int splits, int64_t per) {
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kRgStages * kRgV];
  __shared__ __attribute__((aligned(16))) float Us[kRgStages * kRgU];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (problem, column block, rank tile, split)
  int id = blockIdx.x;
  const int n0 = p0.blocks * (p0.r / 16) * splits;
  const bool second = id >= n0;
  if (second) id -= n0;
  const RankGradProblem& pb = second ? p1 : p0;
  const int r = pb.r, ldu = pb.ldu;
  const int rt = r / 16;
  const int s = id % splits;
  const int j0 = ((id / splits) % rt) * 16;
  const int cb = id / (splits * rt);
  const int64_t c0 = static_cast<int64_t>(cb) * kRgCols;
  // grouped: the U columns of this column block's part (blocks never straddle parts)
  int part = 0;
#pragma unroll
  for (int l = 0; l < 3; ++l) part += (l + 1 < pb.lp.g && c0 >= pb.lp.end[l]) ? 1 : 0;
  const int uj0 = part * pb.lp.rpart + j0;
  const int64_t cn = pb.cn;
  const int64_t mb = s * per;
  const int64_t me = (mb + per < M) ? mb + per : M;
  const int nch = me > mb ? static_cast<int>((me - mb + kRgRows - 1) / kRgRows) : 0;

  if (wave == kRgWaves) {
    // ======================= copy wave =======================
    // V instruction u: rows 2u, 2u+1 (lane / 32), 16 bytes at column 8 (lane % 32);
    // U instruction q: rows 16q + lane / 4, floats j0 + 4 (lane % 4) .. +3.
    // (bf16: the lane fetches the column chunk that rg_swz puts in its slot;
    // row 2u + lane / 32 gives rg_swz = 2 ((u / 2) % 4) + 8 (lane / 32))
    const int v_voff = static_cast<int>((lane >> 5) * cn * 2);
    const int v_chunk = lane & 31, v_key = 8 * (lane >> 5);
    const int u_voff = static_cast<int>(((lane >> 2) * ldu + uj0 + 4 * (lane & 3)) * 4);
    auto copy_chunk = [&](int c) {
      const int64_t m0 = mb + static_cast<int64_t>(c) * kRgRows;
      const int64_t rows = (m0 < me) ? (me - m0 < kRgRows ? me - m0 : kRgRows) : 0;
      const int64_t mr = (m0 < M) ? m0 : M;
      // rows [m0, m0 + rows) from column c0; the last row ends at cn
      const __amdgpu_buffer_rsrc_t vr = make_rsrc(pb.V + mr * cn + c0, rows > 0 ? (rows * cn - c0) * 2 : 0);
      const __amdgpu_buffer_rsrc_t ur = make_rsrc(pb.U + mr * ldu, rows > 0 ? (M - mr) * ldu * 4 : 0);
      uint16_t* vs = Vs + (c % kRgStages) * kRgV;
      float* us = Us + (c % kRgStages) * kRgU;
      // (whole offsets in the vector operand: the scalar offset is not range checked)
#pragma unroll
      for (int u = 0; u < 16; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            vr, (lds_void*)(vs + u * (2 * kRgCols)), 16,
            v_voff + 16 * (kF16 ? v_chunk : (v_chunk ^ (v_key | (2 * ((u >> 1) & 3))))) + static_cast<int>(u * 4 * cn),
            0, 0, 0);
#pragma unroll
      for (int q = 0; q < 2; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ur, (lds_void*)(us + q * 256), 16, u_voff + q * 64 * ldu, 0, 0, 0);
    };
    constexpr int kCopies = 18;  // per chunk
    copy_chunk(0);
    copy_chunk(1);
    copy_chunk(2);
    for (int c = 0; c < nch; ++c) {
      copy_chunk(c + 3);
      // loads complete in issue order: with the copies of chunks c+1 .. c+3
      // outstanding, chunk c has landed
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<3 * kCopies>();
      // Bare barriers: a fenced one would wait for the copies still in
      // flight. This wave writes LDS only through the copies counted above.
      __builtin_amdgcn_s_barrier();  // chunk c is in LDS
      __builtin_amdgcn_s_barrier();  // its slot has been read
      __builtin_amdgcn_sched_barrier(0);
    }
    // no copy may still be writing LDS when the wave ends
    wait_vmcnt<0>();
    return;
  }

  // ======================= compute waves =======================
  const int i = lane & 15, g = lane >> 4;
  if constexpr (!kF16) {
    // bf16: wave w owns the 32 columns 32 w .. +31 (two 16-column MFMA tiles)
    // and all 32 rows of every chunk, so no sums cross waves. Contraction
    // slot e of lane (i, g) is chunk row 4 e + g. The U^T operand: U[4 e +
    // g][j0 + i], split as hi = U with the low 16 bits dropped and lo =
    // bf16(U - hi), two MFMAs per tile. The V operand: two transposing LDS
    // reads per tile; lane (i, g) addresses, in read h, row 4 (i / 4) + 16 h
    // + g at columns 4 (i % 4) .. +3 of the tile, and receives column i of
    // the four rows the lanes i % 4 + 4 s address.
    int voff[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 4 * (i >> 2) + 16 * h + g;
        const int col = 32 * wave + 16 * t + 4 * (i & 3);
        voff[t][h] = row * kRgCols + (((col >> 3) ^ rg_swz(row)) << 3) + (col & 7);
      }
    f32x4 acc2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int c = 0; c < nch; ++c) {
      __syncthreads();  // chunk c is in LDS
      const uint16_t* vs = Vs + (c % kRgStages) * kRgV;
      const float* us = Us + (c % kRgStages) * kRgU + 16 * g + i;
      uint32_t ahi[4], alo[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float u0 = us[64 * e], u1 = us[64 * (e + 1)];  // rows 4 e + g, 4 (e + 1) + g
        const uint32_t h0 = __float_as_uint(u0) >> 16, h1 = __float_as_uint(u1) >> 16;
        const uint32_t l0 = f32_to_bf16_rne(u0 - __uint_as_float(h0 << 16));
        const uint32_t l1 = f32_to_bf16_rne(u1 - __uint_as_float(h1 << 16));
        ahi[e >> 1] = h0 | (h1 << 16);
        alo[e >> 1] = l0 | (l1 << 16);
      }
      const u32x4 ah = u32x4{ahi[0], ahi[1], ahi[2], ahi[3]}, al = u32x4{alo[0], alo[1], alo[2], alo[3]};
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x2 b0 = rg_ld_tr(vs + voff[t][0]), b1 = rg_ld_tr(vs + voff[t][1]);
        const u32x4 bv = u32x4{b0[0], b0[1], b1[0], b1[1]};
        acc2[t] = mma16<false>(ah, bv, acc2[t]);
        acc2[t] = mma16<false>(al, bv, acc2[t]);
      }
      __syncthreads();  // the slot may be refilled
    }
    // acc2[t][v] = sum for rank j0 + 4 g + v, column c0 + 32 w + 16 t + i
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t col = c0 + 32 * wave + 16 * t + i;
      if (col < cn) {  // cn % 16 == 0: a tile is whole or absent
#pragma unroll
        for (int v = 0; v < 4; ++v)
          pb.part[(static_cast<int64_t>(s) * r + j0 + 4 * g + v) * cn + col] = acc2[t][v];
      }
    }
    return;
  }
  const int quad = wave & 3, half = wave >> 2;
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c = 0; c < nch; ++c) {
    __syncthreads();  // chunk c is in LDS
    const uint16_t* vs = Vs + (c % kRgStages) * kRgV + 64 * quad + 4 * i;
    const float* us = Us + (c % kRgStages) * kRgU + i;
#pragma unroll
    for (int e = 0; e < kRgRows / 8; ++e) {
      const int row = 4 * (2 * e + half) + g;
      const float a = us[row * 16];
      const u32x2 xv = *reinterpret_cast<const u32x2*>(vs + row * kRgCols);
      acc[0] = mfma_16x16x4_f32(a, lo16<kF16>(xv[0]), acc[0]);
      acc[1] = mfma_16x16x4_f32(a, hi16<kF16>(xv[0]), acc[1]);
      acc[2] = mfma_16x16x4_f32(a, lo16<kF16>(xv[1]), acc[2]);
      acc[3] = mfma_16x16x4_f32(a, hi16<kF16>(xv[1]), acc[3]);
    }
    __syncthreads();  // the slot may be refilled
  }
  // the copy wave has ended (or waits on its last copies): the ring is free
  __syncthreads();

  // acc[t][v] = sum for rank j0 + 4g + v, column c0 + 64 quad + 4i + t.
  // Waves 4..7 hand their sums to waves 0..3 through LDS (fixed order).
  f32x4* red = reinterpret_cast<f32x4*>(Vs);
  if (half == 1) {
#pragma unroll
    for (int t = 0; t < 4; ++t) red[(quad * 4 + t) * 64 + lane] = acc[t];
  }
  __syncthreads();
  if (half == 1) return;
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] += red[(quad * 4 + t) * 64 + lane];
  const int64_t col = c0 + 64 * quad + 4 * i;
  if (col < cn) {  // cn % 16 == 0: a run of 4 is whole
#pragma unroll
    for (int v = 0; v < 4; ++v)
      *reinterpret_cast<f32x4*>(pb.part + (static_cast<int64_t>(s) * r + j0 + 4 * g + v) * cn + col) =
          f32x4{acc[0][v], acc[1][v], acc[2][v], acc[3][v]};
  }
}

// da[j][c] = sum_s part0[s][j][c] (r0 x k); db[c][j] = scale * sum_s part1[s][j][c]
// (n x r1), each summed in split order.
__global__ void rank_grad_final_kernel(const float* __restrict__ part0, const float* __restrict__ part1, int64_t k,
                                       int64_t n, int r0, int r, int splits, float scale, float* __restrict__ da,
                                       float* __restrict__ db) {
  int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t na = static_cast<int64_t>(r0) * k;
  if (idx < na) {
    da[idx] = sum_splits(part0 + idx, na, splits);
    return;
  }
  idx -= na;
  if (idx >= static_cast<int64_t>(r) * n) return;
  const int64_t c = idx / r;
  const int j = static_cast<int>(idx % r);
  db[idx] = scale * sum_splits(part1 + j * n + c, static_cast<int64_t>(r) * n, splits);
}

// Decode form (m <= 16, partial sums only): 4 waves, one 32-wide chunk per
// wave, splits of 4 chunks (skinny_splits), so every wave makes exactly one
// trip to memory with only the loads its chunk needs.
template <int RT>
void launch_skinny_decode_rt(dim3 grid, hipStream_t st, const uint16_t* P, const uint16_t* Q, int64_t m, int64_t qn,
                             int r, int rpad, float* out_f32, int splits, bool f16) {
  if (f16) {
    hipLaunchKernelGGL((skinny_kernel<RT, 4, true, 1>), grid, dim3(256), 0, st, P, Q, m, qn, r, rpad, 1.0f, 1.0f,
                       out_f32, nullptr, splits);
  } else {
    hipLaunchKernelGGL((skinny_kernel<RT, 4, false, 1>), grid, dim3(256), 0, st, P, Q, m, qn, r, rpad, 1.0f, 1.0f,
                       out_f32, nullptr, splits);
  }
}

template <int RT>
void launch_skinny_rt(dim3 grid, hipStream_t st, const uint16_t* P, const uint16_t* Q, int64_t m, int64_t qn, int r,
                      int rpad, float scale, float scale2, float* out_f32, uint16_t* out_bf16, int splits, bool f16) {
  constexpr int kWaves = (RT <= 2) ? 16 : (RT <= 4 ? 8 : 4);
  if (f16) {
    hipLaunchKernelGGL((skinny_kernel<RT, kWaves, true>), grid, dim3(kWaves * 64), 0, st, P, Q, m, qn, r, rpad, scale,
                       scale2, out_f32, out_bf16, splits);
  } else {
    hipLaunchKernelGGL((skinny_kernel<RT, kWaves, false>), grid, dim3(kWaves * 64), 0, st, P, Q, m, qn, r, rpad, scale,
                       scale2, out_f32, out_bf16, splits);
  }
}

template <bool kF16>
void launch_proj(dim3 grid, hipStream_t st, const uint16_t* P, const uint16_t* Q, int64_t m, int64_t qn, int r,
                 int splits, int64_t per, float* part) {
  if (r <= 16) {
    hipLaunchKernelGGL((proj_kernel<1, kF16>), grid, dim3(384), 0, st, P, Q, m, qn, r, splits, per, part);
  } else if (r <= 32) {
    hipLaunchKernelGGL((proj_kernel<2, kF16>), grid, dim3(384), 0, st, P, Q, m, qn, r, splits, per, part);
  } else {
    hipLaunchKernelGGL((proj_kernel<4, kF16>), grid, dim3(384), 0, st, P, Q, m, qn, r, splits, per, part);
  }
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

bool proj_fast(int r) { return r > 0 && r <= 64; }

int proj_splits(int64_t m, int64_t qn) {
  // about one workgroup per CU, at least one 128-column chunk per split
  const int64_t blocks = (m + kPjRows - 1) / kPjRows;
  int64_t s = 256 / blocks;
  const int64_t by_cols = (qn + kPjCols - 1) / kPjCols;
  if (s > by_cols) s = by_cols;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

int skinny_prefill_splits(int64_t m, int64_t qn, int r) {
  if (proj_fast(r)) return proj_splits(m, qn);
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
                                 hipStream_t st, bool f16) {
  const int splits = skinny_prefill_splits(m, qn, r);
  if (proj_fast(r)) {
    // columns per split: a multiple of the 128-column chunk
    const int64_t per = ((qn + splits - 1) / splits + kPjCols - 1) / kPjCols * kPjCols;
    const dim3 grid(static_cast<unsigned>((m + kPjRows - 1) / kPjRows), splits);
    if (f16) {
      launch_proj<true>(grid, st, P, Q, m, qn, r, splits, per, part);
    } else {
      launch_proj<false>(grid, st, P, Q, m, qn, r, splits, per, part);
    }
  } else {
    hipError_t e = launch_skinny(P, Q, m, qn, r, rpad, 1.0f, 1.0f, part, nullptr, splits, st, f16);
    if (e != hipSuccess) return e;
  }
  const int64_t total = m * rpad;
  const dim3 fgrid(static_cast<unsigned>((total + 255) / 256));
  if (f16) {
    hipLaunchKernelGGL(skinny_final_kernel<true>, fgrid, dim3(256), 0, st, part, m, r, rpad, splits, scale, scale2,
                       out_f32, out_bf16);
  } else {
    hipLaunchKernelGGL(skinny_final_kernel<false>, fgrid, dim3(256), 0, st, part, m, r, rpad, splits, scale, scale2,
                       out_f32, out_bf16);
  }
  return hipGetLastError();
}

int skinny_splits(int64_t m, int64_t qn) {
  if (m > 16) return 1;
  // four 32-wide chunks (one per wave) per workgroup: the decode projection
  // is one memory round trip per workgroup, so it wants many of them
  const int64_t s = ((qn + 31) / 32 + 3) / 4;
  return static_cast<int>(s < 1 ? 1 : (s > 128 ? 128 : s));
}

hipError_t launch_skinny_decode(const uint16_t* P, const uint16_t* Q, int64_t m, int64_t qn, int r, int rpad,
                                float* part, int splits, hipStream_t s, bool f16) {
  if (m > 16) return hipErrorInvalidValue;
  const dim3 grid(1, static_cast<unsigned>(splits));
  if (rpad % 32 != 0 || r > rpad) return hipErrorInvalidValue;
  // rank tiles of 16 that hold the r real slots (the partial sums are written for j < r only)
  switch ((r + 15) / 16) {
    case 1: launch_skinny_decode_rt<1>(grid, s, P, Q, m, qn, r, rpad, part, splits, f16); break;
    case 2: launch_skinny_decode_rt<2>(grid, s, P, Q, m, qn, r, rpad, part, splits, f16); break;
    case 3: launch_skinny_decode_rt<3>(grid, s, P, Q, m, qn, r, rpad, part, splits, f16); break;
    case 4: launch_skinny_decode_rt<4>(grid, s, P, Q, m, qn, r, rpad, part, splits, f16); break;
    case 5: launch_skinny_decode_rt<5>(grid, s, P, Q, m, qn, r, rpad, part, splits, f16); break;
    case 6: launch_skinny_decode_rt<6>(grid, s, P, Q, m, qn, r, rpad, part, splits, f16); break;
    case 7: launch_skinny_decode_rt<7>(grid, s, P, Q, m, qn, r, rpad, part, splits, f16); break;
    case 8: launch_skinny_decode_rt<8>(grid, s, P, Q, m, qn, r, rpad, part, splits, f16); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_skinny(const uint16_t* P, const uint16_t* Q, int64_t m, int64_t qn, int r, int rpad, float scale,
                         float scale2, float* out_f32, uint16_t* out_bf16, int splits, hipStream_t s, bool f16) {
  const dim3 grid(static_cast<unsigned>((m + 15) / 16), static_cast<unsigned>(splits));
  switch (rpad / 16) {
    case 0: launch_skinny_rt<0>(grid, s, P, Q, m, qn, r, rpad, scale, scale2, out_f32, out_bf16, splits, f16); break;
    case 2: launch_skinny_rt<2>(grid, s, P, Q, m, qn, r, rpad, scale, scale2, out_f32, out_bf16, splits, f16); break;
    case 4: launch_skinny_rt<4>(grid, s, P, Q, m, qn, r, rpad, scale, scale2, out_f32, out_bf16, splits, f16); break;
    case 6: launch_skinny_rt<6>(grid, s, P, Q, m, qn, r, rpad, scale, scale2, out_f32, out_bf16, splits, f16); break;
    case 8: launch_skinny_rt<8>(grid, s, P, Q, m, qn, r, rpad, scale, scale2, out_f32, out_bf16, splits, f16); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_lora_transpose(const uint16_t* a, const uint16_t* b, int64_t n, int64_t k, int r, int rpad,
                                 uint16_t* at, uint16_t* bt, hipStream_t st, const LoraParts* parts) {
  LoraParts lp;
  lp.g = 1;
  lp.rpart = r;
  lp.end[0] = static_cast<int>(n);
  const int64_t tiles = k / kTrCols + (n + kTrCols - 1) / kTrCols;
  hipLaunchKernelGGL(lora_transpose_kernel, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, st, a, b, n, k, r, rpad,
                     parts != nullptr ? *parts : lp, at, bt);
  return hipGetLastError();
}

hipError_t launch_rank_reduce(const float* U, const uint16_t* V, int64_t m, int64_t cn, int r, float scale,
                              int splits, float* part, float* out, int c_major, hipStream_t st, bool f16) {
  const dim3 grid(static_cast<unsigned>((cn + 127) / 128), static_cast<unsigned>((r + 15) / 16),
                  static_cast<unsigned>(splits));
  if (r % 16 == 0) {
    if (f16) {
      hipLaunchKernelGGL((rank_partial_kernel<true, true>), grid, dim3(1024), 0, st, U, V, m, cn, r, splits, part);
    } else {
      hipLaunchKernelGGL((rank_partial_kernel<true, false>), grid, dim3(1024), 0, st, U, V, m, cn, r, splits, part);
    }
  } else {
    if (f16) {
      hipLaunchKernelGGL((rank_partial_kernel<false, true>), grid, dim3(1024), 0, st, U, V, m, cn, r, splits, part);
    } else {
      hipLaunchKernelGGL((rank_partial_kernel<false, false>), grid, dim3(1024), 0, st, U, V, m, cn, r, splits, part);
    }
  }
  const int64_t total = static_cast<int64_t>(r) * cn;
  hipLaunchKernelGGL(rank_final_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st, part, cn,
                     r, splits, scale, out, c_major);
  return hipGetLastError();
}

bool rank_grads_fused(int r) { return r > 0 && r % 16 == 0; }

int rank_grad_splits(int64_t m, int64_t n, int64_t k, int r0, int r1) {
  // about one workgroup per CU over both problems, at least one 32-row chunk per split
  if (!rank_grads_fused(r0) || !rank_grads_fused(r1)) return rank_reduce_splits(m, n, k, r0);
  const int64_t per_split = ((k + kRgCols - 1) / kRgCols) * (r0 / 16) + ((n + kRgCols - 1) / kRgCols) * (r1 / 16);
  int64_t s = 256 / per_split;  // at most one workgroup per CU: no second round
  const int64_t by_rows = (m + kRgRows - 1) / kRgRows;
  if (s > by_rows) s = by_rows;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  return static_cast<int>(s);
}

hipError_t launch_rank_grads(const float* dh, const uint16_t* x, int64_t k, const float* h, const uint16_t* dy,
                             int64_t n, int64_t m, int r0, const LoraParts* parts, float scale, int splits, float* part,
                             float* da, float* db, hipStream_t st, bool f16) {
  // rows per split: a multiple of the 32-row chunk
  const int64_t per = ((m + splits - 1) / splits + kRgRows - 1) / kRgRows * kRgRows;
  LoraParts one;
  one.g = 1;
  one.rpart = 0;
  one.end[0] = static_cast<int>(n);
  const int r1 = parts != nullptr ? parts->rpart : r0;
  RankGradProblem p0{dh, x, k, part, static_cast<int>((k + kRgCols - 1) / kRgCols), r0, r0, one};
  RankGradProblem p1{h, dy, n, part + static_cast<int64_t>(splits) * r0 * k, static_cast<int>((n + kRgCols - 1) / kRgCols),
                     r1, r0, parts != nullptr ? *parts : one};
  const int64_t wgs = (static_cast<int64_t>(p0.blocks) * (r0 / 16) + static_cast<int64_t>(p1.blocks) * (r1 / 16)) * splits;
  if (f16) {
    hipLaunchKernelGGL(rank_grad_kernel<true>, dim3(static_cast<unsigned>(wgs)), dim3((kRgWaves + 1) * 64), 0, st, p0,
                       p1, m, splits, per);
  } else {
    hipLaunchKernelGGL(rank_grad_kernel<false>, dim3(static_cast<unsigned>(wgs)), dim3((kRgWaves + 1) * 64), 0, st, p0,
                       p1, m, splits, per);
  }
  const int64_t total = static_cast<int64_t>(r0) * k + static_cast<int64_t>(r1) * n;
  hipLaunchKernelGGL(rank_grad_final_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, st,
                     p0.part, p1.part, k, n, r0, r1, splits, scale, da, db);
  return hipGetLastError();
}

}  // namespace qlora
