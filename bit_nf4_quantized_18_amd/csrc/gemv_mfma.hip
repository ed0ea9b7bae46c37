// Decode path, 3 to 16 tokens (any k) and one or two tokens at k > 12288:
// Y = X W16^T + s H B^T with W read straight from its packed NF4 form, in one
// launch (one or two tokens at k <= 12288 take the row-per-wave kernel of
// gemv_kernels.hip).
//
// Ultralytics glossary "QLoRA", section "Come funziona QLoRA": each frozen
// layer dequantizes its NF4 weights to bfloat16 right before the matmul and
// adds the LoRA path output ("LoRA y QLoRA en Profundidad", "La Idea Central":
// H = X A^T, then (alpha / r) H B^T). At a handful of tokens the layer is
// bound by the HBM stream of the packed weight (0.5 B of codes + 1/64 B of
// scale codes per weight) and by the latency of one trip to memory, so the
// kernel is built around that stream:
//   * a workgroup owns 16 weight rows; its 16 waves x 4 lane groups split the
//     row's 64-blocks round-robin, so every lane loads whole blocks (32 B of
//     codes, two 16-byte loads), from clamped addresses (an out-of-range block
//     gets a zero scale) so that no load sits behind a guard;
//   * per block a lane decodes the scale, builds a 16-entry bf16 table in
//     registers (nf4_lut.h) and looks up 8 weights per table access;
//   * the dot products run on the matrix cores (16x16x32 bf16 MFMA with the
//     tokens padded to 16), so the vector ALU only unpacks;
//   * the X fragments (and, with kFuseH, the A fragments of the LoRA-down
//     product H = X A^T) come through LDS: each wave copies the 256-k slice
//     its lane groups multiply into a private region in whole runs, so every
//     workgroup computes H for itself without a launch or a barrier of its
//     own. Without kFuseH (r > 16), H arrives as partial sums from the
//     skinny kernel;
//   * partial sums of the waves are reduced in a fixed order in LDS, so
//     results do not depend on scheduling.
#include "bufmem.h"
#include "internal.h"
#include "mfma.h"
#include "nf4_lut.h"

namespace qlora {
namespace {

constexpr int kGroup = 256;

// 8 consecutive bf16 (x0x1, x2x3, x4x5, x6x7) -> the order lut8_decode_order
// produces weights in, (x0x2, x4x6, x1x3, x5x7): an MFMA pairs operand slots
// by position, so both operands only need the same order.
__device__ __forceinline__ u32x4 decode_order(u32x4 v) {
  const uint32_t in[4] = {v[0], v[1], v[2], v[3]};
  uint32_t out[4];
  to_decode_order(in, out);
  return u32x4{out[0], out[1], out[2], out[3]};
}

// First H slot of output row p: part l (rows up to P.end[l]) owns slots
// l rb .. (l+1) rb - 1; with one part, 0.
__device__ __forceinline__ int part_slot0(const LoraParts& P, int p, int rb) {
  int off = 0;
#pragma unroll
  for (int l = 0; l + 1 < 4; ++l) off += (l + 1 < P.g && p >= P.end[l]) ? rb : 0;
  return off;
}

// Multi-pass form for k > 4096: one workgroup per group of 16 weight rows,
// passes of 64 blocks (one per lane group). In each pass a wave stages the
// 256-k slice of X, then of A, that its lane groups multiply through its own
// LDS region (see the persistent form below for the layout), so neither the
// fragment loads nor the H product need anything from another wave.
template <int WAVES, bool kDQ, bool kFuseH, bool kF16>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(PackedW w, const uint16_t* __restrict__ x, int M,
                                                          const uint16_t* __restrict__ a,
                                                          const float* __restrict__ hpart, int hsplits,
                                                          const uint16_t* __restrict__ b, int rh, int rb,
                                                          LoraParts P, float s, uint16_t* __restrict__ y,
                                                          float* __restrict__ h_out, Levels L) {
  static_assert(WAVES == 16, "one pass covers 64 blocks, four per wave");
  constexpr int kLaneGroups = WAVES * 4;
  constexpr int kSlice = 16 * 512;  // one wave's region: 16 rows x 256 k of bf16
  constexpr int kRedBytes = (kFuseH ? 2 : 1) * WAVES * 64 * 16;
  constexpr int kStage = WAVES * kSlice;
  static_assert(kStage >= kRedBytes, "the reductions reuse the staging regions");
  __shared__ __attribute__((aligned(16))) unsigned char stage[kStage];
  __shared__ float h_lds[16 * QLORA_MAX_RANK];
  __shared__ uint16_t b_lds[16 * QLORA_MAX_RANK];
  f32x4(*red)[64] = reinterpret_cast<f32x4(*)[64]>(stage);
  f32x4(*hred)[64] = reinterpret_cast<f32x4(*)[64]>(stage + WAVES * 64 * 16);
  // the same buffers as floats: the reduction reads one component per lane
  const float* redf = reinterpret_cast<const float*>(stage);
  const float* hredf = reinterpret_cast<const float*>(stage + WAVES * 64 * 16);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int G = wave * 4 + g;
  // 32-bit offsets: the host guarantees n * k <= 2^31
  const int K = static_cast<int>(w.k), N = static_cast<int>(w.n);
  const int nbk = K / 64;
  const int n0 = blockIdx.x * 16;
  const int n = n0 + i;
  const int n_c = n < N ? n : N - 1;  // clamped: every load is unconditional
  // X through a buffer resource sized to its M rows, A to its rh rows: rows
  // past them read zeros without touching memory
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), static_cast<short>(0),
                                                                        M * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a), static_cast<short>(0),
                                                                        kFuseH ? rh * K * 2 : 0, 0x00020000);
  const int wv_u = __builtin_amdgcn_readfirstlane(wave);
  unsigned char* region = stage + wv_u * kSlice;
  const int crow = lane >> 5;
  // the wave's slice of pass `base`: copy t moves rows 2t and 2t+1, lane l
  // fetches piece (l & 31) ^ row of row 2t + (l >> 5) into slot l of the copy
  auto copy_slice = [&](__amdgpu_buffer_rsrc_t rsrc, int rows, int base) {
    const int ncopy = (rows + 1) >> 1;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t < ncopy) {
        const int row = 2 * t + crow;
        const int goff = row * K * 2 + (base + 4 * wv_u) * 128 + 16 * ((lane & 31) ^ row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(region + t * 1024), 16, goff, 0, 0, 0);
      }
    }
  };
  // fragment j of lane (i, g): piece 8 g + j of row i
  auto read_frag = [&](int j) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(region + i * 512 + 16 * ((8 * g + j) ^ i));
  };

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 hacc = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int kBPer = (16 * QLORA_MAX_RANK + WAVES * 64 - 1) / (WAVES * 64);  // B values per thread
  uint16_t bv[kBPer];
  const int blast = N * rb - 1;
  if (rb > 0) {
    // this workgroup's 16 rows of B (contiguous in memory), into registers
    // now and into LDS after the main product (indices clamped to the last
    // element of B; rows past N are never stored)
#pragma unroll
    for (int u = 0; u < kBPer; ++u) {
      const int e = n0 * rb + tid + u * WAVES * 64;
      bv[u] = b[e < blast ? e : blast];
    }
  }
  if (!kFuseH && rh > 0) {
    // H = sum of the LoRA-down partials (fixed order)
    const int mr = M * rh;
    for (int idx = tid; idx < mr; idx += WAVES * 64) {
      float hv = 0.0f;
#pragma unroll 8
      for (int sp = 0; sp < hsplits; ++sp) hv += hpart[sp * mr + idx];  // loads in flight together, sums in order
      h_lds[idx] = hv;
      if (h_out != nullptr && blockIdx.x == 0) h_out[idx] = hv;
    }
  }

  for (int base = 0; base < nbk; base += kLaneGroups) {
    const bool has_slice = base + wave * 4 < nbk;  // wave-uniform
    const int kb = base + G;
    const bool kval = kb < nbk;
    const int kb_c = kval ? kb : nbk - 1;
    // this pass's X slice, then its codes and scales; wait for the copies
    // only (the previous pass's reads of the region are done: lgkmcnt below)
    __builtin_amdgcn_sched_barrier(0);
    if (has_slice) copy_slice(xrsrc, M, base);
    __builtin_amdgcn_sched_barrier(0);
    const u32x4* cp = reinterpret_cast<const u32x4*>(w.codes + (n_c * (K / 2) + kb_c * 32));
    const u32x4 c0 = cp[0];
    const u32x4 c1 = cp[1];
    const int bi = n_c * nbk + kb_c;
    uint8_t scode = 0;
    float gsc;
    if (kDQ) {
      scode = w.scale_codes[bi];
      gsc = w.group_scale[static_cast<uint32_t>(bi) / kGroup];
    } else {
      gsc = w.absmax[bi];
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<2 + (kDQ ? 2 : 1)>();
    __builtin_amdgcn_sched_barrier(0);
    u32x4 xa[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xa[j] = u32x4{0, 0, 0, 0};
    if (has_slice && kval && i < M) {
#pragma unroll
      for (int j = 0; j < 8; ++j) xa[j] = read_frag(j);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) xa[j] = decode_order(xa[j]);
    if (kFuseH) {
      // the region's X is in registers: this pass's slice of A replaces it
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the fragment reads are done
      if (has_slice) copy_slice(arsrc, rh, base);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (has_slice) {
      const bool ok = (n < N) && kval;
      const float sc = kDQ ? dq_unit(scode, w.dq) * gsc : gsc;
      const BlockLut lut = make_block_lut<kF16>(L.v, ok ? sc : 0.0f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t cw = (j < 4) ? c0[j] : c1[j - 4];
        uint32_t wv[4];
        lut8_decode_order(lut, cw, wv);
        acc = mma16<kF16>(xa[j], u32x4{wv[0], wv[1], wv[2], wv[3]}, acc);
      }
    }
    if (kFuseH) {
      // H product of the pass from the wave's own copies of A
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();
      __builtin_amdgcn_sched_barrier(0);
      if (has_slice) {
        u32x4 af[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) af[j] = u32x4{0, 0, 0, 0};
        if (kval && i < rh) {
#pragma unroll
          for (int j = 0; j < 8; ++j) af[j] = read_frag(j);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) hacc = mma16<kF16>(xa[j], decode_order(af[j]), hacc);
      }
    }
    // the next pass's copies overwrite the region: its reads must be done
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int u = 0; u < kBPer; ++u) {
    const int idx = tid + u * WAVES * 64;
    if (idx < 16 * rb) b_lds[idx] = bv[u];  // rb = 0: never, bv unset
  }

  __syncthreads();  // every wave is done with its region
  red[wave][lane] = acc;
  if (kFuseH) hred[wave][lane] = hacc;
  __syncthreads();
  const int l2 = tid & 63, v = tid >> 6;  // used by the first 256 threads
  const int mo = 4 * (l2 >> 4) + v;       // token row of the 16 x 16 tile
  if (kFuseH) {
    // H[mo][j] of the (token, rank) tile, j = l2 & 15
    if (tid < 256) {
      const int j = l2 & 15;
      float hv = 0.0f;
#pragma unroll
      for (int wv = 0; wv < WAVES; ++wv) hv += hredf[(wv * 64 + l2) * 4 + v];
      if (mo < M && j < rh) {
        h_lds[mo * rh + j] = hv;
        if (h_out != nullptr && blockIdx.x == 0) h_out[mo * rh + j] = hv;
      }
    }
    __syncthreads();
  }
  if (tid >= 256) return;
  const int no = n0 + (l2 & 15);
  if (mo >= M || no >= N) return;
  float sum = 0.0f;
#pragma unroll
  for (int wv = 0; wv < WAVES; ++wv) sum += redf[(wv * 64 + l2) * 4 + v];
  if (rb > 0) {
    float lo = 0.0f;
    const uint16_t* brow = b_lds + (l2 & 15) * rb;
    const float* hrow = h_lds + mo * rh + part_slot0(P, no, rb);
    for (int j = 0; j < rb; ++j) lo = fmaf(hrow[j], to_f32<kF16>(brow[j]), lo);
    sum = fmaf(s, lo, sum);
  }
  y[mo * N + no] = to16<kF16>(sum);
}

// Persistent form for k <= 4096 (one pass covers a row): a workgroup takes
// row groups rg = blockIdx.x, + gridDim.x, ... (grid = number of CUs) and
// software-pipelines them: the codes, scales and B rows of the next row group
// are in flight while the current one is unpacked and multiplied. X is loaded
// once (the same fragments serve every row group) and, with kFuseH, H is
// computed once per workgroup, in its first row group.
//
// X and A reach the fragments through LDS, one private 8 KB region per wave:
// wave w's lane groups need the 256-k slice [256 w, 256 w + 256) of every
// token (rank) row, 512 contiguous bytes per row, so the wave copies its
// slice global -> LDS in whole 1 KB runs (two rows per copy) and reads its
// fragments back. Read straight from global, each 16-byte fragment load
// would touch a different cache line per lane group and token (64 lines per
// load instead of 8 per copy). Piece p of row i is stored in slot p ^ i of
// the row, so the 16 rows of one piece fall in 16 different bank groups. The
// region holds X first; once X is in registers it receives the wave's slice
// of A, which only that wave reads: H needs no barrier of its own.
template <bool kDQ, bool kFuseH, bool kF16>
__global__ __launch_bounds__(1024) void gemv_persistent_kernel(PackedW w, const uint16_t* __restrict__ x, int M,
                                                               const uint16_t* __restrict__ a,
                                                               const float* __restrict__ hpart, int hsplits,
                                                               const uint16_t* __restrict__ b, int rh, int rb,
                                                               LoraParts P, float s, uint16_t* __restrict__ y,
                                                               float* __restrict__ h_out, Levels L) {
  constexpr int WAVES = 16;
  constexpr int kSlice = 16 * 512;  // one wave's region: 16 rows x 256 k of bf16
  constexpr int kRedBytes = (kFuseH ? 2 : 1) * WAVES * 64 * 16;
  constexpr int kStage = WAVES * kSlice;
  constexpr int kBPer = (16 * QLORA_MAX_RANK + WAVES * 64 - 1) / (WAVES * 64);  // B values per thread
  __shared__ __attribute__((aligned(16))) unsigned char stage[kStage > kRedBytes ? kStage : kRedBytes];
  __shared__ float h_lds[16 * QLORA_MAX_RANK];
  __shared__ uint16_t b_lds[16 * QLORA_MAX_RANK];
  f32x4(*red)[64] = reinterpret_cast<f32x4(*)[64]>(stage);
  f32x4(*hred)[64] = reinterpret_cast<f32x4(*)[64]>(stage + WAVES * 64 * 16);
  // the same buffers as floats: the reduction reads one component per lane
  const float* redf = reinterpret_cast<const float*>(stage);
  const float* hredf = reinterpret_cast<const float*>(stage + WAVES * 64 * 16);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int G = wave * 4 + g;  // this lane group's block of every row group
  const int K = static_cast<int>(w.k), N = static_cast<int>(w.n);
  const int nbk = K / 64;  // <= 64
  const int nrg = (N + 15) / 16;
  const bool kval = G < nbk;
  const int kb_c = kval ? G : nbk - 1;
  const int wv_u = __builtin_amdgcn_readfirstlane(wave);
  const int blast = N * rb - 1;
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), static_cast<short>(0),
                                                                        M * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a), static_cast<short>(0),
                                                                        kFuseH ? rh * K * 2 : 0, 0x00020000);

  struct Loads {
    u32x4 c0, c1;
    uint8_t scode;  // widened where it is used, so that nothing waits for it earlier
    float gsc;
    uint16_t bv[kBPer];
  };
  // loads of row group rg < nrg; with real = false the same instructions on
  // the first element of every array (one cache line each, results unused)
  auto issue = [&](int rgc, Loads& T, bool real) {
    const int n = rgc * 16 + i;
    const int n_c = real ? (n < N ? n : N - 1) : 0;
    const int kb_r = real ? kb_c : 0;
    const u32x4* cp = reinterpret_cast<const u32x4*>(w.codes + (n_c * (K / 2) + kb_r * 32));
    T.c0 = cp[0];
    T.c1 = cp[real ? 1 : 0];
    const int bi = n_c * nbk + kb_r;
    if (kDQ) {
      T.scode = w.scale_codes[bi];
      T.gsc = w.group_scale[static_cast<uint32_t>(bi) / kGroup];
    } else {
      T.scode = 0;
      T.gsc = w.absmax[bi];
    }
    // B rows: always kBPer loads (from X's first element when there is no
    // B), so that every path issues the same number of loads per row group
#pragma unroll
    for (int u = 0; u < kBPer; ++u) {
      const int e = rgc * 16 * rb + tid + u * WAVES * 64;
      const uint16_t* bp = (rb > 0 && real) ? b + (e < blast ? e : blast) : x;
      T.bv[u] = *bp;
    }
  };
  constexpr int kTaskLoads = 2 + (kDQ ? 2 : 1) + kBPer;  // per issue()

  // This wave's region and its copies: copy t moves rows 2t and 2t+1; lane l
  // fetches piece (l & 31) ^ row of row 2t + (l >> 5) into slot l of the copy.
  // Rows past the matrix (tokens >= M, ranks >= rh) read zeros; a wave whose
  // slice starts past K copies nothing (its lane groups have no block).
  unsigned char* region = stage + wv_u * kSlice;
  const bool has_slice = wave * 4 < nbk;  // wave-uniform
  const int crow = lane >> 5;
  auto copy_slice = [&](__amdgpu_buffer_rsrc_t rsrc, int rows) {
    const int ncopy = (rows + 1) >> 1;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t < ncopy) {
        const int row = 2 * t + crow;
        const int goff = row * K * 2 + wv_u * 512 + 16 * ((lane & 31) ^ row);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(region + t * 1024), 16, goff, 0, 0, 0);
      }
    }
  };
  // fragment j of lane (i, g): piece 8 g + j of row i
  auto read_frag = [&](int j) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(region + i * 512 + 16 * ((8 * g + j) ^ i));
  };

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 hacc = f32x4{0.f, 0.f, 0.f, 0.f};
  Loads T0, T1;
  const int rg0 = blockIdx.x;
  // X slice first, then the first row group's loads; wait for the X copies
  // only (every load issued after them may stay in flight)
  __builtin_amdgcn_sched_barrier(0);
  if (has_slice) copy_slice(xrsrc, M);
  __builtin_amdgcn_sched_barrier(0);
  issue(rg0, T0, true);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<kTaskLoads>();
  __builtin_amdgcn_sched_barrier(0);
  u32x4 xa[8];  // X fragments of this lane's block: the same for every row group
#pragma unroll
  for (int j = 0; j < 8; ++j) xa[j] = u32x4{0, 0, 0, 0};
  if (kval && i < M) {
#pragma unroll
    for (int j = 0; j < 8; ++j) xa[j] = read_frag(j);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) xa[j] = decode_order(xa[j]);
  if (kFuseH) {
    // the region's X has been read into registers: A's slice replaces it
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the fragment reads are done
    if (has_slice) copy_slice(arsrc, rh);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!kFuseH && rh > 0) {
    // H = sum of the LoRA-down partials (fixed order)
    const int mr = M * rh;
    for (int idx = tid; idx < mr; idx += WAVES * 64) {
      float hv = 0.0f;
#pragma unroll 8
      for (int sp = 0; sp < hsplits; ++sp) hv += hpart[sp * mr + idx];  // loads in flight together, sums in order
      h_lds[idx] = hv;
      if (h_out != nullptr && blockIdx.x == 0) h_out[idx] = hv;
    }
  }

  auto step = [&](int rg, Loads& Tc, Loads& Tn) {
    const bool has_next = rg + static_cast<int>(gridDim.x) < nrg;  // uniform
    // the next row group's loads, or after the last one the same number of
    // stand-in loads: the waits below count the same on every path
    issue(rg + static_cast<int>(gridDim.x), Tn, has_next);
    // wave-uniform guard; lane groups past the row's blocks get a zero scale
    if (wave * 4 < nbk) {
      const int n = rg * 16 + i;
      const bool ok = (n < N) && kval;
      const float sc = kDQ ? dq_unit(Tc.scode, w.dq) * Tc.gsc : Tc.gsc;
      const BlockLut lut = make_block_lut<kF16>(L.v, ok ? sc : 0.0f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t cw = (j < 4) ? Tc.c0[j] : Tc.c1[j - 4];
        uint32_t wv[4];
        lut8_decode_order(lut, cw, wv);
        acc = mma16<kF16>(xa[j], u32x4{wv[0], wv[1], wv[2], wv[3]}, acc);
      }
    }
    const bool first = rg == rg0;
    if (kFuseH && first) {
      // H product, once: wait for this wave's copies of A (everything issued
      // after them is the next row group's loads); only this wave reads them
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<kTaskLoads>();
      __builtin_amdgcn_sched_barrier(0);
      if (has_slice) {
        u32x4 af[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) af[j] = u32x4{0, 0, 0, 0};
        if (kval && i < rh) {
#pragma unroll
          for (int j = 0; j < 8; ++j) af[j] = read_frag(j);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) hacc = mma16<kF16>(xa[j], decode_order(af[j]), hacc);
      }
    }
    // epilogue of row group rg
    __syncthreads();  // LDS free: the previous epilogue's reads (and the A slice's) are done
    red[wave][lane] = acc;
    if (kFuseH && first) hred[wave][lane] = hacc;
#pragma unroll
    for (int u = 0; u < kBPer; ++u) {
      const int idx = tid + u * WAVES * 64;
      if (idx < 16 * rb) b_lds[idx] = Tc.bv[u];
    }
    __syncthreads();
    const int l2 = tid & 63, v = tid >> 6;
    const int mo = 4 * (l2 >> 4) + v;
    if (kFuseH && first) {
      if (tid < 256) {
        const int j = l2 & 15;
        float hv = 0.0f;
#pragma unroll
        for (int wv = 0; wv < WAVES; ++wv) hv += hredf[(wv * 64 + l2) * 4 + v];
        if (mo < M && j < rh) {
          h_lds[mo * rh + j] = hv;
          if (h_out != nullptr && blockIdx.x == 0) h_out[mo * rh + j] = hv;
        }
      }
      __syncthreads();
    }
    const int no = rg * 16 + (l2 & 15);
    if (tid < 256 && mo < M && no < N) {
      float sum = 0.0f;
#pragma unroll
      for (int wv = 0; wv < WAVES; ++wv) sum += redf[(wv * 64 + l2) * 4 + v];
      if (rb > 0) {
        float lo = 0.0f;
        const uint16_t* brow = b_lds + (l2 & 15) * rb;
        const float* hrow = h_lds + mo * rh + part_slot0(P, no, rb);
        for (int j = 0; j < rb; ++j) lo = fmaf(hrow[j], to_f32<kF16>(brow[j]), lo);
        sum = fmaf(s, lo, sum);
      }
      y[mo * N + no] = to16<kF16>(sum);
    }
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  for (int rg = rg0; rg < nrg; rg += 2 * gridDim.x) {
    step(rg, T0, T1);
    if (rg + gridDim.x < nrg) step(rg + gridDim.x, T1, T0);
  }
}

}  // namespace

namespace {

template <bool kF16>
hipError_t launch_gemv_t(const PackedW& w, const uint16_t* x, int64_t m, const uint16_t* a, const float* hpart,
                         int hsplits, const uint16_t* b, int r, float s, uint16_t* y, float* h_out, hipStream_t st,
                         const LoraParts& P) {
  constexpr int kWaves = 16;
  const int64_t nrg = (w.n + 15) / 16;
  const bool fuse = gemv_fuses_h(m, w.k, r, P.g > 1 ? &P : nullptr);
  const int rb = P.g > 1 ? P.rpart : r;
  if (w.k <= 4096) {
    const unsigned grid = static_cast<unsigned>(nrg < device_cus() ? nrg : device_cus());
    auto kern = w.dq ? (fuse ? gemv_persistent_kernel<true, true, kF16> : gemv_persistent_kernel<true, false, kF16>)
                     : (fuse ? gemv_persistent_kernel<false, true, kF16> : gemv_persistent_kernel<false, false, kF16>);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kWaves * 64), 0, st, w, x, static_cast<int>(m), a, hpart, hsplits, b,
                       r, rb, P, s, y, h_out, codebook_table(w.codebook));
    return hipGetLastError();
  }
  auto kern = w.dq ? (fuse ? gemv_kernel<kWaves, true, true, kF16> : gemv_kernel<kWaves, true, false, kF16>)
                   : (fuse ? gemv_kernel<kWaves, false, true, kF16> : gemv_kernel<kWaves, false, false, kF16>);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(nrg)), dim3(kWaves * 64), 0, st, w, x, static_cast<int>(m), a,
                     hpart, hsplits, b, r, rb, P, s, y, h_out, codebook_table(w.codebook));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_mfma(const PackedW& w, const uint16_t* x, int64_t m, const uint16_t* a, const float* hpart,
                            int hsplits, const uint16_t* b, int r, float s, uint16_t* y, float* h_out, hipStream_t st,
                            bool f16, const LoraParts* parts) {
  LoraParts one;
  one.g = 1;
  one.rpart = r;
  one.end[0] = static_cast<int>(w.n);
  const LoraParts& P = parts != nullptr ? *parts : one;
  return f16 ? launch_gemv_t<true>(w, x, m, a, hpart, hsplits, b, r, s, y, h_out, st, P)
             : launch_gemv_t<false>(w, x, m, a, hpart, hsplits, b, r, s, y, h_out, st, P);
}

}  // namespace qlora
