// Fused dequant-GEMMs over the packed NF4 weight (prefill / training shapes).
//
// Ultralytics glossary "QLoRA", section "Come funziona QLoRA": each frozen
// layer dequantizes its NF4 weights to bfloat16 right before the matmul, adds
// the LoRA path, and the backward computes gradients through the dequantized
// weights. Here the dequantization happens inside the K-loop of the GEMM:
// packed codes are read from HBM, turned into bf16 tiles in registers and
// staged in LDS for the matrix cores; a bf16 copy of W never exists in HBM.
//
//   forward  (kTransW = false): Y[m][n]  = sum_k X[m][k]  W[n][k] + sum_j Hs[m][j] B[n][j]
//   backward (kTransW = true):  dX[m][k] = sum_n dY[m][n] W[n][k] + sum_j dHs[m][j] At[k][j]
//
// Workgroup: 512 threads, a 256 (tokens) x 128 (outputs) tile, 64-deep
// contraction steps (one NF4 block per weight row and step).
//   * Waves 0-3 (consumers) each own a 128 x 64 sub-tile, 8 x 4 tiles of the
//     16x16x32 bf16 MFMA. They only read LDS and issue MFMAs; the fragments
//     of the next half-step are read while the current MFMAs run.
//   * Waves 4-7 (producers) copy the A tile from global memory straight
//     into LDS (buffer loads with the LDS-destination bit: no registers, no
//     LDS write instructions), and stream the packed codes and scales two
//     steps ahead, build each block's bf16 lookup table (nf4_lut.h), unpack
//     the codes and write the weight tile into LDS.
//   With one consumer and one producer wave per SIMD, unpacking (VALU) and
//   LDS traffic overlap the consumers' matrix-core work. LDS holds a ring of
//   three stages (3 x 48 KB): stage kt+2 is filled during step kt, and one
//   barrier per step suffices; before it every producer waits until its own
//   copies for stage kt+2 have landed (loads complete in issue order, so one
//   counter wait covers them).
// All global reads go through buffer resources: rows past M or N and blocks
// past the end read as zeros in hardware, with no branch, clamp or select
// (a guarded load would make the compiler wait for every outstanding load);
// per-thread offsets are computed once, a step adds one constant.
// LDS rows are 128 B without padding; the 16-byte chunk c of row r is stored
// at chunk c ^ ((r >> 1) & 7), so 16 lanes reading one chunk of 16
// consecutive rows hit 64 distinct banks. In the backward the weight tile
// keeps the weight's own orientation (64 contraction rows x 128 output
// columns, so the producers write whole 16-byte runs as in the forward), and
// the consumers read their fragments with the transposing LDS load
// ds_read_b64_tr_b16 (two per fragment). The MFMA computes the transposed
// product (weights as the first operand): each lane ends with 4 consecutive
// output columns of one token row and stores 8 contiguous bytes. Tiles are
// ordered so that the workgroups on one XCD (ids congruent mod 8) share token
// rows in that XCD's L2. The rank-r LoRA term is one more pass of MFMAs.
// kF16 builds the same kernel for IEEE-half compute: half lookup tables, the
// f16 MFMA and a half output; everything else is bit-pattern movement.
#include <type_traits>

#include "bufmem.h"
#include "internal.h"
#include "mfma.h"
#include "nf4_lut.h"

namespace qlora {
namespace {

constexpr int kBM = 256, kBP = 128, kBQ = 64;
constexpr int kStages = 3;
constexpr int kGroup = 256;
constexpr int kXcds = 8;
constexpr int kAStage = kBM * kBQ;  // bf16 elements
constexpr int kBStage = kBP * kBQ;

// element offset of (row, 16-byte chunk) in a swizzled 64-wide LDS tile
__device__ __forceinline__ int swz(int row, int chunk) { return row * kBQ + ((chunk ^ ((row >> 1) & 7)) << 3); }

// Backward weight tile: 64 contraction rows n x 128 output columns, the
// weight's own orientation. Chunk c of row n is stored at
// (c ^ ((c >> 2) & 1)) ^ swz_t_key(n): the transposed fragment reads below
// then hit every bank once per 32 lanes, and the producers' 16-byte stores
// (lanes 2i, 2i+1 writing chunk j of quarters 2b, 2b+1 of one row) fall on 8
// distinct 16-byte bank groups per 8 lanes: the odd quarter's chunks are
// swapped in pairs.
__device__ __forceinline__ int swz_t_key(int n) { return 2 * (n & 3) + 8 * ((n >> 3) & 1); }
__device__ __forceinline__ int swz_t(int n, int chunk) {
  return n * kBP + (((chunk ^ ((chunk >> 2) & 1)) ^ swz_t_key(n)) << 3);
}

// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4p + e receives element
// e of the 8-byte rows addressed by lanes p, p + 4, p + 8 and p + 12.
__device__ __forceinline__ u32x2 ld_tr4(const uint16_t* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Lanes 2i and 2i+1 of a producer wave unpack the two halves of one 64-weight
// block and so share its table. Each converts only the level pairs 2q + h
// (h = lane % 2, q = 0..3; lv holds its 8 levels) and takes the other four
// from its neighbour by a DPP swap; sel_l / sel_h order the two sources per
// lane so that every lane ends with make_block_lut's table.
template <bool kF16>
__device__ __forceinline__ BlockLut make_block_lut_pair(const float (&lv)[8], float s, uint32_t sel_l, uint32_t sel_h) {
  BlockLut t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t own = cvt_16x2<kF16>(lv[2 * q] * s, lv[2 * q + 1] * s);
    // quad_perm [1, 0, 3, 2]: the value of lane l ^ 1
    const uint32_t oth = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(own), 0xB1, 0xF, 0xF, true));
    t.tl[q] = byte_perm(oth, own, sel_l);
    t.th[q] = byte_perm(oth, own, sel_h);
  }
  return t;
}

template <bool kTransW, bool kDQ, bool kF16>
__global__ __launch_bounds__(512) void nf4_gemm_kernel(PackedW w, const uint16_t* __restrict__ A, int64_t M,
                                                       int64_t P, int64_t Qn, const uint16_t* __restrict__ ep_a,
                                                       const uint16_t* __restrict__ ep_b, int64_t ep_ld, int ep_lim,
                                                       int rpad, LoraParts lp, uint16_t* __restrict__ out, Levels L) {
  __shared__ __attribute__((aligned(16))) uint16_t As[kStages * kAStage];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kStages * kBStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // --- tile of this workgroup (XCD-aware order) ----------------------------
  // 32-bit tile arithmetic (the host bounds the tile count by 2^31); the tile
  // origin is made explicitly wave-uniform so that addresses and buffer
  // resources derived from it stay in scalar registers.
  const uint32_t tiles_p = static_cast<uint32_t>((P + kBP - 1) / kBP);
  const uint32_t tiles_m = static_cast<uint32_t>((M + kBM - 1) / kBM);
  const uint32_t T = tiles_p * tiles_m;
  const uint32_t id = blockIdx.x;
  const uint32_t xcd = id % kXcds, local = id / kXcds;
  const uint32_t start = xcd * (T / kXcds) + (xcd < T % kXcds ? xcd : T % kXcds);
  const uint32_t lin = start + local;  // bijection of [0, T)
  // Pairs of token-row tiles are interleaved along the output tiles, so a
  // run of consecutive tiles (one XCD's) covers 2 token rows x half as many
  // weight-row tiles: each weight tile and each token tile it reads is
  // shared by 2 or more workgroups of the XCD.
  const uint32_t full = (tiles_m / 2) * 2 * tiles_p;
  uint32_t mt, pt;
  if (lin < full) {
    const uint32_t rem = lin % (2 * tiles_p);
    mt = 2 * (lin / (2 * tiles_p)) + (rem & 1);
    pt = rem >> 1;
  } else {
    mt = (tiles_m / 2) * 2 + (lin - full) / tiles_p;
    pt = (lin - full) % tiles_p;
  }
  const int64_t m0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(mt)) * kBM;
  const int64_t p0 = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(pt)) * kBP;

  const int64_t K = w.k;
  const int64_t nbk = K / 64;
  const int nk = static_cast<int>((Qn + kBQ - 1) / kBQ);

  if (wave >= 4) {
    // ======================= producers =======================
    // The producers' serial path (A copies, then the unpack) sets the step;
    // a priority above the consumers' lets their instructions win the SIMD's
    // arbitration (1.5-2% per launch, forward and dX, in A/B runs)
    __builtin_amdgcn_s_setprio(1);
    const int pt = tid - 256;
    const int pw = __builtin_amdgcn_readfirstlane(wave - 4);
    // W: forward -> k-half lane%2 of one of the wave's 32 weight rows;
    //    backward -> weight row q0 + 32 (pw/2) + lane/2, k-quarter
    //    2 (pw%2) + lane%2 of the output tile.
    // Either way lanes 2i and 2i+1 hold the two halves of one 64-weight block.
    // The LDS write path takes 8 lanes of a 16-byte store per cycle over a
    // 128-byte span of banks, and tile rows 2i and 2i+1 share a swizzle key.
    // Forward, lanes 8g..8g+7 therefore take rows of four different keys,
    // g%2 + 2(q + 4((g/2)%2)) + 16(g/4) with q = (lane/2)%4, so their stores
    // fall on 8 distinct 16-byte bank groups (with rows pt/2 every store
    // instruction took two passes).
    const int fwd_row = ((lane >> 3) & 1) + 2 * (((lane >> 1) & 3) + 4 * ((lane >> 4) & 1)) + 16 * (lane >> 5);
    const int w_r = kTransW ? (pw >> 1) * 32 + (lane >> 1) : pw * 32 + fwd_row;
    const int w_c = kTransW ? (2 * (pw & 1) + (lane & 1)) * 32 : (pt & 1) * 32;
    // table halves: lane h = lane % 2 converts the level pairs 2q + h; its own
    // pair is the low source of the byte permutes for h = 0, the high one for
    // h = 1
    const int hp = lane & 1;
    float lv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lv[2 * q] = hp ? L.v[4 * q + 2] : L.v[4 * q];
      lv[2 * q + 1] = hp ? L.v[4 * q + 3] : L.v[4 * q + 1];
    }
    const uint32_t sel_l = hp ? 0x02000604u : 0x06040200u;
    const uint32_t sel_h = hp ? 0x03010705u : 0x07050301u;
    // A resource: this tile's rows only (rows past M read as zeros)
    const __amdgpu_buffer_rsrc_t arsrc = make_rsrc(A + m0 * Qn, (M - m0 < kBM ? M - m0 : kBM) * Qn * 2);
    const __amdgpu_buffer_rsrc_t crsrc = make_rsrc(w.codes, w.n * K / 2);
    const __amdgpu_buffer_rsrc_t srsrc =
        kDQ ? make_rsrc(w.scale_codes, w.n * nbk) : make_rsrc(w.absmax, w.n * nbk * 4);
    const __amdgpu_buffer_rsrc_t grsrc = make_rsrc(w.group_scale, ((w.n * nbk + kGroup - 1) / kGroup) * 4);
    // A tile, global -> LDS without registers: load u of producer wave pw
    // fills the 1 KB of LDS rows 8 (8 pw + u) .. +7, lane l writing the 16
    // bytes of row l / 8, stored chunk l % 8, so it fetches the logical chunk
    // that the swizzle puts there. Offsets fit 32 bits: the host bounds Qn.
    int a_voff[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = (pw * 8 + u) * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ ((row >> 1) & 7);
      a_voff[u] = static_cast<int>((row * Qn + chunk * 8) * 2);
    }
    // per-step byte offsets: A moves by 64 columns; the weight moves along k
    // (forward) or by 64 rows (backward)
    const int64_t wrow0 = kTransW ? w_r : p0 + w_r;
    const int64_t wk0 = kTransW ? p0 + w_c : w_c;
    const int c_voff = static_cast<int>((wrow0 * K + wk0) / 2);
    const int s_voff = static_cast<int>(wrow0 * nbk + wk0 / 64);
    const int c_step = kTransW ? static_cast<int>(kBQ * K / 2) : kBQ / 2;
    const int s_step = kTransW ? static_cast<int>(kBQ * nbk) : 1;
    const bool wk_ok = wk0 < K;  // backward: the output tile may pass K

    // code ring, one slot per LDS stage: stage s's codes are held in slot
    // s % 3 from two steps before its unpack until it
    u32x4 rc[kStages];
    uint32_t rs[kStages];  // scale codes (double quant)
    float rg[kStages];     // group maxima (double quant) or absmax values

    // st = kt % kStages, a constant in every call below (the step loop
    // advances three steps at a time), so the LDS addresses fold
    auto dma_a = [&](int kt, int st) {
      uint16_t* as = As + st * kAStage + pw * (8 * 512);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(arsrc, (lds_void*)(as + u * 512), 16,
                                                 a_voff[u] + kt * kBQ * 2, 0, 0, 0);
    };
    auto load_w = [&](int kt, u32x4& c, uint32_t& sc, float& gs) {
      c = __builtin_amdgcn_raw_buffer_load_b128(crsrc, c_voff + kt * c_step, 0, 0);
      const int soff = s_voff + kt * s_step;
      if (kDQ) {
        sc = __builtin_amdgcn_raw_buffer_load_b8(srsrc, soff, 0, 0);
        gs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           grsrc, static_cast<int>((static_cast<uint32_t>(soff) / kGroup) * 4), 0, 0));
      } else {
        sc = 0;
        gs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srsrc, soff * 4, 0, 0));
      }
    };
    auto store_w = [&](int st, u32x4 c, uint32_t sc, float gs) {
      const float s = kDQ ? dq_unit(sc, w.dq) * gs : gs;
      // (backward: both halves of a block lie on the same side of K; the
      // forward's blocks are all inside it)
      const BlockLut lut = make_block_lut_pair<kF16>(lv, kTransW && !wk_ok ? 0.0f : s, sel_l, sel_h);
      uint16_t* bs = Bs + st * kBStage;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t wv[4];
        lut8_natural_order(lut, c[j], wv);
        if (kTransW) {
          // row n = w_r of the tile keeps the weight's orientation
          st16(bs + swz_t(w_r, (w_c >> 3) + j), u32x4{wv[0], wv[1], wv[2], wv[3]});
        } else {
          st16(bs + swz(w_r, (w_c >> 3) + j), u32x4{wv[0], wv[1], wv[2], wv[3]});
        }
      }
    };
    // Loads complete in issue order, so "at most the last kWLoads loads
    // outstanding" means that everything issued before this step's weight
    // loads -- in particular this step's A tile -- has landed in LDS.
    constexpr int kWLoads = kDQ ? 3 : 2;

    // prologue: A of stages 0 and 1 and unpacked W of stages 0 and 1 in LDS;
    // codes of stage 2 loaded, of stage 3 in flight
    dma_a(0, 0);
    dma_a(1, 1);
    load_w(0, rc[0], rs[0], rg[0]);
    load_w(1, rc[1], rs[1], rg[1]);
    store_w(0, rc[0], rs[0], rg[0]);
    load_w(2, rc[2], rs[2], rg[2]);
    store_w(1, rc[1], rs[1], rg[1]);
    load_w(3, rc[0], rs[0], rg[0]);
    // same state at the loop head from here and from the loop's back edge:
    // only the codes of the next stage outstanding
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kWLoads>();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // step kt: stage kt+2 into LDS (A by DMA, W unpacked from the codes
    // loaded two steps ago), then the codes of stage kt+4. Every step does
    // the same work, so the compiler sees one fixed sequence of loads: near
    // the end the stages past the last one are filled too, from zeros (reads
    // outside the buffer resources) or from unused in-range bytes, into LDS
    // slots that are read neither now nor later.
    // S = kt % 3: stage kt + 2 is unpacked from slot (S + 2) % 3, and the
    // codes of stage kt + 4 go to slot (S + 1) % 3, whose stage kt + 1 was
    // unpacked in the previous step.
    auto step = [&](int kt, auto s_c) {
      constexpr int S = decltype(s_c)::value;
      constexpr int st = (S + 2) % kStages, nx = (S + 1) % kStages;
      dma_a(kt + 2, st);
      store_w(st, rc[st], rs[st], rg[st]);
      load_w(kt + 4, rc[nx], rs[nx], rg[nx]);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<kWLoads>();
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();
    };
    static_assert(kStages == 3, "the step loop advances one ring turn at a time");
    for (int kt = 0; kt < nk; kt += 3) {
      step(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
      if (kt + 2 < nk) step(kt + 2, std::integral_constant<int, 2>{});
    }
    // no load may still be writing LDS when the wave ends
    wait_vmcnt<0>();
    return;
  }

  // ======================= consumers =======================
  const int i = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wp = wave & 1;
  const int sw = (i >> 1) & 7;
  // element offsets (within a stage row) of this lane's fragment chunk, per half-step
  const int col0 = ((0 + g) ^ sw) << 3, col1 = ((4 + g) ^ sw) << 3;
  const int arow = (wm * 128 + i) * kBQ, brow = (wp * 64 + i) * kBQ;
  // backward: the first operand of the MFMA is column k0 + i of the [n][k]
  // tile, contraction slots n = 32 half + 8g + e'. Lane 16g + 4t + p supplies
  // the address of row 32 half + 8g + t (then + 4) at columns k0 + 4p .. +3
  // (k0 = 64 wp + 16 nt): logical chunk 8 wp + 2 nt + p / 2, in quarter
  // 2 wp + nt / 2; with swz_t_key(n) = 2t + 8 (g & 1) (and the odd quarters'
  // pair swap) the stored chunk is
  // ((p / 2) ^ (nt / 2)) | ((nt ^ t) << 1) | ((wp ^ (g & 1)) << 3).
  int toff[4] = {0, 0, 0, 0};
  if (kTransW) {
    const int tp = i & 3, tt = i >> 2;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      toff[nt] = (8 * g + tt) * kBP + 8 * (((tp >> 1) ^ (nt >> 1)) | ((nt ^ tt) << 1) | ((wp ^ (g & 1)) << 3)) +
                 4 * (tp & 1);
  }

  f32x4 acc[4][8];  // [weight tile nt][token tile mt]: acc = W x^T tile
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // two register sets of fragments: while the MFMAs of one half-step run,
  // the other set is filled from LDS
  u32x4 fa0[8], fb0[4], fa1[8], fb1[4];
  // st = kt % kStages, a constant in every call (the loop below advances
  // three steps at a time)
  auto read = [&](int st, int half, u32x4(&xa)[8], u32x4(&xb)[4]) {
    const int col = half ? col1 : col0;
    const uint16_t* as = As + st * kAStage + arow + col;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) xa[mt] = ld16(as + 16 * mt * kBQ);
    if (kTransW) {
      const uint16_t* bs = Bs + st * kBStage + half * (32 * kBP);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const u32x2 lo = ld_tr4(bs + toff[nt]), hi = ld_tr4(bs + toff[nt] + 4 * kBP);
        xb[nt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    } else {
      const uint16_t* bs = Bs + st * kBStage + brow + col;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) xb[nt] = ld16(bs + 16 * nt * kBQ);
    }
  };
  auto mma = [&](const u32x4(&xa)[8], const u32x4(&xb)[4]) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = mma16<kF16>(xb[nt], xa[mt], acc[nt][mt]);
  };

  auto cstep = [&](int kt, auto s_c) {
    constexpr int S = decltype(s_c)::value;  // kt % 3
    read(S, 1, fa1, fb1);                                       // second half of this step
    mma(fa0, fb0);                                              // first half
    if (kt + 1 < nk) read((S + 1) % kStages, 0, fa0, fb0);      // next step, written two steps ago
    mma(fa1, fb1);                                              // second half
    __syncthreads();
  };
  __syncthreads();
  read(0, 0, fa0, fb0);
  for (int kt = 0; kt < nk; kt += 3) {
    cstep(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < nk) cstep(kt + 1, std::integral_constant<int, 1>{});
    if (kt + 2 < nk) cstep(kt + 2, std::integral_constant<int, 2>{});
  }

  // LoRA term: rpad more contraction slots, operands straight from global memory.
  // Grouped forward: the output columns are lp.g parts (tiles never straddle
  // two) and part l only sees slots l rpart .. (l+1) rpart - 1, which carry its
  // own H; row p of ep_b holds that part's B row.
  int slot_shift = 0;
  if (!kTransW) {
    int part = 0;
#pragma unroll
    for (int l = 0; l < 3; ++l) part += (l + 1 < lp.g && p0 >= lp.end[l]) ? 1 : 0;
    slot_shift = part * lp.rpart;
  }
  for (int ks = 0; ks < rpad / 32; ++ks) {
    u32x4 xa[8], xb[4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int64_t m = m0 + wm * 128 + 16 * mt + i;
      xa[mt] = ld16(ep_a + (m < M ? m : M - 1) * rpad + 32 * ks + 8 * g);  // rows past M are never stored
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t p = p0 + wp * 64 + 16 * nt + i;
      xb[nt] = (p < P) ? ld8_bf16_window(ep_b + p * ep_ld, 32 * ks + 8 * g - slot_shift, ep_lim, (ep_ld % 8) == 0)
                       : u32x4{0, 0, 0, 0};
    }
    mma(xa, xb);
  }

  // Output through LDS: the ring is free after the last step's barrier (no
  // copy is in flight any more), so each consumer wave stages its 128 x 64
  // bf16 sub-tile there (rows padded to 72 elements: the 16 rows of one
  // 8-byte store land in distinct banks) and writes it back as whole
  // 128-byte row runs, 16 bytes per lane. Lane holds out[m = .. + i][p = .. + 4g .. 4g+3].
  constexpr int kEpRow = 72;
  uint16_t* ep = As + wave * (128 * kEpRow);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const f32x4 c = acc[nt][mt];
      *reinterpret_cast<u32x2*>(ep + (16 * mt + i) * kEpRow + 16 * nt + 4 * g) =
          u32x2{cvt_16x2<kF16>(c[0], c[1]), cvt_16x2<kF16>(c[2], c[3])};
    }
  const int rr = lane >> 3, cc = lane & 7;
  const int64_t pcol = p0 + wp * 64 + 8 * cc;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int row = 8 * it + rr;
    const u32x4 v = ld16(ep + row * kEpRow + 8 * cc);
    const int64_t m = m0 + wm * 128 + row;
    if (m < M && pcol < P) *reinterpret_cast<u32x4*>(out + m * P + pcol) = v;  // P % 16 == 0: a run of 8 is whole
  }
}

unsigned tiles(int64_t m, int64_t p) { return static_cast<unsigned>(((m + kBM - 1) / kBM) * ((p + kBP - 1) / kBP)); }

}  // namespace

hipError_t launch_gemm_fwd(const PackedW& w, const uint16_t* x, int64_t m, const uint16_t* hs, const uint16_t* b,
                           int r, int rpad, const LoraParts& parts, uint16_t* y, hipStream_t st, bool f16) {
  auto kern = f16 ? (w.dq ? nf4_gemm_kernel<false, true, true> : nf4_gemm_kernel<false, false, true>)
                  : (w.dq ? nf4_gemm_kernel<false, true, false> : nf4_gemm_kernel<false, false, false>);
  hipLaunchKernelGGL(kern, dim3(tiles(m, w.n)), dim3(512), 0, st, w, x, m, w.n, w.k, hs, b, static_cast<int64_t>(r), r,
                     rpad, parts, y, codebook_table(w.codebook));
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const PackedW& w, const uint16_t* dy, int64_t m, const uint16_t* dhs, const uint16_t* at,
                          int rpad, uint16_t* dx, hipStream_t st, bool f16) {
  auto kern = f16 ? (w.dq ? nf4_gemm_kernel<true, true, true> : nf4_gemm_kernel<true, false, true>)
                  : (w.dq ? nf4_gemm_kernel<true, true, false> : nf4_gemm_kernel<true, false, false>);
  hipLaunchKernelGGL(kern, dim3(tiles(m, w.k)), dim3(512), 0, st, w, dy, m, w.k, w.n, dhs, at,
                     static_cast<int64_t>(rpad), rpad, rpad, LoraParts{}, dx, codebook_table(w.codebook));
  return hipGetLastError();
}

}  // namespace qlora
