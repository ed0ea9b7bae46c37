// Decode path, one or two tokens and k <= 12288: Y = X W16^T + s H B^T with
// W read straight from its packed NF4 form (3 to 16 tokens, and k > 12288:
// gemv_mfma.hip).
//
// Ultralytics glossary "QLoRA", section "Come funziona QLoRA": each frozen
// layer restores its weights as level[code] * block scale, in bfloat16,
// right before the matmul, and adds the LoRA path ("LoRA y QLoRA en
// Profundidad", "La Idea Central": H = X A^T, then (alpha / r) H B^T). At one
// or two tokens the layer is bound by the HBM stream of the packed weight
// (0.5 B of codes + 1/64 B of scale codes per weight) and by how few vector
// instructions per weight the kernel spends on it:
//   * the 16-entry codebook is expanded once per workgroup into a 256-entry
//     LDS table indexed by a whole code byte: entry e holds the two 16-bit
//     levels of its nibbles (low nibble -> low half), so one byte-permute (to
//     form the address) and one LDS read give two weights. The table is
//     stored 64 times, interleaved, and lane l reads copy l, so the 64 lanes
//     of a read always hit 64 different banks;
//   * the per-block scale is applied to the block's float32 partial sum,
//     after the products of X with the 16-bit levels. In exact arithmetic
//     that is sum_k x_k L[c_k] s_b, the restored weight; the operand carries
//     the 16-bit rounding of the level rather than of level * scale (relative
//     difference at most 2^-8 per weight, inside the layer's 1e-2 bound);
//   * one wave per weight row, 2-wide dot products on the vector ALU, no
//     partial sums across waves; H = X A^T (r <= 32, or 16 slots per part
//     for grouped weights) is computed by every workgroup for the slots it
//     needs, in the prologue; above that, H arrives as split partial sums of
//     the decode projection kernel.
#include <type_traits>

#include "bufmem.h"
#include "internal.h"
#include "mfma.h"
#include "nf4_lut.h"

namespace qlora {
namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kTabBytes = 256 * 64 * 4;          // 256 code bytes x 64 lane copies x 4 B
constexpr int kNontemporal = 2;                   // cache-policy bits of a buffer load: nt
struct GemvArgs {
  PackedW w;
  const uint16_t* x;
  int M;
  const uint16_t* a;   // fused H: the A rows (r x k, or g rpart x k)
  int rh;              // rows of A / slots of H in total
  const float* hpart;  // partial-sum H: hsplits x M x rh float32
  int hsplits;
  const uint16_t* b;   // n x rb
  int rb;              // slots per output row (r, or rpart)
  LoraParts P;
  float s;
  uint16_t* y;
  float* h_out;
  Levels L;
};

__device__ __forceinline__ int part_of(const LoraParts& P, int row) {
  int l = 0;
#pragma unroll
  for (int q = 0; q + 1 < 4; ++q) l += (q + 1 < P.g && row >= P.end[q]) ? 1 : 0;
  return l;
}

__device__ __forceinline__ int part_begin(const LoraParts& P, int l) { return l == 0 ? 0 : P.end[l - 1]; }

// 16-bit level c of the table (bf16 or IEEE half, round to nearest even).
template <bool kF16>
__device__ __forceinline__ uint32_t level16(const Levels& L, int c) {
  float v = L.v[0];
#pragma unroll
  for (int q = 1; q < 16; ++q) v = (c == q) ? L.v[q] : v;
  return to16<kF16>(v);
}

// The pair table: dword (e * 64 + copy) = level16(e & 15) | level16(e >> 4) << 16.
// Thread tid writes dwords tid + 1024 i, i = 0..15: entry e = wave + 16 i,
// so its low nibble is the (uniform) wave index and its high nibble is i.
template <bool kF16>
__device__ __forceinline__ void build_pair_table(unsigned char* tab, const Levels& L, int tid, int wv) {
  const uint32_t lo = level16<kF16>(L, wv);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const uint32_t hi = level16<kF16>(L, q);
    *reinterpret_cast<uint32_t*>(tab + 4 * (tid + kThreads * q)) = lo | (hi << 16);
  }
}

// 8 weights (one dword of codes: element 2b in the low nibble of byte b) as
// four dwords of 16-bit levels in natural order, from the pair table. The
// byte-permute forms the LDS address (code byte << 8) | (lane << 2).
__device__ __forceinline__ u32x4 lookup8(const unsigned char* tab, uint32_t cw, uint32_t lane4) {
  u32x4 r;
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    const uint32_t addr = __builtin_amdgcn_perm(cw, lane4, 0x0C0C0400u | ((4u + bb) << 8));
    r[bb] = *reinterpret_cast<const uint32_t*>(tab + addr);
  }
  return r;
}

// Buffer resources of one call: out-of-range offsets read zeros.
struct Rsrc {
  __amdgpu_buffer_rsrc_t codes, sc, gs, am, x, a, b, hp;
  int codes_oob, x_oob, a_oob, b_oob, hp_oob;
};

__device__ __forceinline__ Rsrc make_rsrcs(const GemvArgs& g, int nbk) {
  Rsrc R;
  const int N = static_cast<int>(g.w.n), K = static_cast<int>(g.w.k);
  const int nb = N * nbk;
  R.codes_oob = N * (K / 2);
  R.codes = make_rsrc(g.w.codes, R.codes_oob);
  R.sc = make_rsrc(g.w.scale_codes, g.w.dq ? nb : 0);
  R.gs = make_rsrc(g.w.group_scale, g.w.dq ? 4 * ((nb + 255) / 256) : 0);
  R.am = make_rsrc(g.w.absmax, g.w.dq ? 0 : 4 * nb);
  R.x_oob = g.M * K * 2;
  R.x = make_rsrc(g.x, R.x_oob);
  R.a_oob = g.rh * K * 2;
  R.a = make_rsrc(g.a, g.a != nullptr ? R.a_oob : 0);
  R.b_oob = N * g.rb * 2;
  R.b = make_rsrc(g.b, g.b != nullptr ? R.b_oob : 0);
  R.hp_oob = g.hsplits * g.M * g.rh * 4;
  R.hp = make_rsrc(g.hpart, g.hpart != nullptr ? R.hp_oob : 0);
  return R;
}

// H from split partial sums (hsplits x M x rh float32). Thread t takes
// output o = t % (M rh) and the splits grp, grp + groups, ... (grp = t /
// (M rh), at most eight each), issued in the prologue with the other early
// loads; the group sums meet in the partial-sum area and are added in group
// order: a fixed order, so results do not depend on scheduling.
struct HPart {
  float v[8];
  bool fast;
  int groups;
};

__device__ __forceinline__ HPart issue_hpart(const GemvArgs& g, const Rsrc& R, int tid) {
  HPart H;
  const int mr = g.M * g.rh;
  H.groups = mr <= kThreads ? kThreads / mr : 0;
  if (H.groups > g.hsplits) H.groups = g.hsplits;
  H.fast = H.groups > 0 && g.hsplits <= 8 * H.groups;
  const int o = H.fast ? tid % mr : 0, grp = H.fast ? tid / mr : 0;
  const bool active = H.fast && grp < H.groups;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int sp = grp + H.groups * u;
    const int off = (active && sp < g.hsplits) ? 4 * (sp * mr + o) : R.hp_oob;
    H.v[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(R.hp, off, 0, 0));
  }
  return H;
}

// Before a barrier: the group sums into the partial-sum area, from float
// offset off.
__device__ __forceinline__ void put_hpart(const GemvArgs& g, float* red, const HPart& H, int tid) {
  const int mr = g.M * g.rh;
  if (H.fast && tid < H.groups * mr) {
    float v = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u) v += H.v[u];
    red[tid] = v;
  }
}

// Calls f(integral_constant<int, t>) for t = T .. E-1.
template <int T, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (T < E) {
    f(std::integral_constant<int, T>{});
    static_for<T + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// m <= 2 tokens, k <= 4096: one wave per weight row.
//
// Lane l takes the 32 weights [2048 h + 32 l, 2048 h + 32 l + 32) of the row
// for h = 0, 1: each code load is a whole 1 KB run of the row (16 bytes per
// lane), the lane's weights are half of block 32 h + l / 2 (one scale each),
// and the products are 2-wide dot products (v_dot2_f32_bf16) with X held in
// registers in the same order; per half block the float32 sum is multiplied
// by the block scale. The LoRA-up term enters as lane j's share s H[j] B[row][j]
// (j < rb), and one wave sum (DPP, then the four row sums) gives the output. No
// partial sums cross waves: the only barriers are the pair table's and H's.
// H (fused, up to 32 slots) is one contiguous A row per wave, read in whole
// 1 KB runs and dotted with X read from LDS in the same order.
// X is held in registers for k <= 4096 (two 2048-wide halves) and read from
// LDS per row for k <= 12288 (six halves)
constexpr int kHalvesReg = 2;
constexpr int kHalvesLds = 6;
constexpr int kRowsX = 2 * 2 * 2048 * kHalvesLds;  // X staging: up to 2 tokens x 12288 bf16
constexpr int kRowsH = 2 * QLORA_MAX_RANK;  // H: up to 2 tokens x 128 slots
constexpr int kRowsSmem = kTabBytes + kRowsX + 4 * kRowsH + 4 * kThreads;

// v + (v moved across lanes by the DPP control kCtrl)
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false);
  return v + __builtin_bit_cast(float, s);
}

// Sum over the 64 lanes, returned in every lane: quad sums and 16-lane row
// sums by DPP (no LDS round trip), then the four row sums read as scalars.
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_add<0x124>(v);  // row_ror 4
  v = dpp_add<0x128>(v);  // row_ror 8
  const int bits = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(bits, 48));
  return (r0 + r1) + (r2 + r3);
}

template <bool kF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (kF16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c, false);
  }
}

// Loads of one weight row for lane l (one 1 KB run per 2048-wide half, the
// halves' scale codes or absmax values, the row's two candidate group scales,
// B[row][l]).
template <int kNH>
struct RowLoads {
  u32x4 c[kNH];
  uint32_t s[kNH];  // scale code bytes (DQ) or absmax bits
  u32x2 gs;         // group scales of (row nbk) >> 8 and the next (DQ)
  uint32_t b;       // B[row][lane] for lane < rb
};

// 2 kNH + 2 vector loads in every form: the code runs, the scale codes (or
// absmax values), the group scales (a second B load without double
// quantization), B; the prologue's explicit wait counts on it. Halves past
// k read zeros from out-of-range offsets, so the count never changes.
template <int kNH>
constexpr int row_loads() {
  return 2 * kNH + 2;
}

template <bool kDQ, int kNH>
__device__ __forceinline__ void load_row(RowLoads<kNH>& L, const Rsrc& R, const GemvArgs& g, int row, int lane, int K,
                                         int nbk) {
  // the codes are read once per call: streaming (nontemporal) loads, which
  // measured 3-6% faster than plain ones on every one-token shape
#pragma unroll
  for (int h = 0; h < kNH; ++h) {
    const int k0 = 2048 * h + 32 * lane;
    const int off = k0 < K ? row * (K / 2) + (k0 >> 1) : R.codes_oob;
    L.c[h] = __builtin_amdgcn_raw_buffer_load_b128(R.codes, off, 0, kNontemporal);
  }
#pragma unroll
  for (int h = 0; h < kNH; ++h) {
    const int blk = 32 * h + (lane >> 1);
    if (kDQ) {
      L.s[h] = __builtin_amdgcn_raw_buffer_load_b8(R.sc, blk < nbk ? row * nbk + blk : 0x7FFFFFF0, 0, 0);
    } else {
      L.s[h] = __builtin_amdgcn_raw_buffer_load_b32(R.am, blk < nbk ? 4 * (row * nbk + blk) : 0x7FFFFFF0, 0, 0);
    }
  }
  if (kDQ) {
    L.gs = __builtin_amdgcn_raw_buffer_load_b64(R.gs, 4 * ((row * nbk) >> 8), 0, 0);
  } else {
    L.gs = __builtin_amdgcn_raw_buffer_load_b64(R.b, R.b_oob, 0, 0);  // stand-in: same load count
  }
  L.b = __builtin_amdgcn_raw_buffer_load_b16(R.b, lane < g.rb ? 2 * (row * g.rb + lane) : R.b_oob, 0, 0);
}

// kXL: k up to 12288, X read from LDS for every row (no fused H); otherwise
// k up to 4096 with X in registers.
template <bool kF16, bool kDQ, int kM, int kH, int kRPW, bool kXL>
__global__ __launch_bounds__(kThreads) void gemv_rows_kernel(GemvArgs g) {
  static_assert(kM == 1 || kM == 2, "one or two tokens");
  static_assert(!(kXL && kH == 1), "H is fused only with X in registers");
  constexpr int kNH = kXL ? kHalvesLds : kHalvesReg;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kRowsSmem];
  unsigned char* tab = smem;
  unsigned char* xst = smem + kTabBytes;
  float* hl = reinterpret_cast<float*>(smem + kTabBytes + kRowsX);
  float* scratch = reinterpret_cast<float*>(smem + kTabBytes + kRowsX + 4 * kRowsH);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lane4 = static_cast<uint32_t>(lane) << 2;
  const int K = static_cast<int>(g.w.k), N = static_cast<int>(g.w.n);
  const int nbk = K >> 6;
  const int row0 = blockIdx.x * (kWaves * kRPW);
  const int row_end = row0 + kWaves * kRPW < N ? row0 + kWaves * kRPW : N;
  const Rsrc rs = make_rsrcs(g, nbk);
  const int dq_mode = g.w.dq;
  // row of step q (stand-ins past the end reload the last row)
  auto row_of = [&](int q) {
    const int r = row0 + wv + kWaves * q;
    return r < N ? r : N - 1;
  };

  // X into LDS in the order of the lanes' weights: copy t = (tok, h, c)
  // holds, for every lane l, the 8 values X[tok][2048 h + 32 l + 8 c ..], so
  // each later fragment read is one contiguous 1 KB (no bank conflicts).
  // At most 2 tokens x 6 halves x 4 copies, up to three per wave.
  const int nh = (K + 2047) >> 11;
  const int ncopy = kM * nh * 4;
  for (int t = wv; t < ncopy; t += kWaves) {
    const int tok = t / (nh * 4), h = (t >> 2) % nh, c = t & 3;
    const int kk = 2048 * h + 32 * lane + 8 * c;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs.x, (lds_void*)(xst + t * 1024), 16,
                                             kk < K ? (tok * K + kk) * 2 : rs.x_oob, 0, 0, 0);
  }
  // the first rows' loads, so that HBM is busy while the table is built;
  // two rows ahead per wave (three or more in flight made every shape
  // slower, one made the multi-row shapes slower)
  constexpr int kAheadMax = 2;
  constexpr int kAhead = kRPW < kAheadMax ? kRPW : kAheadMax;
  RowLoads<kNH> rl[kRPW];
  static_for<0, kAhead>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    __builtin_amdgcn_sched_barrier(0);
    load_row<kDQ, kNH>(rl[q], rs, g, row_of(q), lane, K, nbk);
    __builtin_amdgcn_sched_barrier(0);
  });
  build_pair_table<kF16>(tab, g.L, tid, wv);
  // this wave's X copy has landed (it was issued before the row loads: the
  // compiler does not track global -> LDS copies, so the count is explicit)
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<kAhead * row_loads<kNH>()>();
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  // X staging offset of (tok, h, c) for lane l: ((tok nh + h) 4 + c) 1024 + 16 l
  auto xoff = [&](int tok, int kk) {
    const int h = kk >> 11, l = (kk & 2047) >> 5, c = (kk & 31) >> 3;
    return ((tok * nh + h) * 4 + c) * 1024 + 16 * l;
  };

  // H's slots for this workgroup: [s0, s0 + ns); wave w takes slot s0 + w
  // (and s0 + 16 + w when ns > 16)
  int s0 = 0, ns = 0, hl0 = 0;
  bool own_out = blockIdx.x == 0;
  if (kH == 1) {
    if (g.P.g > 1) {
      const int l0 = part_of(g.P, row0), l1 = part_of(g.P, row_end - 1);
      s0 = l0 * g.rb;
      ns = (l1 - l0 + 1) * g.rb;
      hl0 = l0;
    } else {
      ns = g.rh;
    }
  }
  // A row of slot j in whole 1 KB runs: lane l holds 8 values of every run
  auto load_a = [&](u32x4 (&af)[8], int j) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int off = q * 1024 + lane * 16;
      af[q] = __builtin_amdgcn_raw_buffer_load_b128(rs.a, off < K * 2 ? j * K * 2 + off : rs.a_oob, 0, 0);
    }
  };
  u32x4 af[8];
  const bool has_slot = kH == 1 && wv < ns;
  if (has_slot) load_a(af, s0 + wv);

  HPart HP{};
  if (kH == 2) HP = issue_hpart(g, rs, tid);

  // H: dot of the A row with X read from LDS in the same order
  auto h_slot = [&](int j) {
#pragma unroll
    for (int tok = 0; tok < kM; ++tok) {
      float p = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int kk = 512 * q + 8 * lane;
        u32x4 xv = u32x4{0, 0, 0, 0};
        if (kk < K) xv = *reinterpret_cast<const u32x4*>(xst + xoff(tok, kk));
#pragma unroll
        for (int d = 0; d < 4; ++d) p = dot2<kF16>(af[q][d], xv[d], p);
      }
      p = wave_sum(p);
      if (lane == 0) {
        hl[tok * 32 + (j - s0)] = p;
        if (g.h_out != nullptr) {
          // single linear: the first workgroup writes H; grouped: the
          // workgroup that holds the part's first row
          bool own = own_out;
          if (g.P.g > 1) {
            const int l = j / g.rb, pb = part_begin(g.P, l);
            own = pb >= row0 && pb < row_end;
          }
          if (own) g.h_out[tok * g.rh + j] = p;
        }
      }
    }
  };
  if (has_slot) {
    h_slot(s0 + wv);
    if (wv + kWaves < ns) {
      load_a(af, s0 + kWaves + wv);
      h_slot(s0 + kWaves + wv);
    }
  }
  if (kH == 2) put_hpart(g, scratch, HP, tid);
  __syncthreads();
  if (kH == 2) {
    // H from the split partial sums into hl[tok * rh + j]
    const int mr = g.M * g.rh;
    for (int idx = tid; idx < mr; idx += kThreads) {
      float hv = 0.0f;
      if (HP.fast) {
        for (int grp = 0; grp < HP.groups; ++grp) hv += scratch[grp * mr + idx];
      } else {
#pragma unroll 8
        for (int sp = 0; sp < g.hsplits; ++sp) hv += g.hpart[sp * mr + idx];
      }
      hl[idx] = hv;
      if (g.h_out != nullptr && blockIdx.x == 0) g.h_out[idx] = hv;
    }
    __syncthreads();
  }

  // X in registers (k <= 4096), in the order of the lane's weights (zeros
  // past K); with kXL each row reads its fragments from LDS instead
  u32x4 xr[kM][kHalvesReg][4];
  if constexpr (!kXL) {
#pragma unroll
    for (int tok = 0; tok < kM; ++tok)
#pragma unroll
      for (int h = 0; h < kHalvesReg; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          xr[tok][h][c] = h < nh ? *reinterpret_cast<const u32x4*>(xst + ((tok * nh + h) * 4 + c) * 1024 + 16 * lane)
                                 : u32x4{0, 0, 0, 0};
  }
  const int hstride = kH == 1 ? 32 : g.rh;

  static_for<0, kRPW>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    if constexpr (q >= 1 && q + kAhead - 1 < kRPW) {
      __builtin_amdgcn_sched_barrier(0);
      load_row<kDQ, kNH>(rl[q + kAhead - 1], rs, g, row_of(q + kAhead - 1), lane, K, nbk);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int row = row0 + wv + kWaves * q;
    if (row < N) {
      const RowLoads<kNH>& L = rl[q];
      float acc[kM];
#pragma unroll
      for (int tok = 0; tok < kM; ++tok) acc[tok] = 0.0f;
#pragma unroll
      for (int h = 0; h < kNH; ++h) {
        if (h < nh) {
          float p[kM];
#pragma unroll
          for (int tok = 0; tok < kM; ++tok) p[tok] = 0.0f;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const u32x4 wv4 = lookup8(tab, L.c[h][d], lane4);
#pragma unroll
            for (int tok = 0; tok < kM; ++tok) {
              const u32x4 xv = kXL ? *reinterpret_cast<const u32x4*>(xst + ((tok * nh + h) * 4 + d) * 1024 + 16 * lane)
                                   : xr[tok][h < kHalvesReg ? h : 0][d];
#pragma unroll
              for (int e = 0; e < 4; ++e) p[tok] = dot2<kF16>(wv4[e], xv[e], p[tok]);
            }
          }
          const int blk = 32 * h + (lane >> 1);
          float sc;
          if (kDQ) {
            const int grp = (row * nbk + blk) >> 8;
            const float gsv = __builtin_bit_cast(float, grp == ((row * nbk) >> 8) ? L.gs[0] : L.gs[1]);
            sc = dq_unit(L.s[h] & 0xFFu, dq_mode) * gsv;
          } else {
            sc = __builtin_bit_cast(float, L.s[h]);
          }
          sc = blk < nbk ? sc : 0.0f;
#pragma unroll
          for (int tok = 0; tok < kM; ++tok) acc[tok] = fmaf(sc, p[tok], acc[tok]);
        }
      }
      if (kH != 0 && lane < g.rb) {
        // lane j's share of s H B^T: the slot of this row's part
        int off;
        if (kH == 1) {
          off = g.P.g > 1 ? (part_of(g.P, row) - hl0) * g.rb : 0;
        } else {
          off = g.P.g > 1 ? part_of(g.P, row) * g.rb : 0;
        }
        const float bj = to_f32<kF16>(static_cast<uint16_t>(L.b));
#pragma unroll
        for (int tok = 0; tok < kM; ++tok) acc[tok] = fmaf(g.s * hl[tok * hstride + off + lane], bj, acc[tok]);
      }
#pragma unroll
      for (int tok = 0; tok < kM; ++tok) {
        const float v = wave_sum(acc[tok]);
        if (lane == 0) g.y[static_cast<int64_t>(tok) * N + row] = to16<kF16>(v);
      }
    }
  });
}

}  // namespace

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

bool gemv_fuses_h(int64_t m, int64_t k, int r, const LoraParts* parts) {
  if (r <= 0) return false;
  // 3 to 16 tokens, or k > 12288 (the matrix-core kernels of
  // gemv_mfma.hip): up to 16 slots
  if (m > 2 || k > 2048 * kHalvesLds) return r <= 16;
  // one or two tokens with X read from LDS per row: H from partial sums
  if (k > 2048 * kHalvesReg) return false;
  const bool grouped = parts != nullptr && parts->g > 1;
  return grouped ? parts->rpart <= 16 : r <= 32;
}

namespace {

template <bool kF16, bool kDQ, int kM, int kRPW>
void launch_rows_rpw(const GemvArgs& g, int kh, hipStream_t st) {
  const unsigned grid = static_cast<unsigned>((g.w.n + kWaves * kRPW - 1) / (kWaves * kRPW));
  if (g.w.k > 2048 * kHalvesReg) {  // H from partial sums here (kh is 0 or 2)
    auto kern = kh == 0 ? gemv_rows_kernel<kF16, kDQ, kM, 0, kRPW, true> : gemv_rows_kernel<kF16, kDQ, kM, 2, kRPW, true>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, st, g);
    return;
  }
  auto kern = kh == 0   ? gemv_rows_kernel<kF16, kDQ, kM, 0, kRPW, false>
              : kh == 1 ? gemv_rows_kernel<kF16, kDQ, kM, 1, kRPW, false>
                        : gemv_rows_kernel<kF16, kDQ, kM, 2, kRPW, false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, st, g);
}

// rows per wave for the one-wave-per-row form: enough waves for one
// workgroup per CU
template <bool kF16, bool kDQ, int kM>
void launch_rows(const GemvArgs& g, int kh, hipStream_t st) {
  const int64_t per = (g.w.n + int64_t(kWaves) * device_cus() - 1) / (int64_t(kWaves) * device_cus());
  if (per <= 1) {
    launch_rows_rpw<kF16, kDQ, kM, 1>(g, kh, st);
  } else if (per <= 2) {
    launch_rows_rpw<kF16, kDQ, kM, 2>(g, kh, st);
  } else if (per <= 3) {
    launch_rows_rpw<kF16, kDQ, kM, 3>(g, kh, st);
  } else if (per <= 4) {
    launch_rows_rpw<kF16, kDQ, kM, 4>(g, kh, st);
  } else if (per <= 6) {
    launch_rows_rpw<kF16, kDQ, kM, 6>(g, kh, st);
  } else {
    launch_rows_rpw<kF16, kDQ, kM, 8>(g, kh, st);
  }
}

template <bool kF16, bool kDQ>
hipError_t launch_gemv_dq(const GemvArgs& g, int kh, hipStream_t st) {
  if (g.M == 1) {
    launch_rows<kF16, kDQ, 1>(g, kh, st);
  } else {
    launch_rows<kF16, kDQ, 2>(g, kh, st);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const PackedW& w, const uint16_t* x, int64_t m, const uint16_t* a, const float* hpart,
                       int hsplits, const uint16_t* b, int r, float s, uint16_t* y, float* h_out, hipStream_t st,
                       bool f16, const LoraParts* parts) {
  if (m < 1 || m > 16 || w.n % 16 != 0 || w.k % 64 != 0 || r < 0 || r > QLORA_MAX_RANK) return hipErrorInvalidValue;
  if (m > 2 || w.k > 2048 * kHalvesLds) return launch_gemv_mfma(w, x, m, a, hpart, hsplits, b, r, s, y, h_out, st, f16, parts);
  GemvArgs g;
  g.w = w;
  g.x = x;
  g.M = static_cast<int>(m);
  g.a = a;
  g.rh = r;
  g.hpart = hpart;
  g.hsplits = hsplits;
  g.b = b;
  if (parts != nullptr && parts->g > 1) {
    g.P = *parts;
    g.rb = parts->rpart;
  } else {
    g.P = LoraParts{};
    g.P.g = 1;
    g.P.rpart = r;
    g.P.end[0] = static_cast<int>(w.n);
    g.rb = r;
  }
  g.s = s;
  g.y = y;
  g.h_out = h_out;
  g.L = codebook_table(w.codebook);
  const bool fuse = gemv_fuses_h(m, w.k, r, parts);
  if (r > 0 && !fuse && hpart == nullptr) return hipErrorInvalidValue;
  const int kh = r == 0 ? 0 : (fuse ? 1 : 2);
  if (f16) return w.dq ? launch_gemv_dq<true, true>(g, kh, st) : launch_gemv_dq<true, false>(g, kh, st);
  return w.dq ? launch_gemv_dq<false, true>(g, kh, st) : launch_gemv_dq<false, false>(g, kh, st);
}

}  // namespace qlora
