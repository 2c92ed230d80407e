// Weight-streaming GEMM for decode-shaped (skinny) activations on gfx950.
//
//   Y[m, o] = s[o] * sum_k X[m, k] * W[o, k]        W: out x in, K contiguous
//
// At M <= 64 tokens the work is bound by reading W from HBM once (264 MB per
// shared-expert layer), so the kernel is organised around that stream:
//   * a workgroup owns RT 16-row tiles of W and a K range; its 4 waves split
//     the range in 64-element steps (wave w takes steps w, w+4, ...), so the
//     workgroup reads 4 * 64 contiguous K of every row at a time;
//   * every lane loads 16 contiguous weight bytes per row tile per step
//     (lane = 16 rows x 4 K-groups), two steps ahead of the MFMAs;
//   * FP8 E4M3FN codes are widened to BF16 in registers (exact: every E4M3FN
//     value is a BF16 value) and multiplied on the matrix cores with
//     v_mfma_f32_16x16x32_bf16 against the BF16 activations, fp32 accumulate.
//     The A and B operands use the same K permutation, so any K order inside
//     a step is consistent;
//   * the per-row scale is applied once to the fp32 sum (the weight-sharding
//     page's loading section keeps FP8 scales outside the flat buffer);
//   * the 4 waves' partial sums are added in LDS; with more than one K split
//     per row tile the workgroups write fp32 partials that a small finalize
//     kernel adds in split order.
// The MLP's gate_up projection runs in a fused mode: a workgroup owns gate
// rows j..j+8RT and the matching up rows I+j..I+j+8RT, and writes
// h = bf16(silu(G_gate) * G_up) directly (vLLM PR #50656 report, test code:
// gate rows first, SiLU of the gate half times the up half).
#include "gemm_common.h"

namespace swr {
namespace {

// Per-lane weight data of one step for one 16-row tile: 16 K elements.
template <bool FP8>
struct WFrag;
template <>
struct WFrag<true> {
  u32x4 v;
};
template <>
struct WFrag<false> {
  u32x4 v[2];
};

template <bool FP8>
__device__ inline void load_w(WFrag<FP8>& f, const uint8_t* p);
template <>
__device__ inline void load_w<true>(WFrag<true>& f, const uint8_t* p) {
  f.v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
template <>
__device__ inline void load_w<false>(WFrag<false>& f, const uint8_t* p) {
  f.v[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  f.v[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
}

template <bool FP8>
__device__ inline void to_operands(const WFrag<FP8>& f, bf16x8& a0, bf16x8& a1);
template <>
__device__ inline void to_operands<true>(const WFrag<true>& f, bf16x8& a0, bf16x8& a1) {
  a0 = fp8x8_to_bf16(f.v[0], f.v[1]);
  a1 = fp8x8_to_bf16(f.v[2], f.v[3]);
}
template <>
__device__ inline void to_operands<false>(const WFrag<false>& f, bf16x8& a0, bf16x8& a1) {
  a0 = as_bf16x8(f.v[0]);
  a1 = as_bf16x8(f.v[1]);
}

template <int MT, int RT, bool FP8>
struct Step {
  WFrag<FP8> w[RT];
  u32x4 x[MT][2];
};

template <int MT, int RT, bool FP8>
__device__ inline void load_step(Step<MT, RT, FP8>& st, const uint8_t* const (&wp)[RT],
                                 const uint16_t* const (&xp)[MT], int64_t k) {
  constexpr int64_t eb = FP8 ? 1 : 2;
#pragma unroll
  for (int t = 0; t < RT; ++t) load_w<FP8>(st.w[t], wp[t] + k * eb);
#pragma unroll
  for (int b = 0; b < MT; ++b) {
    const u32x4* p = reinterpret_cast<const u32x4*>(xp[b] + k);
    st.x[b][0] = p[0];
    st.x[b][1] = p[1];
  }
}

template <int MT, int RT, bool FP8>
__device__ inline void mma_step(const Step<MT, RT, FP8>& st, f32x4 (&acc)[RT][MT]) {
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    bf16x8 a0, a1;
    to_operands<FP8>(st.w[t], a0, a1);
#pragma unroll
    for (int b = 0; b < MT; ++b) {
      acc[t][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_bf16x8(st.x[b][0]), acc[t][b], 0, 0, 0);
      acc[t][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, as_bf16x8(st.x[b][1]), acc[t][b], 0, 0, 0);
    }
  }
}

// First weight row of tile t of row block bx.  A row block holds a.rb
// output rows (gate rows and as many up rows in SILU mode), which may be
// fewer than its RT tiles cover: rows past the block's end are masked.
template <int RT>
__device__ inline int64_t tile_row(const StreamArgs& a, int t, int64_t bx) {
  if (a.mode == OUT_SILU_BF16) {
    constexpr int half = RT / 2;
    const int64_t j0 = bx * a.rb;
    return t < half ? j0 + t * 16 : a.inter + j0 + (t - half) * 16;
  }
  return bx * a.rb + t * 16;
}

// End (exclusive) of the output rows of row block bx: weight rows for plain
// modes, gate indices j in SILU mode (gate row j and up row I + j).
__device__ inline int64_t block_row_end(const StreamArgs& a, int64_t bx) {
  const int64_t end = (bx + 1) * a.rb;
  const int64_t cols = a.mode == OUT_SILU_BF16 ? a.inter : a.rows;
  return end < cols ? end : cols;
}

__device__ inline void store4(const StreamArgs& a, int64_t tok, int64_t row, const float (&v)[4], bool bf16_out) {
  if (bf16_out) {
    uint16_t* y = static_cast<uint16_t*>(a.Y) + tok * a.ldy + row;
    if (row + 4 <= a.rows && ((reinterpret_cast<uintptr_t>(y) & 7) == 0)) {
      uint2 o;
      o.x = uint32_t(bf16_bits(v[0])) | (uint32_t(bf16_bits(v[1])) << 16);
      o.y = uint32_t(bf16_bits(v[2])) | (uint32_t(bf16_bits(v[3])) << 16);
      *reinterpret_cast<uint2*>(y) = o;
    } else {
      for (int i = 0; i < 4; ++i)
        if (row + i < a.rows) y[i] = bf16_bits(v[i]);
    }
  } else {
    float* y = static_cast<float*>(a.Y) + tok * a.ldy + row;
    if (row + 4 <= a.rows && ((reinterpret_cast<uintptr_t>(y) & 15) == 0)) {
      *reinterpret_cast<float4*>(y) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      for (int i = 0; i < 4; ++i)
        if (row + i < a.rows) y[i] = v[i];
    }
  }
}

// Second half of every streaming GEMM workgroup.  NPART partial fp32 sums of
// RT row tiles x MT token blocks sit in LDS token-major, red[part][token][row]
// with a row stride of 16 * RT + 4 floats: a lane's four outputs of an MFMA
// tile (rows 4 * (lane / 16) + 0..3, token lane % 16) are one 16-byte write,
// and the 16 tokens of a write land 16 bytes apart, in distinct bank groups.
template <int MT, int RT>
struct Red {
  static constexpr int RS = 16 * RT + 4;  // floats per token row
  static constexpr int bytes(int nparts) { return nparts * MT * 16 * RS * 4; }
};

template <int MT, int RT>
__device__ inline void red_put(float* red, int part, int t, int b, int lane, const f32x4& v) {
  *reinterpret_cast<f32x4*>(red + (part * MT * 16 + b * 16 + (lane & 15)) * Red<MT, RT>::RS + t * 16 +
                            4 * (lane >> 4)) = v;
}

// The output rows a thread finishes: row group rg = tid % G4 of its row block
// (G4 = 4 per output tile), the same for every token it handles.  Their
// scales are loaded here, before the cross-wave sum, so that the finish does
// not wait on them.
struct EpiRows {
  int64_t row;   // first of 4 output rows (the gate index in SILU mode)
  int64_t urow;  // first of the 4 matching up rows (SILU mode)
  int col;       // offset of `row` in the LDS token row
  bool live;     // inside the row block
  f32x4 sg, su;  // scales of the 4 rows (ones for split-K partials)
};

template <int RT>
__device__ inline int epi_groups(const StreamArgs& a) {
  return (a.mode == OUT_SILU_BF16 ? RT / 2 : RT) * 4;
}

template <int RT>
__device__ inline EpiRows epi_rows(const StreamArgs& a, int64_t bx) {
  const bool silu_mode = a.mode == OUT_SILU_BF16;
  const int rg = threadIdx.x % epi_groups<RT>(a);
  EpiRows e;
  e.row = tile_row<RT>(a, rg / 4, bx) + 4 * (rg % 4);
  e.urow = silu_mode ? tile_row<RT>(a, rg / 4 + RT / 2, bx) + 4 * (rg % 4) : 0;
  e.col = 4 * rg;
  // masked rows of a short row block belong to the next block
  e.live = e.row < block_row_end(a, bx);
  e.sg = f32x4{1.f, 1.f, 1.f, 1.f};
  e.su = e.sg;
  if (a.scale && a.ksplit == 1 && e.live) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e.sg[i] = e.row + i < a.rows ? a.scale[e.row + i] : 0.f;
      if (silu_mode) e.su[i] = a.scale[e.urow + i];
    }
  }
  return e;
}

// Adds the NPART partial sums for one token and 4 consecutive rows per item
// and applies the output mode (scale, SiLU*up, bf16 rounding) or writes a
// split-K partial.  Consecutive threads take consecutive row groups of one
// token, so the global stores of a wave cover whole runs of a token's row.
template <int MT, int RT, int NPART = kWaves, int NT = kThreads>
__device__ inline void finish_tile(const StreamArgs& a, const float* red, const EpiRows& e, int64_t tok0,
                                   int64_t split) {
  if (!e.live) return;
  const bool silu_mode = a.mode == OUT_SILU_BF16;
  constexpr int RS = Red<MT, RT>::RS;
  const int g4 = epi_groups<RT>(a);
  const int ucol = 8 * RT + e.col;  // the up rows sit RT / 2 tiles further
  auto sum_at = [&](int tl, int col) {
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NPART; ++w) v += *reinterpret_cast<const f32x4*>(red + (w * MT * 16 + tl) * RS + col);
    return v;
  };
  for (int tl = threadIdx.x / g4; tl < MT * 16; tl += NT / g4) {
    const int64_t tok = tok0 + tl;
    if (tok >= a.M) break;
    const f32x4 g = sum_at(tl, e.col);
    if (silu_mode) {
      const f32x4 u = sum_at(tl, ucol);
      if (a.ksplit > 1) {
        // SILU mode: rows = 2 I with I a multiple of 16, so these are aligned
        float* pg = a.partial + (split * a.M + tok) * a.rows;
        *reinterpret_cast<f32x4*>(pg + e.row) = g;
        *reinterpret_cast<f32x4*>(pg + e.urow) = u;
        continue;
      }
      float h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = silu(g[i] * e.sg[i]) * (u[i] * e.su[i]);
      // h is [M, ldy] with I columns; `row` is the gate index j
      StreamArgs hb = a;
      hb.rows = a.inter;
      store4(hb, tok, e.row, h, true);
      continue;
    }
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = g[i];
    if (a.ksplit > 1) {
      float* pr = a.partial + (split * a.M + tok) * a.rows + e.row;
      if (e.row + 4 <= a.rows && (reinterpret_cast<uintptr_t>(pr) & 15) == 0) {
        *reinterpret_cast<f32x4*>(pr) = g;
      } else {
        for (int i = 0; i < 4; ++i)
          if (e.row + i < a.rows) pr[i] = v[i];
      }
      continue;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] *= e.sg[i];
    store4(a, tok, e.row, v, a.mode == OUT_BF16);
  }
}

template <int MT, int RT, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void stream_gemm_kernel(StreamArgs a) {
  constexpr int64_t eb = FP8 ? 1 : 2;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int grp = lane >> 4;

  const int64_t k_begin = int64_t(blockIdx.y) * a.kper;
  const int64_t k_end = min(a.K, k_begin + a.kper);
  const int nsub = int((k_end - k_begin) / kStepK);
  const int64_t tok0 = int64_t(blockIdx.z) * 16 * MT;

  const uint8_t* wp[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    int64_t r = tile_row<RT>(a, t, blockIdx.x) + r16;
    r = min(r, a.rows - 1);  // rows past the end are loaded from the last row and never stored
    wp[t] = a.W + (r * a.K + k_begin + grp * 16) * eb;
  }
  const uint16_t* xp[MT];
#pragma unroll
  for (int b = 0; b < MT; ++b) {
    const int64_t m = min(tok0 + b * 16 + r16, a.M - 1);
    xp[b] = a.X + m * a.ldx + k_begin + grp * 16;
  }

  f32x4 acc[RT][MT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int b = 0; b < MT; ++b) acc[t][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // two steps in flight per wave
  Step<MT, RT, FP8> s0, s1;
  int s = wave;
  if (s < nsub) load_step<MT, RT, FP8>(s0, wp, xp, int64_t(s) * kStepK);
  if (s + kWaves < nsub) load_step<MT, RT, FP8>(s1, wp, xp, int64_t(s + kWaves) * kStepK);
  // output rows and their scales, loaded long before the finish needs them
  const EpiRows e = epi_rows<RT>(a, blockIdx.x);
  for (; s < nsub; s += 2 * kWaves) {
    mma_step<MT, RT, FP8>(s0, acc);
    if (s + 2 * kWaves < nsub) load_step<MT, RT, FP8>(s0, wp, xp, int64_t(s + 2 * kWaves) * kStepK);
    if (s + kWaves < nsub) {
      mma_step<MT, RT, FP8>(s1, acc);
      if (s + 3 * kWaves < nsub) load_step<MT, RT, FP8>(s1, wp, xp, int64_t(s + 3 * kWaves) * kStepK);
    }
  }

  // ---- add the 4 waves' sums in LDS
  __shared__ __attribute__((aligned(16))) float red[Red<MT, RT>::bytes(kWaves) / 4];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int b = 0; b < MT; ++b) red_put<MT, RT>(red, wave, t, b, lane, acc[t][b]);
  __syncthreads();
  finish_tile<MT, RT>(a, red, e, tok0, blockIdx.y);
}

// ---------------------------------------------------------------------------
// Staged variant (K a multiple of 256).  Same arithmetic and output modes as
// stream_gemm_kernel; the difference is how the operands reach the MFMAs:
//   * a K stage is 256 elements (512 for one FP8 token block outside the SiLU
//     mode); the workgroup's 16*RTL rows x one stage of W are loaded with
//     consecutive threads on consecutive 16-byte pieces of a row, so one wave
//     instruction reads 4 rows x 256 B (fp8) or 2 rows x 512 B (bf16) -- long
//     runs per DRAM page instead of 16 rows x 64 B;
//   * a row block may hold fewer output rows than its tiles (StreamArgs::rb):
//     rows past its end read nothing and are never stored, which lets the
//     planner make the workgroup count fill whole waves of the CUs;
//   * HBM latency under full load is microseconds, so a skinny GEMM is bound
//     by bytes in flight per CU: W pieces run D stages ahead in a register
//     ring (tens of KB per workgroup); the activations, which come from L2,
//     run DX stages ahead in a ring of their own;
//   * each stage passes through a double-buffered LDS tile whose 16-byte
//     pieces are XOR-swizzled by row (piece c of row r sits at
//     r * CPR + (c ^ (r % 16))), so the MFMA fragment reads (16 rows, one
//     piece each) hit 16 distinct bank groups; a step multiplies stage s out
//     of one buffer while it writes stage s + 1 into the other;
//   * two ways to share a stage between the waves:
//     - token split (4 waves, WK = false): wave w works on token block w % MT
//       and on MT of the stage's 4 groups of 64 K (group w / MT and on); each
//       wave reads and widens the W pieces of its K groups, so with MT token
//       blocks every W piece is widened MT times -- the mode for one token
//       block, where it is a pure K split;
//     - K split with X in LDS (WK and XL; 8 waves in two row halves for 1, 2
//       or 4 token blocks): wave w works on K group w % 4 of row half w / 4 for
//       every token block, so each W piece is read from LDS and widened once;
//       the stage's X tile (16*MT token rows x 512 B) is loaded with
//       row-contiguous 16-byte pieces, which keeps the L2 -> CU traffic of X
//       in whole cache lines, and passes through a second double-buffered LDS
//       tile (piece p of token row r at r * 32 + (p ^ (r % 16))); two waves
//       per SIMD cover each other's LDS and load latencies, and each holds
//       half the accumulators;
//     the waves of a K group add their sums in LDS at the end.
//   * loads go through buffer resources with the stage offset in the scalar
//     offset; a stage past the workgroup's last reads through a resource with
//     no records and gets zeros, so the unrolled main loop has no branches and
//     the compiler's wait counts stay exact.
// Workgroups per CU of a staged kernel: two where registers (about 196 next
// to the accumulators) and LDS allow, otherwise one -- the accumulators then
// sit in AGPRs and the rings get about 220 VGPRs.  One 16-token block over 32
// or fewer rows (the down GEMM and small views at decode) has few
// workgroups, so each keeps a deep ring instead; eight waves fill a CU.
constexpr int staged_occupancy(int MT, int RTL, bool FP8, bool WK, bool XL, int SK, int NW) {
  const int EB = FP8 ? 1 : 2;
  const int TILE = 16 * RTL * SK * EB;
  const int XT = XL ? 16 * MT * SK * 2 : 0;
  const int KQ = WK ? 4 : 4 / MT;
  const int ACC = WK ? (RTL / (NW / 4)) * MT : RTL;
  const int RED = KQ * MT * 16 * (16 * RTL + 4) * 4;
  const int LDS = (2 * TILE + 2 * XT) > RED ? (2 * TILE + 2 * XT) : RED;
  const bool DEEP = MT == 1 && RTL <= 2;
  return (NW == 8 || DEEP || ACC >= 16 || LDS > 80 * 1024) ? 1 : 2;
}

template <int MT, int RTL, bool FP8, bool WK, bool XL, int SK = kStageK, int NW = kWaves>
struct StagedShape {
  static_assert(XL == WK, "K-split waves read X from LDS; token-split waves load their own");
  static_assert(SK == kStageK || (!WK && SK == 2 * kStageK), "longer stages only with token-split waves");
  static_assert(NW == 4 || (NW == 8 && WK && XL && RTL % 2 == 0), "8 waves: K split, X in LDS, two row halves");
  static constexpr int NT = 64 * NW;                   // threads per workgroup
  static constexpr int RH = NW / 4;                    // row halves (8 waves: wave / 4 picks one)
  static constexpr int RTW = RTL / RH;                 // row tiles per wave (K-split modes)
  static constexpr int EB = FP8 ? 1 : 2;
  static constexpr int G = SK / 64;                    // 64-K groups per stage
  static constexpr int CPR = SK * EB / 16;             // 16-byte pieces per row per stage
  static constexpr int TILE = 16 * RTL * SK * EB;      // bytes of W per stage
  static constexpr int NV = TILE / (16 * NT);          // W pieces per thread per stage
  static constexpr int XT = XL ? 16 * MT * SK * 2 : 0;  // bytes of X per stage in LDS
  static constexpr int XNV = XT / (16 * NT);           // X pieces per thread per stage (XL)
  static constexpr int KQ = WK ? 4 : 4 / MT;           // waves that share a token block (K groups)
  static constexpr int QN = WK ? 1 : G * MT / 4;       // K groups per wave per stage
  static constexpr int XF = WK ? MT : QN;              // X fragment pairs per lane per stage
  static constexpr int ACC = WK ? RTW * MT : RTL;      // 16x16 accumulator tiles per wave
  static constexpr int XS = XL ? 4 * XNV : 8 * XF;     // VGPRs of one stage of X in the ring
  static constexpr int WS = 4 * NV;                     // VGPRs of one stage of W pieces
  static constexpr int RED = Red<MT, RTL>::bytes(KQ);  // bytes of the final cross-wave sum
  static constexpr int LDS = (2 * TILE + 2 * XT) > RED ? (2 * TILE + 2 * XT) : RED;
  // Register budget of the rings (VGPRs): with eight waves (two per SIMD)
  // 256 registers per wave less the accumulators and fragments.
  static constexpr bool DEEP = MT == 1 && RTL <= 2;
  static constexpr int OCC = staged_occupancy(MT, RTL, FP8, WK, XL, SK, NW);
  static constexpr int FREE = NW == 8 ? 256 - 4 * ACC - 52 - 8 * MT - 16
                                      : (OCC == 2 ? 196 - 4 * ACC : (DEEP ? 440 - 4 * ACC : 220 - (XL ? 8 * MT : 0)));
  static constexpr int WCAP = OCC == 2 || NW == 8 ? 112 : 128;
  // One 16-token block: X is cheap, so W and X of a stage share a slot (D
  // deep).  More tokens: X runs DX = 4 or 2 stages ahead in a ring of its own
  // and W gets the rest, at most WCAP VGPRs.  Eight waves keep two stages of
  // each in flight: with twice the waves per CU that is as many bytes in
  // flight as four stages of four waves, and deeper rings measured slower
  // (17-32 tokens: 54.3 against 57.6 us per shared-expert MLP at 24 tokens).
  static constexpr int DX0 = MT == 1 ? 0 : (NW == 8 ? 2 : (MT == 2 && NV < 8 ? 4 : 2));
  static constexpr int MT1CAP = DEEP ? 208 : 140;
  static constexpr int RING = MT == 1 ? (FREE < MT1CAP ? FREE : MT1CAP) / (WS + XS)
                                      : ((FREE - DX0 * XS) < WCAP ? (FREE - DX0 * XS) : WCAP) / WS;
  static constexpr int STEP = MT == 1 ? 2 : DX0;  // D must be a multiple of this (and even)
  static constexpr int DMAX = DEEP ? 20 : (NW == 8 ? 2 : 12);
  static constexpr int D1 = RING < STEP ? STEP : (RING > DMAX ? DMAX : RING);
  static constexpr int D = D1 - (D1 % STEP);
  static constexpr int DX = MT == 1 ? D : DX0;
};

// The body of a staged workgroup: row block bx, K split by, token block bz.
template <int MT, int RTL, bool FP8, bool WK, bool XL, int SK = kStageK, int NW = kWaves>
__device__ inline void staged_body(const StreamArgs& a, int64_t bx, int64_t by, int64_t bz, uint8_t* lds) {
  using S = StagedShape<MT, RTL, FP8, WK, XL, SK, NW>;
  constexpr int EB = S::EB, CPR = S::CPR, TILE = S::TILE, NV = S::NV, D = S::D, DX = S::DX, KQ = S::KQ;
  constexpr int QN = S::QN, XT = S::XT, XF = S::XF, NT = S::NT, RTW = S::RTW;
  constexpr int XNV = S::XNV;
  static_assert(D % DX == 0 && D % 2 == 0, "ring depths must nest");
  static_assert(NV >= 1 && TILE % (16 * NT) == 0, "tile must split evenly over the workgroup");
  static_assert(!XL || XNV * 16 * NT == XT, "X tile must split evenly over the workgroup");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int grp = lane >> 4;
  // token split: token block wave % MT, K groups kq*MT .. kq*MT + MT - 1;
  // K split: every token block, K group kq = wave % 4, row tiles rh*RTW ..
  // rh*RTW + RTW - 1 (rh = wave / 4: one half of the rows with 8 waves)
  const int blk = WK ? 0 : wave % MT;
  const int kq = WK ? wave % 4 : wave / MT;
  const int rh = WK ? wave / 4 : 0;

  const int64_t k_begin = by * a.kper;
  const int64_t k_end = min(a.K, k_begin + a.kper);
  const int nst = int((k_end - k_begin) / SK);
  const int64_t tok0 = bz * 16 * MT;

  // Buffer resources; a stage at or past nst is loaded through a copy with
  // num_records = 0, so every lane reads nothing and gets zeros.  The stage
  // offset goes in the scalar offset: the per-lane offsets stay constant.
  const int w_records = int(a.rows * a.K * EB);
  auto wres_at = [&](int st) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.W), 0, st < nst ? w_records : 0, 0x00020000);
  };
  // a lane offset at or past every buffer's end: that lane reads nothing
  constexpr int kOutOfRange = 0x7FFFFFF0;
  int wsrc[NV];
  int wdst[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int v = j * NT + tid;
    const int row = v / CPR;
    const int piece = v % CPR;
    const int64_t r = tile_row<RTL>(a, row / 16, bx) + (row % 16);
    // rows past the row block (or the matrix) read nothing and are never stored
    const bool up_tile = a.mode == OUT_SILU_BF16 && row / 16 >= RTL / 2;
    const int64_t j_out = up_tile ? r - a.inter : r;
    wsrc[j] = j_out < block_row_end(a, bx) ? int((r * a.K + k_begin) * EB + piece * 16) : kOutOfRange;
    wdst[j] = (row * CPR + (piece ^ (row & 15))) * 16;
  }
  // A-fragment LDS offsets for row tile 0 (tile t adds t * 16 rows): K group
  // g4 = kq*QN + q covers pieces 4*g4 .. 4*g4+3 (fp8)
  constexpr int kTileStride = 16 * CPR * 16;
  int aoff[QN][2];
#pragma unroll
  for (int q = 0; q < QN; ++q) {
    const int g4 = kq * QN + q;
    if (FP8) {
      const int piece = 4 * g4 + grp;
      aoff[q][0] = (r16 * CPR + (piece ^ r16)) * 16;
      aoff[q][1] = aoff[q][0];
    } else {
      const int p0 = 2 * (4 * g4 + grp);
      aoff[q][0] = (r16 * CPR + (p0 ^ r16)) * 16;
      aoff[q][1] = (r16 * CPR + ((p0 + 1) ^ r16)) * 16;
    }
  }
  const int x_records = int(a.M * a.ldx * 2);
  auto xres_at = [&](int st) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.X), 0, st < nst ? x_records : 0, 0x00020000);
  };
  // Register-direct X (token split): one token row, K group q at +q*64; the
  // lane's fragment is k = 16*grp .. 16*grp+15 of the group, token row r16
  // of the block.
  const int64_t m_x = min(tok0 + blk * 16 + r16, a.M - 1);
  const int xsrc = int((m_x * a.ldx + k_begin + (4 * kq * QN + grp) * 16) * 2);
  // XL: piece i of a thread is piece (i*NT + tid) % 32 of token row
  // (i*NT + tid) / 32 of the stage tile; rows past M read nothing.
  int xg[XL ? XNV : 1];
  int xdst[XL ? XNV : 1];
  int xfrag[2];  // XL: LDS offsets of the lane's two X fragments in token block 0
#pragma unroll
  for (int i = 0; i < (XL ? XNV : 1); ++i) {
    const int v = i * NT + tid;
    const int row = v / 32, piece = v % 32;
    xg[i] = tok0 + row < a.M ? int(((tok0 + row) * a.ldx + k_begin) * 2 + piece * 16) : kOutOfRange;
    xdst[i] = (row * 32 + (piece ^ (row & 15))) * 16;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int piece = 8 * kq + 2 * grp + h;
    xfrag[h] = (r16 * 32 + (piece ^ r16)) * 16;
  }

  f32x4 acc[S::ACC];
#pragma unroll
  for (int t = 0; t < S::ACC; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wr[D][NV];
  // One stage of X per ring slot: XR pieces per lane -- the lane's share of
  // the stage tile (XL), or its fragments, piece 2q+h = K group q, half h.
  constexpr int XR = XL ? XNV : 2 * XF;
  u32x4 xr[DX][XR];
  auto load_w = [&](u32x4(&r)[NV], int st) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      r[j] = __builtin_bit_cast(u32x4,
                                __builtin_amdgcn_raw_buffer_load_b128(wres_at(st), wsrc[j], st * (SK * EB), 2 /* nt */));
    }
  };
  auto load_x = [&](u32x4(&x)[XR], int st) {
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int q = i / 2, h = i % 2;
      const int off = XL ? xg[i] : xsrc + q * 64 * 2 + 16 * h;
      x[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xres_at(st), off, st * SK * 2, 0));
    }
  };
  auto store_w = [&](int buf, const u32x4(&r)[NV]) {
#pragma unroll
    for (int j = 0; j < NV; ++j) *reinterpret_cast<u32x4*>(lds + buf * TILE + wdst[j]) = r[j];
  };
  auto store_x = [&](int buf, const u32x4(&x)[XR]) {
#pragma unroll
    for (int i = 0; i < XR; ++i) *reinterpret_cast<u32x4*>(lds + 2 * TILE + buf * XT + xdst[i]) = x[i];
  };
  // The raw W fragments of row tile t, K group q (token split) or of the
  // wave's K group: one 16-byte LDS read for FP8, two for BF16.
  constexpr int FV = FP8 ? 1 : 2;
  auto w_read = [&](int buf, int t, int q, u32x4 (&v)[FV]) {
    const uint8_t* base = lds + buf * TILE + t * kTileStride;
#pragma unroll
    for (int h = 0; h < FV; ++h) v[h] = *reinterpret_cast<const u32x4*>(base + aoff[q][h]);
  };
  auto w_widen = [&](const u32x4 (&v)[FV], bf16x8& a0, bf16x8& a1) {
    if (FP8) {
      a0 = fp8x8_to_bf16(v[0][0], v[0][1]);
      a1 = fp8x8_to_bf16(v[0][2], v[0][3]);
    } else {
      a0 = as_bf16x8(v[0]);
      a1 = as_bf16x8(v[FV - 1]);
    }
  };
  // The fragment reads of all row tiles are issued before the first
  // conversion, so the LDS latency is paid once per K group rather than once
  // per row tile.
  auto compute = [&](int buf, const u32x4(&x)[XR]) {
    if (WK) {
      // each W fragment is read and widened once and used by every token
      // block; the fragments are read in groups of at most 4 row tiles
      constexpr int TG = RTW < 4 ? RTW : 4;
      u32x4 xf[MT][2];
#pragma unroll
      for (int t0 = 0; t0 < RTW; t0 += TG) {
        u32x4 wv[TG][FV];
#pragma unroll
        for (int t = 0; t < TG; ++t) w_read(buf, rh * RTW + t0 + t, 0, wv[t]);
        if (t0 == 0) {
#pragma unroll
          for (int b = 0; b < MT; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              xf[b][h] = *reinterpret_cast<const u32x4*>(lds + 2 * TILE + buf * XT + b * 16 * 512 + xfrag[h]);
        }
#pragma unroll
        for (int t = 0; t < TG; ++t) {
          bf16x8 a0, a1;
          w_widen(wv[t], a0, a1);
#pragma unroll
          for (int b = 0; b < MT; ++b) {
            f32x4& c = acc[(t0 + t) * MT + b];
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_bf16x8(xf[b][0]), c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, as_bf16x8(xf[b][1]), c, 0, 0, 0);
          }
        }
      }
    } else {
      // token split: one K group's fragments at a time (QN groups per stage)
#pragma unroll
      for (int q = 0; q < QN; ++q) {
        u32x4 wv[RTL][FV];
#pragma unroll
        for (int t = 0; t < RTL; ++t) w_read(buf, t, q, wv[t]);
#pragma unroll
        for (int t = 0; t < RTL; ++t) {
          bf16x8 a0, a1;
          w_widen(wv[t], a0, a1);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_bf16x8(x[2 * q]), acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, as_bf16x8(x[2 * q + 1]), acc[t], 0, 0, 0);
        }
      }
    }
  };

  // Stage s uses W slot s % D, X slot s % DX and LDS buffer s % 2.  The
  // prologue loads stages 0 .. D-1 and writes stage 0 to LDS.  Step s then
  // reads stage s from LDS and multiplies it while the same waves write
  // stage s + 1 into the other buffer and refill its register slot with stage
  // s + 1 + D; one barrier per step closes both.  The LDS writes, the
  // fragment reads and the MFMAs of a step thus overlap instead of running
  // one after the other in every wave.
#pragma unroll
  for (int j = 0; j < D; ++j) {
    load_w(wr[j], j);
    if (j + DX - D >= 0) load_x(xr[(j + DX - D) % DX], j + DX - D);
    __builtin_amdgcn_sched_barrier(0);
  }
  // output rows and their scales, loaded behind the first stages (loads
  // retire in order) and long before the finish needs them
  const EpiRows e = epi_rows<RTL>(a, bx);
  __builtin_amdgcn_sched_barrier(0);
  store_w(0, wr[0]);
  if (XL) store_x(0, xr[0]);
  load_w(wr[0], D);
  if (XL) load_x(xr[0], DX);
  __syncthreads();

  // The loop is unrolled D times so every register index is a compile-time
  // constant.  Full groups of D stages run without any branch (one back edge
  // keeps the wait counts exact); the last partial group runs in a tail.
  // Stages past the end were loaded as zeros and are written but never read.
  auto step = [&](const int j, const int s) {
    const int n = (j + 1) % D;  // register slot of stage s + 1
    compute(j & 1, xr[j % DX]);
    if (!XL) load_x(xr[j % DX], s + DX);
    store_w((j + 1) & 1, wr[n]);
    if (XL) store_x((j + 1) & 1, xr[n % DX]);
    load_w(wr[n], s + 1 + D);
    if (XL) load_x(xr[n % DX], s + 1 + DX);
    __syncthreads();
  };
  int s0 = 0;
  for (; s0 + D <= nst; s0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) step(j, s0 + j);
  }
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (s0 + j < nst) step(j, s0 + j);

  float* red = reinterpret_cast<float*>(lds);
  constexpr int TW = WK ? RTW : RTL;
#pragma unroll
  for (int t = 0; t < TW; ++t)
#pragma unroll
    for (int b = 0; b < (WK ? MT : 1); ++b)
      red_put<MT, RTL>(red, kq, rh * TW + t, blk + b, lane, acc[t * (WK ? MT : 1) + b]);
  __syncthreads();
  finish_tile<MT, RTL, KQ, NT>(a, red, e, tok0, by);
}

template <int MT, int RTL, bool FP8, bool WK, bool XL, int SK, int NW = kWaves>
__global__ __launch_bounds__(64 * NW, (StagedShape<MT, RTL, FP8, WK, XL, SK, NW>::OCC)) void staged_gemm_kernel(
    StreamArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[StagedShape<MT, RTL, FP8, WK, XL, SK, NW>::LDS];
  staged_body<MT, RTL, FP8, WK, XL, SK, NW>(a, blockIdx.x, blockIdx.y, blockIdx.z, lds);
}

// Several projections in one launch (the views of one reassembled layer):
// workgroup x belongs to the group g with first[g] <= x < first[g + 1] and
// runs that group's row block x - first[g].  No K split.
struct GroupArgs {
  StreamArgs g[kMaxGroup];
  int first[kMaxGroup + 1];
  int n;
};

template <int MT, int RTL, bool FP8>
__global__ __launch_bounds__(kThreads, (StagedShape<MT, RTL, FP8, false, false>::OCC)) void grouped_staged_kernel(
    GroupArgs ga) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[StagedShape<MT, RTL, FP8, false, false>::LDS];
  const int x = blockIdx.x;
  int g = 0;
  while (g + 1 < ga.n && x >= ga.first[g + 1]) ++g;
  staged_body<MT, RTL, FP8, false, false>(ga.g[g], x - ga.first[g], 0, blockIdx.z, lds);
}

// The same with eight K-split waves and X through LDS (FP8 weights).
template <int MT, int RTL>
__global__ __launch_bounds__(512, 1) void grouped_staged8_kernel(GroupArgs ga) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[StagedShape<MT, RTL, true, true, true, kStageK, 8>::LDS];
  const int x = blockIdx.x;
  int g = 0;
  while (g + 1 < ga.n && x >= ga.first[g + 1]) ++g;
  staged_body<MT, RTL, true, true, true, kStageK, 8>(ga.g[g], x - ga.first[g], 0, blockIdx.z, lds);
}

// Adds the split-K partials in split order and applies scale / SiLU / rounding.
// One thread per (token, 4 consecutive output columns); where the partial rows
// and the scales are 16-byte aligned each split is one 16-byte load.
__global__ __launch_bounds__(kThreads) void splitk_finalize_kernel(StreamArgs a) {
  const bool silu_mode = a.mode == OUT_SILU_BF16;
  const int64_t cols = silu_mode ? a.inter : a.rows;
  const int64_t groups = (cols + 3) / 4;
  const int64_t total = a.M * groups;
  const bool vec = a.rows % 4 == 0 && cols % 4 == 0 && (reinterpret_cast<uintptr_t>(a.partial) & 15) == 0 &&
                   (!a.scale || (reinterpret_cast<uintptr_t>(a.scale) & 15) == 0);
  for (int64_t q = int64_t(blockIdx.x) * kThreads + threadIdx.x; q < total; q += int64_t(gridDim.x) * kThreads) {
    const int64_t tok = q / groups;
    const int64_t c0 = (q % groups) * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    float u[4] = {0.f, 0.f, 0.f, 0.f};
    float sg[4] = {1.f, 1.f, 1.f, 1.f};
    float su[4] = {1.f, 1.f, 1.f, 1.f};
    if (vec) {
      f32x4 gv = f32x4{0.f, 0.f, 0.f, 0.f}, uv = gv;
      for (int s = 0; s < a.ksplit; ++s) {
        const float* p = a.partial + (int64_t(s) * a.M + tok) * a.rows + c0;
        gv += *reinterpret_cast<const f32x4*>(p);
        if (silu_mode) uv += *reinterpret_cast<const f32x4*>(p + a.inter);
      }
      const f32x4 one = f32x4{1.f, 1.f, 1.f, 1.f};
      const f32x4 gs = a.scale ? *reinterpret_cast<const f32x4*>(a.scale + c0) : one;
      const f32x4 us = a.scale && silu_mode ? *reinterpret_cast<const f32x4*>(a.scale + a.inter + c0) : one;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = gv[i];
        u[i] = uv[i];
        sg[i] = gs[i];
        su[i] = us[i];
      }
    } else {
      for (int s = 0; s < a.ksplit; ++s) {
        const float* p = a.partial + (int64_t(s) * a.M + tok) * a.rows;
        for (int i = 0; i < 4; ++i) {
          if (c0 + i < cols) {
            v[i] += p[c0 + i];
            if (silu_mode) u[i] += p[a.inter + c0 + i];
          }
        }
      }
      for (int i = 0; i < 4; ++i) {
        if (c0 + i >= cols || !a.scale) continue;
        sg[i] = a.scale[c0 + i];
        if (silu_mode) su[i] = a.scale[a.inter + c0 + i];
      }
    }
    if (silu_mode) {
      for (int i = 0; i < 4; ++i) v[i] = silu(v[i] * sg[i]) * (u[i] * su[i]);
      StreamArgs hb = a;
      hb.rows = a.inter;
      store4(hb, tok, c0, v, true);
    } else {
      for (int i = 0; i < 4; ++i) v[i] *= sg[i];
      store4(a, tok, c0, v, a.mode == OUT_BF16);
    }
  }
}

// Any shape and alignment; one thread per output.  Used only when K is not a
// multiple of 64 or an operand is not 16-byte aligned (odd projections).
__global__ __launch_bounds__(kThreads) void generic_gemm_kernel(StreamArgs a, int fp8) {
  const bool silu_mode = a.mode == OUT_SILU_BF16;
  const int64_t cols = silu_mode ? a.inter : a.rows;
  const int64_t total = a.M * cols;
  for (int64_t q = int64_t(blockIdx.x) * kThreads + threadIdx.x; q < total; q += int64_t(gridDim.x) * kThreads) {
    const int64_t tok = q / cols;
    const int64_t c = q % cols;
    const uint16_t* x = a.X + tok * a.ldx;
    auto dot = [&](int64_t row) {
      float acc = 0.f;
      for (int64_t k = 0; k < a.K; ++k) {
        float w;
        if (fp8) {
          const uint32_t code = a.W[row * a.K + k];
          w = static_cast<float>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(code, 1.0f, false)[0]);
        } else {
          w = __builtin_bit_cast(float, uint32_t(reinterpret_cast<const uint16_t*>(a.W)[row * a.K + k]) << 16);
        }
        const float xv = __builtin_bit_cast(float, uint32_t(x[k]) << 16);
        acc = fmaf(xv, w, acc);
      }
      return acc * (a.scale ? a.scale[row] : 1.f);
    };
    float y;
    if (silu_mode) {
      y = silu(dot(c)) * dot(a.inter + c);
    } else {
      y = dot(c);
    }
    if (a.mode == OUT_F32)
      static_cast<float*>(a.Y)[tok * a.ldy + c] = y;
    else
      static_cast<uint16_t*>(a.Y)[tok * a.ldy + c] = bf16_bits(y);
  }
}

template <int MT, int RT, bool FP8>
hipError_t launch_stream(const StreamArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((stream_gemm_kernel<MT, RT, FP8>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int RT, bool FP8>
hipError_t dispatch_mt(int mt, const StreamArgs& a, dim3 grid, hipStream_t stream) {
  switch (mt) {
    case 1:
      return launch_stream<1, RT, FP8>(a, grid, stream);
    case 2:
      return launch_stream<2, RT, FP8>(a, grid, stream);
    default:
      return launch_stream<4, RT, FP8>(a, grid, stream);
  }
}

}  // namespace

namespace {

// Output rows of a full row block of rt tiles (gate rows in SILU mode).
int64_t full_rows(const GemmProblem& p, int rt) { return p.mode == OUT_SILU_BF16 ? 8 * rt : 16 * rt; }

int64_t row_blocks_of(const GemmProblem& p, int64_t rb) {
  const int64_t cols = p.mode == OUT_SILU_BF16 ? p.rows / 2 : p.rows;
  return (cols + rb - 1) / rb;
}

// Shortens the row blocks of a staged plan so that its workgroups fill whole
// waves of the CUs: with `slots` workgroups resident at once, the count is
// rounded up to a multiple of `slots` by giving each row block fewer rows (a
// multiple of 4, at least half the tiles' rows).  A CU that would otherwise
// idle in the last wave takes a share instead; the masked rows cost LDS and
// matrix-core work but no HBM bytes.
void fill_slots(GemmPlan& plan, const GemmProblem& p, int64_t tok_blocks, int64_t slots) {
  const int64_t cols = p.mode == OUT_SILU_BF16 ? p.rows / 2 : p.rows;
  const int64_t full = full_rows(p, plan.rt);
  const int64_t per_block = tok_blocks * plan.ksplit;  // workgroups per row block
  if (per_block < 1 || slots < 1) return;              // no tokens: nothing to launch
  const int64_t wgs = row_blocks_of(p, full) * per_block;
  const int64_t waves = (wgs + slots - 1) / slots;
  const int64_t blocks = waves * slots / per_block;  // row blocks that fit in those waves
  if (blocks <= row_blocks_of(p, full)) return;
  int64_t rb = (cols + blocks - 1) / blocks;
  rb = (rb + 3) / 4 * 4;
  if (rb >= full || 2 * rb < full || row_blocks_of(p, rb) * per_block > waves * slots) return;
  plan.rb = rb;
}

// K splits of a staged plan with `wgs` workgroups over `stages` stages: the
// split doubles while fewer than 160 workgroups would run and each split
// keeps at least 4 stages (the split-K finalize costs about as much as a 1/8
// split); none past 64 tokens or without scratch for the partial sums.
int64_t staged_split(int64_t wgs, int64_t stages, int64_t M, bool may_split) {
  int64_t ks = 1;
  if (M <= 64 && may_split)
    while (wgs * ks < 160 && stages / (2 * ks) >= 4) ks *= 2;
  return ks;
}

// Fills ksplit/kper/partial_bytes for `ks` K splits of `granule`-element pieces.
void set_split(GemmPlan& plan, const GemmProblem& p, int64_t ks, int64_t granule) {
  const int64_t units = (p.K + granule - 1) / granule;
  if (ks > units) ks = units;
  if (ks < 1) ks = 1;
  const int64_t per = (units + ks - 1) / ks;
  plan.kper = per * granule;
  plan.ksplit = int((p.K + plan.kper - 1) / plan.kper);
  plan.partial_bytes = plan.ksplit > 1 ? int64_t(plan.ksplit) * p.M * p.rows * 4 : 0;
}

}  // namespace

bool plan_is_valid(const GemmProblem& p, const GemmPlan& plan) {
  const bool silu_mode = p.mode == OUT_SILU_BF16;
  const int64_t inter = silu_mode ? p.rows / 2 : 0;
  if (plan.kind == 1) return true;
  if (!(aligned(p.W, 16) && aligned(p.X, 16) && p.ldx % 8 == 0)) return false;
  if (plan.kind == 3)
    return p.K % kTileK == 0 && (plan.rt == 256 || plan.rt == 128) && plan.ksplit == 1 &&
           p.rows * p.K * (p.dtype == SWR_FP8_E4M3FN ? 1 : 2) < (INT64_C(1) << 31) && p.ldx < (INT64_C(1) << 22);
  // row blocks: whole tiles (the streaming kind), or a multiple of 4 rows
  // up to the tiles' rows (staged kinds)
  const int64_t full = full_rows(p, plan.rt);
  if (plan.kind == 0 ? plan.rb != full : (plan.rb < 4 || plan.rb % 4 != 0 || plan.rb > full)) return false;
  if (plan.kind == 6) {
    // staged with eight K-split waves in two row halves and X through LDS:
    // 1, 2 or 4 token blocks; 64-row blocks, 128 for FP8
    if (plan.mt != 1 && plan.mt != 2 && plan.mt != 4) return false;
    if (!(plan.rt == 4 || (plan.rt == 8 && p.dtype == SWR_FP8_E4M3FN))) return false;
    if (silu_mode && inter % (8 * plan.rt) != 0) return false;
    return plan.sk == kStageK && p.K % kStageK == 0 && plan.kper % kStageK == 0 &&
           p.rows * p.K * (p.dtype == SWR_FP8_E4M3FN ? 1 : 2) < (INT64_C(1) << 31) &&
           p.M * p.ldx * 2 < (INT64_C(1) << 31);
  }
  if (plan.mt != 1 && plan.mt != 2 && plan.mt != 4) return false;
  if (plan.rt != 1 && plan.rt != 2 && plan.rt != 4 && !(plan.kind == 2 && plan.rt == 8)) return false;
  if (plan.rt == 8 && (plan.mt == 1 || p.dtype != SWR_FP8_E4M3FN)) return false;
  if (silu_mode && (plan.rt < 2 || inter % (8 * plan.rt) != 0)) return false;
  if (plan.kind == 0) return p.K % kStepK == 0 && plan.rt == 4 && plan.kper % 256 == 0;
  if (plan.kind == 2) {
    if (plan.sk != kStageK &&
        !(plan.sk == 2 * kStageK && plan.mt == 1 && p.dtype == SWR_FP8_E4M3FN && plan.rt <= 4))
      return false;
    return p.K % plan.sk == 0 && plan.kper % plan.sk == 0 &&
           p.rows * p.K * (p.dtype == SWR_FP8_E4M3FN ? 1 : 2) < (INT64_C(1) << 31) &&
           p.M * p.ldx * 2 < (INT64_C(1) << 31);
  }
  return false;
}

GemmPlan plan_gemm(const GemmProblem& p, bool may_split) {
  GemmPlan plan{};
  const bool silu_mode = p.mode == OUT_SILU_BF16;
  const int64_t inter = silu_mode ? p.rows / 2 : 0;
  const bool aligned_ok = aligned(p.W, 16) && aligned(p.X, 16) && p.ldx % 8 == 0;
  plan.mt = p.M <= 16 ? 1 : (p.M <= 32 ? 2 : 4);
  const int64_t tok_blocks = (p.M + 16 * plan.mt - 1) / (16 * plan.mt);
  const int64_t w_bytes = p.rows * p.K * (p.dtype == SWR_FP8_E4M3FN ? 1 : 2);
  if (aligned_ok && p.M > 64 && p.K % kTileK == 0 && w_bytes < (INT64_C(1) << 31) && p.ldx < (INT64_C(1) << 22)) {
    // Prefill-sized M: the tiled MFMA kernel.  256-row weight tiles when they
    // still give at least two waves of workgroups over the 256 CUs.  Its
    // buffer offsets are 32-bit: weights under 2 GiB (larger ones stream),
    // and the launch splits the tokens so that each part's X is under 2 GiB.
    plan.kind = 3;
    const int64_t tiles_m = (p.M + 255) / 256;
    const int64_t cols = silu_mode ? inter : p.rows;
    const int64_t t256 = tiles_m * ((cols + (silu_mode ? 127 : 255)) / (silu_mode ? 128 : 256));
    plan.rt = t256 >= 512 ? 256 : 128;
    plan.mt = 16;
    plan.ksplit = 1;
    plan.kper = p.K;
    plan.partial_bytes = 0;
    return plan;
  }
  if (aligned_ok && p.K % kStageK == 0 && (!silu_mode || inter % 16 == 0) && w_bytes < (INT64_C(1) << 31) &&
      p.M * p.ldx * 2 < (INT64_C(1) << 31)) {
    // Staged kernel.  Row block and K split from a sweep of the shared-expert
    // shapes on MI355X: 32-row blocks when one 16-token block suffices, 64-row
    // blocks otherwise (fewer activation re-reads per weight byte); K is split
    // only while fewer than 160 workgroups would run and each split keeps at
    // least 4 stages (the split-K finalize costs about as much as a 1/8 split).
    plan.kind = 2;
    const bool fp8 = p.dtype == SWR_FP8_E4M3FN;
    if (silu_mode)
      // 128-row blocks (64 gate + 64 up rows) pay off once X is reused by
      // 32+ tokens: the X tile is then read from L2 half as often.
      plan.rt = (plan.mt > 1 && fp8 && inter % 64 == 0) ? 8 : (inter % 32 == 0 ? 4 : 2);
    else
      plan.rt = plan.mt == 1 ? 2 : 4;
    // One FP8 token block over more than two waves of 32-row blocks: the deep
    // 32-row variant holds a CU alone, so every later wave of workgroups waits
    // for its first loads; 64-row blocks run two per CU and cover them
    // (24576 x 7168 at 16 tokens: 35.6 against 43.2 us; no change up to 8192 rows)
    if (!silu_mode && plan.mt == 1 && fp8 && row_blocks_of(p, full_rows(p, 2)) * tok_blocks > 512) plan.rt = 4;
    // 17-64 tokens of FP8 weights: eight K-split waves in two row halves
    // with X through LDS (each weight byte widened once, X read in whole
    // cache lines, two waves per SIMD to cover each other's waits); 128-row
    // blocks.  Measured on the shared-expert shapes against four waves:
    // gate_up 41.9 vs 55.8 us and down 35.4 vs 41.2 us at 64 tokens.
    if (plan.mt >= 2 && fp8 && (!silu_mode || inter % 32 == 0)) {
      plan.kind = 6;
      plan.rt = (!silu_mode || inter % 64 == 0) ? 8 : 4;
    }
    // One FP8 token block: the eight-wave kernel reads each stage's
    // activations once, in whole cache lines, for 128 (gate_up) or 64 rows.
    // From 9 tokens, where those are about as many bytes as the weights of a
    // 32-row block, it wins wherever its blocks, K split as below, give 160
    // workgroups (shared-expert MLP: 50.2 against 57.0 us at 16 tokens, 48.8
    // against 52.6 at 12).  Below 9 tokens only without a K split: the split
    // and its finalize then cost more than they save (7168 x 8192: 15.6
    // against 13.4-14.2 us), while gate_up and the largest projections gain
    // (24576 x 7168 at 8 tokens: 30.2 against 33.4 us).
    if (plan.mt == 1 && fp8 && (!silu_mode || inter % 64 == 0)) {
      const int64_t blocks = row_blocks_of(p, 64);
      if (blocks * (p.M >= 9 ? staged_split(blocks, p.K / kStageK, p.M, may_split) : 1) >= 160) {
        plan.kind = 6;
        plan.rt = silu_mode ? 8 : 4;
      }
    }
    // One FP8 token block outside the SiLU mode (the down GEMM, projections):
    // 512-K stages halve the per-stage fixed cost (LDS round trip, barrier,
    // widening latency); measured 7% faster on the 14336-long down rows, 3%
    // slower on gate_up.
    plan.sk = (plan.kind == 2 && plan.mt == 1 && fp8 && !silu_mode && p.K % (2 * kStageK) == 0) ? 2 * kStageK
                                                                                                 : kStageK;
    plan.rb = full_rows(p, plan.rt);
    const int64_t wgs = row_blocks_of(p, plan.rb) * tok_blocks;
    const int64_t stages = p.K / plan.sk;
    set_split(plan, p, staged_split(wgs, stages, p.M, may_split), plan.sk);
    // every CU busy to the end: 256 CUs times the kernel's workgroups per CU
    const int occ = plan.kind == 6 ? staged_occupancy(plan.mt, plan.rt, fp8, true, true, plan.sk, 8)
                                   : staged_occupancy(plan.mt, plan.rt, fp8, false, false, plan.sk, kWaves);
    fill_slots(plan, p, tok_blocks, 256 * int64_t(occ));
  } else if (aligned_ok && p.K % kStepK == 0 && (!silu_mode || inter % 32 == 0)) {
    plan.kind = 0;
    plan.rt = 4;
    plan.rb = full_rows(p, 4);
    int64_t ks = 1;
    if (p.M <= 64 && may_split) ks = (512 + row_blocks_of(p, plan.rb) - 1) / row_blocks_of(p, plan.rb);
    set_split(plan, p, ks, 256);
  } else {
    plan.kind = 1;
    plan.ksplit = 1;
    plan.kper = p.K;
    return plan;
  }
  return plan;
}

namespace {

template <int MT, int RTL, bool FP8, bool WK, bool XL, int SK = kStageK, int NW = kWaves>
hipError_t launch_staged(const StreamArgs& a, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((staged_gemm_kernel<MT, RTL, FP8, WK, XL, SK, NW>), grid, dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

// Eight-wave K-split kernels with X through LDS: 1, 2 or 4 token blocks, 64
// rows, or 128 rows of FP8 weights.
template <bool FP8>
hipError_t dispatch_staged8(int mt, int rt, const StreamArgs& a, dim3 grid, hipStream_t stream) {
  if (mt == 1) {
    if (rt == 4) return launch_staged<1, 4, FP8, true, true, kStageK, 8>(a, grid, stream);
    if constexpr (FP8)
      if (rt == 8) return launch_staged<1, 8, FP8, true, true, kStageK, 8>(a, grid, stream);
  } else if (mt == 2) {
    if (rt == 4) return launch_staged<2, 4, FP8, true, true, kStageK, 8>(a, grid, stream);
    if constexpr (FP8)
      if (rt == 8) return launch_staged<2, 8, FP8, true, true, kStageK, 8>(a, grid, stream);
  } else if (mt == 4) {
    if (rt == 4) return launch_staged<4, 4, FP8, true, true, kStageK, 8>(a, grid, stream);
    if constexpr (FP8)
      if (rt == 8) return launch_staged<4, 8, FP8, true, true, kStageK, 8>(a, grid, stream);
  }
  return hipErrorInvalidValue;
}

// Instantiated (tile shape x sharing mode x stage length) combinations;
// plan_is_valid admits exactly these.
template <int MT, bool FP8, bool WK, bool XL>
hipError_t dispatch_staged_rt(int rt, int sk, const StreamArgs& a, dim3 grid, hipStream_t stream) {
  if (sk == 2 * kStageK) {
    // 512-K stages: one token block of FP8 weights, token-split waves
    if constexpr (MT == 1 && FP8 && !WK && !XL) {
      switch (rt) {
        case 1:
          return launch_staged<1, 1, true, false, false, 2 * kStageK>(a, grid, stream);
        case 2:
          return launch_staged<1, 2, true, false, false, 2 * kStageK>(a, grid, stream);
        case 4:
          return launch_staged<1, 4, true, false, false, 2 * kStageK>(a, grid, stream);
        default:
          return hipErrorInvalidValue;
      }
    }
    return hipErrorInvalidValue;
  }
  switch (rt) {
    case 1:
      if constexpr (!WK) return launch_staged<MT, 1, FP8, WK, XL>(a, grid, stream);
      return hipErrorInvalidValue;
    case 2:
      if constexpr (!WK) return launch_staged<MT, 2, FP8, WK, XL>(a, grid, stream);
      return hipErrorInvalidValue;
    case 8:
      if constexpr (FP8 && MT > 1) return launch_staged<MT, 8, FP8, WK, XL>(a, grid, stream);
      return hipErrorInvalidValue;
    default:
      return launch_staged<MT, 4, FP8, WK, XL>(a, grid, stream);
  }
}

template <bool FP8, bool WK, bool XL>
hipError_t dispatch_staged(int mt, int rt, int sk, const StreamArgs& a, dim3 grid, hipStream_t stream) {
  switch (mt) {
    case 1:
      if constexpr (!WK) return dispatch_staged_rt<1, FP8, WK, XL>(rt, sk, a, grid, stream);
      return hipErrorInvalidValue;
    case 2:
      return dispatch_staged_rt<2, FP8, WK, XL>(rt, sk, a, grid, stream);
    default:
      return dispatch_staged_rt<4, FP8, WK, XL>(rt, sk, a, grid, stream);
  }
}

}  // namespace

namespace {

StreamArgs make_args(const GemmProblem& p, int64_t kper, int ksplit, float* partial, int64_t rb) {
  StreamArgs a{};
  a.W = static_cast<const uint8_t*>(p.W);
  a.scale = p.scale;
  a.X = static_cast<const uint16_t*>(p.X);
  a.ldx = p.ldx;
  a.M = p.M;
  a.rows = p.rows;
  a.K = p.K;
  a.kper = kper;
  a.inter = p.mode == OUT_SILU_BF16 ? p.rows / 2 : 0;
  a.rb = rb;
  a.Y = p.Y;
  a.ldy = p.ldy;
  a.partial = partial;
  a.mode = p.mode;
  a.ksplit = ksplit;
  return a;
}

template <int MT, int RT, bool FP8>
hipError_t launch_grouped_mt(const GroupArgs& ga, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((grouped_staged_kernel<MT, RT, FP8>), grid, dim3(kThreads), 0, stream, ga);
  return hipGetLastError();
}

}  // namespace

bool grouped_plan(const GemmProblem* ps, int n, int* mt, int* rt) {
  if (n < 1 || n > kMaxGroup) return false;
  const int64_t M = ps[0].M;
  if (M < 1) return false;
  if (M > 64) {
    // prefill-sized: every projection takes the tiled kernel, X in one token
    // part; 256-row tiles when the group gives two waves of them (as plan_gemm)
    int64_t t256 = 0;
    for (int i = 0; i < n; ++i) {
      const GemmProblem& p = ps[i];
      const int64_t eb = p.dtype == SWR_FP8_E4M3FN ? 1 : 2;
      if (p.dtype != ps[0].dtype || p.M != M || p.mode == OUT_SILU_BF16) return false;
      if (!(aligned(p.W, 16) && aligned(p.X, 16) && p.ldx % 8 == 0) || p.K % kTileK != 0) return false;
      if (p.rows * p.K * eb >= (INT64_C(1) << 31) || p.ldx >= (INT64_C(1) << 22) ||
          M * p.ldx * 2 >= (INT64_C(1) << 31))
        return false;
      t256 += ((M + 255) / 256) * ((p.rows + 255) / 256);
    }
    *mt = 16;
    *rt = t256 >= 512 ? 256 : 128;
    return true;
  }
  int64_t blocks = 0;
  *mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  // 64-row blocks (launch_grouped takes 128 for the eight-wave kernel): a
  // group runs several waves of workgroups, and at two per CU one
  // workgroup's loop covers the next one's first loads (the deep 32-row
  // variant holds a CU alone); measured on the 8-projection attention layer
  // at 16 tokens with four waves: 74 against 86 us
  *rt = 4;
  for (int i = 0; i < n; ++i) {
    const GemmProblem& p = ps[i];
    if (p.dtype != ps[0].dtype || p.M != M || p.mode == OUT_SILU_BF16) return false;
    if (!(aligned(p.W, 16) && aligned(p.X, 16) && p.ldx % 8 == 0)) return false;
    if (p.K % kStageK != 0 || p.rows * p.K * (p.dtype == SWR_FP8_E4M3FN ? 1 : 2) >= (INT64_C(1) << 31) ||
        p.M * p.ldx * 2 >= (INT64_C(1) << 31))
      return false;
    blocks += (p.rows + 16 * *rt - 1) / (16 * *rt);
  }
  return blocks < (INT64_C(1) << 29);  // (launch_grouped may double it)
}

hipError_t launch_grouped(const GemmProblem* ps, int n, int mt, int rt, hipStream_t stream) {
  // longest K first: the last workgroups to start are the shortest
  int order[kMaxGroup];
  for (int i = 0; i < n; ++i) order[i] = i;
  for (int i = 1; i < n; ++i)
    for (int j = i; j > 0 && ps[order[j]].K > ps[order[j - 1]].K; --j) {
      const int t = order[j];
      order[j] = order[j - 1];
      order[j - 1] = t;
    }
  if (ps[0].M > 64) {
    StreamArgs as[kMaxGroup];
    for (int i = 0; i < n; ++i) as[i] = make_args(ps[order[i]], ps[order[i]].K, 1, nullptr, 0);
    return launch_tile_group(as, n, rt, ps[0].dtype == SWR_FP8_E4M3FN, stream);
  }
  // Row blocks of one length rb for the whole group, as in fill_slots: the
  // shortest multiple of 4 (at least half the tiles' rows) whose block count
  // still fits the waves of workgroups that full blocks need, so that the
  // last wave is as full as the others.
  const int64_t tok_blocks = (ps[0].M + 16 * mt - 1) / (16 * mt);
  const bool fp8 = ps[0].dtype == SWR_FP8_E4M3FN;
  // FP8: eight K-split waves with X through LDS in 128-row blocks, one
  // workgroup per CU -- at 13-64 tokens, and below where the group has 160
  // such blocks.  Measured on the 8-projection attention layer (385 MB, 444
  // blocks): 62.6 against 70.7 us at 16 tokens, 73.1 against 94.2 at 32 and
  // 95.0 against 139.9 at 64 (64-row blocks: 65.7, 82.4, 117.2 us); 61.0-61.5
  // against 62.3-62.5 at 1 token, 62.1-62.2 against 66.3-66.7 at 12.
  int64_t blocks128 = 0;
  for (int i = 0; i < n; ++i) blocks128 += (ps[i].rows + 127) / 128;
  const bool eight = fp8 && (mt >= 2 || ps[0].M >= 13 || blocks128 >= 160);
  if (eight) rt = 8;
  const int64_t slots =
      eight ? 256 : 256 * int64_t(staged_occupancy(mt, rt, fp8, false, false, kStageK, kWaves));
  auto blocks_for = [&](int64_t rb) {
    int64_t b = 0;
    for (int i = 0; i < n; ++i) b += (ps[i].rows + rb - 1) / rb;
    return b * tok_blocks;
  };
  const int64_t full = 16 * int64_t(rt);
  const int64_t target = (blocks_for(full) + slots - 1) / slots * slots;
  int64_t rb = full;
  for (int64_t r = full - 4; r >= full / 2 && blocks_for(r) <= target; r -= 4) rb = r;
  GroupArgs ga{};
  ga.n = n;
  int first = 0;
  for (int i = 0; i < n; ++i) {
    const GemmProblem& p = ps[order[i]];
    ga.g[i] = make_args(p, p.K, 1, nullptr, rb);
    ga.first[i] = first;
    first += int((p.rows + rb - 1) / rb);
  }
  ga.first[n] = first;
  const dim3 grid = dim3(unsigned(first), 1, unsigned(tok_blocks));
  if (eight) {
    if (mt == 1)
      hipLaunchKernelGGL((grouped_staged8_kernel<1, 8>), grid, dim3(512), 0, stream, ga);
    else if (mt == 2)
      hipLaunchKernelGGL((grouped_staged8_kernel<2, 8>), grid, dim3(512), 0, stream, ga);
    else
      hipLaunchKernelGGL((grouped_staged8_kernel<4, 8>), grid, dim3(512), 0, stream, ga);
    return hipGetLastError();
  }
  if (mt == 1 && rt == 4)
    return fp8 ? launch_grouped_mt<1, 4, true>(ga, grid, stream) : launch_grouped_mt<1, 4, false>(ga, grid, stream);
  if (mt == 1)
    return fp8 ? launch_grouped_mt<1, 2, true>(ga, grid, stream) : launch_grouped_mt<1, 2, false>(ga, grid, stream);
  if (mt == 2)
    return fp8 ? launch_grouped_mt<2, 4, true>(ga, grid, stream) : launch_grouped_mt<2, 4, false>(ga, grid, stream);
  return fp8 ? launch_grouped_mt<4, 4, true>(ga, grid, stream) : launch_grouped_mt<4, 4, false>(ga, grid, stream);
}

hipError_t launch_tile_fp8act(const GemmProblem& p, const float* xscale, hipStream_t stream) {
  if (p.M == 0) return hipSuccess;
  const bool silu_mode = p.mode == OUT_SILU_BF16;
  const int64_t cols = silu_mode ? p.rows / 2 : p.rows;
  const int64_t tiles_m = (p.M + 255) / 256;
  // 256-row weight tiles when they still give two waves of workgroups (as plan_gemm)
  const int64_t t256 = tiles_m * ((cols + (silu_mode ? 127 : 255)) / (silu_mode ? 128 : 256));
  StreamArgs a = make_args(p, p.K, 1, nullptr, 0);
  a.xscale = xscale;
  return launch_tile_gemm(a, t256 >= 512 ? 256 : 128, true, stream);
}

hipError_t launch_gemm(const GemmProblem& p, const GemmPlan& plan, float* partial, hipStream_t stream) {
  StreamArgs a = make_args(p, plan.kper, plan.ksplit, partial, plan.rb);
  const bool fp8 = p.dtype == SWR_FP8_E4M3FN;
  if (plan.kind == 1) {
    const int64_t cols = p.mode == OUT_SILU_BF16 ? a.inter : p.rows;
    int64_t g = (p.M * cols + kThreads - 1) / kThreads;
    if (g > 65536) g = 65536;
    hipLaunchKernelGGL(generic_gemm_kernel, dim3(unsigned(g)), dim3(kThreads), 0, stream, a, fp8 ? 1 : 0);
    return hipGetLastError();
  }
  if (plan.kind == 3) return launch_tile_gemm(a, plan.rt, fp8, stream);
  const int64_t row_blocks = row_blocks_of(p, plan.rb);
  const int64_t tok_blocks = (p.M + 16 * plan.mt - 1) / (16 * plan.mt);
  const dim3 grid = dim3(unsigned(row_blocks), unsigned(plan.ksplit), unsigned(tok_blocks));
  hipError_t e;
  if (plan.kind == 2)
    e = fp8 ? dispatch_staged<true, false, false>(plan.mt, plan.rt, plan.sk, a, grid, stream)
            : dispatch_staged<false, false, false>(plan.mt, plan.rt, plan.sk, a, grid, stream);
  else if (plan.kind == 6)
    e = fp8 ? dispatch_staged8<true>(plan.mt, plan.rt, a, grid, stream)
            : dispatch_staged8<false>(plan.mt, plan.rt, a, grid, stream);
  else
    e = fp8 ? dispatch_mt<4, true>(plan.mt, a, grid, stream) : dispatch_mt<4, false>(plan.mt, a, grid, stream);
  if (e != hipSuccess || plan.ksplit == 1) return e;
  const int64_t cols = p.mode == OUT_SILU_BF16 ? a.inter : p.rows;
  int64_t g = (p.M * ((cols + 3) / 4) + kThreads - 1) / kThreads;
  if (g > 65536) g = 65536;
  hipLaunchKernelGGL(splitk_finalize_kernel, dim3(unsigned(g)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace swr
