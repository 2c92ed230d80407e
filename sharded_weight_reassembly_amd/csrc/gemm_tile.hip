// Tiled MFMA GEMM for prefill-sized token counts on gfx950.
//
//   Y[m, o] = s[o] * sum_k X[m, k] * W[o, k]      (or the fused SiLU*up mode)
//
// At thousands of tokens the weights are reused by every token block, so this
// is a classic LDS-tiled GEMM (measured on MI355X, it is bound by its loads
// into LDS more than by the matrix cores):
//   * a workgroup computes a BM-token x BN-row tile of Y (BM = 256, or 128
//     for FP8 weights where 256 x 256 tiles would not fill two waves of
//     workgroups -- then only for the weight rows past whole waves of
//     256 x 256 tiles) with 2 x WAVES/2 waves; each wave a BM/2 x
//     (2*BN/WAVES) sub-tile with
//     v_mfma_f32_32x32x16_bf16 (tokens are the MFMA rows, weight rows the
//     MFMA columns, so a lane's outputs run along a row of Y);
//   * both operands go from memory straight into an LDS ring with
//     buffer-to-LDS loads (no staging registers), several steps ahead of the
//     MFMAs; 16-byte pieces are XOR-swizzled by row, so the 32-row fragment
//     reads of one MFMA hit distinct banks.  The weight loads carry no
//     streaming hint: a weight tile is read by every token block of its XCD
//     group (measured on MI355X: 1-3.5% faster per GEMM than with the hint);
//   * FP8 weights (tile_gemm_fp8_kernel): steps of 64 K, a three-stage ring
//     two steps ahead; X rows of 128 B with piece p of row r at
//     r * 8 + (p ^ ((r >> 1) & 7)), and the raw FP8 codes, widened to BF16
//     (exact) after the fragment read;
//   * BF16 weights (tile_gemm_bf16d_kernel) and FP8 weights with FP8
//     activations (tile_gemm_f8f8d_kernel): double steps of 128 bytes per row
//     for both operands (64 K of BF16, 128 K of FP8: whole cache lines per
//     load), two or three double stages;
//   * the BF16-activation bodies write their slice pipeline out instruction
//     by instruction: each MFMA is followed by its share of the next slice's
//     fragment reads, so a wave keeps its matrix core fed while its LDS reads
//     are in flight (with one workgroup of eight waves per CU, loads into LDS
//     and fragment reads overlap only this way);
//   * the outputs of a wave are staged through the (then idle) LDS ring and
//     leave in 16-byte stores of whole 128-byte row segments;
//   * tiles are numbered so that each XCD (workgroups are dealt round-robin
//     to the 8 XCDs) works through a compact group of 8 token blocks x all
//     weight blocks, which keeps the X and W tiles of concurrently running
//     workgroups in that XCD's L2 (measured on MI355X: groups of 8 are 1-5%
//     faster per prefill GEMM than groups of 4, 16 no faster, 2 slower);
//   * in SiLU mode a workgroup owns gate rows J0..J0+BN/2 and the matching up
//     rows, laid out so that gate j and up j land in the same lane of
//     different MFMA tiles; the epilogue writes h = bf16(silu(g) * u).
#include <type_traits>

#include "gemm_common.h"

namespace swr {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kTileM = 256;
constexpr int kGroupM = 8;  // token blocks per XCD group

// SiLU for the tile epilogues: z * (1 / (1 + e^-z)) with the hardware
// reciprocal (1 ulp) rather than an IEEE division, a few fp32 ulps from the
// exact value and far inside the BF16 rounding of the output (measured on
// MI355X: the division was about 2% of the FP8-activation prefill MLP).
// Saturates correctly: e^-z = inf gives -0, e^-z = 0 gives z.
__device__ inline float silu_tile(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

__device__ inline int swz(int row, int piece) { return row * 8 + (piece ^ ((row >> 1) & 7)); }

// Output tile of this workgroup: XCD-contiguous ranges, grouped by token blocks.
struct TileCoord {
  int64_t m0;      // first token
  int64_t tile_n;  // weight-row block
};

template <int BN, int BM = kTileM>
__device__ inline TileCoord tile_coord(const StreamArgs& a, int64_t i, int64_t ntiles) {
  const bool silu_mode = a.mode == OUT_SILU_BF16;
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t cols = silu_mode ? a.inter : a.rows;  // output columns
  const int64_t col_tile = silu_mode ? BN / 2 : BN;
  const int64_t tiles_n = (cols + col_tile - 1) / col_tile;
  const int64_t t = (ntiles % 8 == 0) ? (i % 8) * (ntiles / 8) + i / 8 : i;
  const int64_t group = t / (kGroupM * tiles_n);
  const int64_t first_m = group * kGroupM;
  const int64_t gsize = min<int64_t>(tiles_m - first_m, kGroupM);
  TileCoord c;
  c.m0 = (first_m + (t % (kGroupM * tiles_n)) % gsize) * BM;
  c.tile_n = (t % (kGroupM * tiles_n)) / gsize;
  return c;
}

// Weight row held by local B row c (0 <= c < BN) of weight block tile_n; WN
// rows per wave column (SiLU mode: its first half gate rows, second half the
// matching up rows).
template <int BN, int WN>
__device__ inline int64_t w_row(const StreamArgs& a, int64_t tile_n, int c) {
  if (a.mode == OUT_SILU_BF16) {
    const int half = c / WN;
    const int c2 = c % WN;
    const int64_t j = tile_n * (BN / 2) + half * (WN / 2) + (c2 % (WN / 2));
    return c2 < WN / 2 ? j : a.inter + j;
  }
  return tile_n * BN + c;
}

// Epilogue: lane holds column c = l % 32 of each 32 x 32 tile, rows
// 8*(v/4) + 4*(l/32) + v%4; scale, SiLU*up, rounding.
template <int BN, int WN, int TM, int TN>
__device__ inline void tile_epilogue(const StreamArgs& a, const f32x16 (&acc)[TM][TN], int64_t m0, int64_t tile_n,
                                     int wm, int wn, int r32, int kg, const float* lds_scale = nullptr,
                                     const float* lds_tscale = nullptr) {
  const bool silu_mode = a.mode == OUT_SILU_BF16;
  const int tn_out = silu_mode ? TN / 2 : TN;
#pragma unroll
  for (int y = 0; y < tn_out; ++y) {
    const int c = wn * WN + y * 32 + r32;                // local B row
    const int64_t ocol = w_row<BN, WN>(a, tile_n, c);  // output column (gate index j in SiLU mode)
    if (ocol >= (silu_mode ? a.inter : a.rows)) continue;
    float sc = 1.f, su = 1.f;
    if (lds_scale) {
      // scales of local rows c and (SiLU mode) its up row c + WN / 2
      sc = lds_scale[c];
      if (silu_mode) su = lds_scale[c + WN / 2];
    } else if (a.scale) {
      sc = a.scale[ocol];
      if (silu_mode) su = a.scale[a.inter + ocol];
    }
#pragma unroll
    for (int x = 0; x < TM; ++x) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ml = wm * (TM * 32) + x * 32 + 8 * (v / 4) + 4 * kg + (v % 4);
        const int64_t m = m0 + ml;
        if (m >= a.M) continue;
        const float ts = lds_tscale ? lds_tscale[ml] : 1.f;  // token scale (FP8 activations)
        float out = acc[x][y][v] * ts * sc;
        if (silu_mode) {
          const float u = acc[x][y + TN / 2][v] * ts * su;
          out = silu_tile(out) * u;
          static_cast<uint16_t*>(a.Y)[m * a.ldy + ocol] = bf16_bits(out);
        } else if (a.mode == OUT_F32) {
          static_cast<float*>(a.Y)[m * a.ldy + ocol] = out;
        } else {
          static_cast<uint16_t*>(a.Y)[m * a.ldy + ocol] = bf16_bits(out);
        }
      }
    }
  }
}

// The wave's block of the output, staged through LDS so that it leaves in
// 16-byte stores of whole 128-byte row segments (rather than one 2-byte store
// per lane per output): a lane first writes its scaled, rounded outputs into
// the wave's region (row-major, 16-byte pieces of a row XOR-swizzled by the
// row), then reads back 16-byte pieces of rows and stores them.  BF16 outputs
// (plain or SiLU * up); the caller checks that every output row starts
// 16-byte aligned.  The region holds TM * 32 rows of TN * 32 columns.
template <int BN, int WN, int TM, int TN, bool SILU>
__device__ inline void tile_epilogue_lds_m(const StreamArgs& a, const f32x16 (&acc)[TM][TN], int64_t m0,
                                           int64_t tile_n, int wm, int wn, int r32, int kg, int lane, uint8_t* region,
                                           const float* lds_scale, const float* lds_tscale) {
  constexpr bool silu_mode = SILU;
  constexpr int ROWS = TM * 32;
  // output columns of the block: TN * 32, or TN * 16 in SiLU mode; 16-byte pieces per row
  constexpr int cols = silu_mode ? TN * 16 : TN * 32;
  constexpr int cpr = cols / 8;
  const int64_t limit = silu_mode ? a.inter : a.rows;
  const int64_t col0 = silu_mode ? tile_n * (BN / 2) + wn * (WN / 2) : tile_n * BN + wn * WN;
  constexpr int tn_out = silu_mode ? TN / 2 : TN;
  auto pos = [&](int row, int col) { return row * cols * 2 + (((col >> 3) ^ (row & (cpr - 1))) << 4) + (col & 7) * 2; };
#pragma unroll
  for (int y = 0; y < TN; ++y) {
    if (y >= tn_out) break;
    const int c = wn * WN + y * 32 + r32;  // local B row
    const float sc = lds_scale[c];
    const float su = silu_mode ? lds_scale[c + WN / 2] : 1.f;
#pragma unroll
    for (int x = 0; x < TM; ++x) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = x * 32 + 8 * (v / 4) + 4 * kg + (v % 4);
        const float ts = lds_tscale ? lds_tscale[wm * ROWS + row] : 1.f;
        float out = acc[x][y][v] * ts * sc;
        if constexpr (silu_mode) out = silu_tile(out) * (acc[x][y + TN / 2][v] * ts * su);
        *reinterpret_cast<uint16_t*>(region + pos(row, y * 32 + r32)) = bf16_bits(out);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_wave_barrier();
  uint16_t* Y = static_cast<uint16_t*>(a.Y);
  constexpr int pieces = ROWS * cpr;
  static_assert(pieces % 64 == 0, "whole passes of the wave over the block's pieces");
#pragma unroll
  for (int q0 = 0; q0 < pieces; q0 += 64) {
    const int q = q0 + lane;
    const int row = q / cpr, cp = q % cpr;
    const int64_t m = m0 + wm * ROWS + row;
    const int64_t col = col0 + cp * 8;
    if (m >= a.M || col >= limit) continue;
    const u32x4 v = *reinterpret_cast<const u32x4*>(region + row * cols * 2 + ((cp ^ (row & (cpr - 1))) << 4));
    if (col + 8 <= limit) {
      *reinterpret_cast<u32x4*>(Y + m * a.ldy + col) = v;
    } else {
      const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
      for (int e = 0; e < 8 && col + e < limit; ++e) Y[m * a.ldy + col + e] = h[e];
    }
  }
}

// The LDS epilogue with the output mode (SiLU * up, or plain BF16) fixed at
// compile time, so that neither mode computes the other's outputs and the
// swizzled LDS offsets fold into immediates.
template <int BN, int WN, int TM, int TN>
__device__ inline void tile_epilogue_lds(const StreamArgs& a, const f32x16 (&acc)[TM][TN], int64_t m0, int64_t tile_n,
                                         int wm, int wn, int r32, int kg, int lane, uint8_t* region,
                                         const float* lds_scale, const float* lds_tscale) {
  if (a.mode == OUT_SILU_BF16)
    tile_epilogue_lds_m<BN, WN, TM, TN, true>(a, acc, m0, tile_n, wm, wn, r32, kg, lane, region, lds_scale,
                                              lds_tscale);
  else
    tile_epilogue_lds_m<BN, WN, TM, TN, false>(a, acc, m0, tile_n, wm, wn, r32, kg, lane, region, lds_scale,
                                               lds_tscale);
}

// As tile_epilogue_lds, for fp32 outputs (F32 = true; the split-K
// partials of a K-sharded product): twice the bytes, so in two passes of
// TM / 2 row tiles each through the same region.  (Written for either
// element size, but used for fp32 only: the BF16 kernels keep the leaner
// function above.)
template <int BN, int WN, int TM, int TN, bool F32>
__device__ inline void tile_epilogue_lds_t(const StreamArgs& a, const f32x16 (&acc)[TM][TN], int64_t m0,
                                           int64_t tile_n, int wm, int wn, int r32, int kg, int lane, uint8_t* region,
                                           const float* lds_scale, const float* lds_tscale) {
  const bool silu_mode = !F32 && a.mode == OUT_SILU_BF16;
  constexpr bool f32_out = F32;
  constexpr int ROWS = TM * 32;
  static_assert(TM % 2 == 0, "fp32 outputs go in two halves of the row tiles");
  // output columns of the block: TN * 32, or TN * 16 in SiLU mode
  const int cols = silu_mode ? TN * 16 : TN * 32;
  constexpr int eb = F32 ? 4 : 2;      // bytes per output
  constexpr int epp = 16 / eb;          // outputs per 16-byte piece
  const int cpr = cols / epp;           // pieces per row (a power of two)
  const int64_t limit = silu_mode ? a.inter : a.rows;
  const int64_t col0 = silu_mode ? tile_n * (BN / 2) + wn * (WN / 2) : tile_n * BN + wn * WN;
  const int tn_out = silu_mode ? TN / 2 : TN;
  constexpr int passes = F32 ? 2 : 1;
  constexpr int xs = TM / passes;       // row tiles per pass
  auto pos = [&](int row, int col) {
    return row * cols * eb + (((col / epp) ^ (row & (cpr - 1))) << 4) + (col % epp) * eb;
  };
#pragma unroll
  for (int pass = 0; pass < passes; ++pass) {
    if (pass > 0) {
      // this wave's reads of the first half are done before it is overwritten
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int y = 0; y < TN; ++y) {
      if (y >= tn_out) break;
      const int c = wn * WN + y * 32 + r32;  // local B row
      const float sc = lds_scale[c];
      const float su = silu_mode ? lds_scale[c + WN / 2] : 1.f;
#pragma unroll
      for (int x = 0; x < TM; ++x) {
        if (x / (TM / 2) != pass && f32_out) continue;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = x * 32 + 8 * (v / 4) + 4 * kg + (v % 4);  // row in the wave's block
          const int prow = row - pass * xs * 32;                     // row in this pass
          const float ts = lds_tscale ? lds_tscale[wm * ROWS + row] : 1.f;
          float out = acc[x][y][v] * ts * sc;
          if (silu_mode) out = silu_tile(out) * (acc[x][y + TN / 2][v] * ts * su);
          if (f32_out)
            *reinterpret_cast<float*>(region + pos(prow, y * 32 + r32)) = out;
          else
            *reinterpret_cast<uint16_t*>(region + pos(prow, y * 32 + r32)) = bf16_bits(out);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    uint8_t* Y = static_cast<uint8_t*>(a.Y);
    const int pieces = xs * 32 * cpr;
    for (int q = lane; q < pieces; q += 64) {
      const int prow = q / cpr, cp = q % cpr;
      const int64_t m = m0 + wm * ROWS + pass * xs * 32 + prow;
      const int64_t col = col0 + cp * epp;
      if (m >= a.M || col >= limit) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(region + prow * cols * eb + ((cp ^ (prow & (cpr - 1))) << 4));
      uint8_t* dst = Y + (m * a.ldy + col) * eb;
      if (col + epp <= limit) {
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
        const uint8_t* h = reinterpret_cast<const uint8_t*>(&v);
        for (int e = 0; e < epp && col + e < limit; ++e)
          for (int b = 0; b < eb; ++b) dst[e * eb + b] = h[e * eb + b];
      }
    }
  }
}

// The E-byte slot of LDS stage memory that holds wave w's output block in the
// epilogue: the slots of a0, a1, [a2], b0, b1, [b2] in turn.
template <int E, int SA, int SB, int NS, int WAVES>
__device__ inline uint8_t* epi_region(int w, uint8_t* a0, uint8_t* a1, uint8_t* a2, uint8_t* b0, uint8_t* b1,
                                      uint8_t* b2) {
  constexpr int na = SA / E, nb = SB / E;
  static_assert(NS * (na + nb) >= WAVES, "the stages must hold every wave's output block");
  if (w < na) return a0 + w * E;
  w -= na;
  if (w < na) return a1 + w * E;
  w -= na;
  if (NS > 2) {
    if (w < na) return a2 + w * E;
    w -= na;
  }
  if (w < nb) return b0 + w * E;
  w -= nb;
  if (w < nb) return b1 + w * E;
  w -= nb;
  return b2 + w * E;
}

// Whether the LDS-staged epilogue applies: BF16 outputs whose rows all start
// 16-byte aligned.
__device__ inline bool epi_lds_ok(const StreamArgs& a) {
  return a.mode != OUT_F32 && (a.ldy % 8) == 0 && (reinterpret_cast<uintptr_t>(a.Y) % 16) == 0;
}

// The same for fp32 outputs (the kernels' F32OUT instantiations).
__device__ inline bool epi_lds_ok_f32(const StreamArgs& a) {
  return a.mode == OUT_F32 && (a.ldy % 4) == 0 && (reinterpret_cast<uintptr_t>(a.Y) % 16) == 0;
}

// ---------------------------------------------------------------------------
// FP8 weights: both operands reach LDS by buffer-to-LDS loads (no staging
// registers) through a three-stage ring, two k-steps ahead of the MFMAs.
//   * X stage: 256 rows x 128 B (bf16), the swizzled layout above; a load
//     instruction fills 1 KB = 8 rows, and each lane fetches the piece that
//     belongs at its position (the swizzle is applied to the source address);
//   * W stage: BN rows x 64 B of FP8 codes, piece q of row r at
//     r * 4 + (q ^ ((r >> 2) & 3)); a load instruction fills 16 rows;
//   * within each 32-K half s of a step, lane group g (0, 1) of an MFMA takes
//     K = 32*s + 16*g + 8*h .. +7 in the MFMA pair h = 0, 1, for both
//     operands: one 16-byte fragment read of 16 FP8 codes feeds both MFMAs
//     of the pair (the sum over K does not depend on the order);
//   * per step t, software-pipelined by 32-K slice: slice 1 of step t is read
//     while the MFMAs of slice 0 run; once this wave's reads of stage t and
//     its loads of step t + 1 are done (loads complete in issue order), the
//     barrier; the loads of step t + 3 go into stage t; slice 0 of step t + 1
//     is read while the MFMAs of slice 1 run.  The MFMAs after the barrier
//     use fragments already in registers, so no wave waits on LDS there;
//   * the pipeline is written out instruction by instruction: each MFMA is
//     followed by its share of the next slice's fragment reads (the W codes
//     into a second register set, each X fragment right after its last
//     MFMA), and scheduling barriers keep that order.  Left to itself the
//     compiler issues each slice's reads just before the MFMAs that use them
//     and waits on every few (measured on MI355X: the explicit order is 1-5%
//     faster per GEMM);
//   * the outputs leave through LDS (tile_epilogue_lds).
constexpr int kStages = 3;

__device__ inline int wswz(int row, int q) { return row * 4 + (q ^ ((row >> 2) & 3)); }

template <int BN, int WAVES, int BM = kTileM, bool F32OUT = false>
__device__ inline void fp8_tile_body(const StreamArgs& a, int64_t tile, int64_t ntiles) {
  constexpr int WGN = WAVES / 2;
  constexpr int WN = BN / WGN;
  constexpr int TM = BM / 64;
  constexpr int TN = WN / 32;
  constexpr int A_BYTES = BM * kTileK * 2;
  constexpr int B_BYTES = BN * kTileK;
  constexpr int NA = A_BYTES / 1024 / WAVES;
  constexpr int NB = B_BYTES / 1024 / WAVES;
  static_assert(TN >= 1 && NA >= 1 && NB >= 1 && NA * 1024 * WAVES == A_BYTES && NB * 1024 * WAVES == B_BYTES,
                "stage must split into whole 1 KB loads per wave");
  __shared__ __attribute__((aligned(1024))) uint8_t a0[A_BYTES], a1[A_BYTES], a2[A_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[B_BYTES], b1[B_BYTES], b2[B_BYTES];
  __shared__ __attribute__((aligned(4096))) float row_scale[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const TileCoord tc = tile_coord<BN, BM>(a, tile, ntiles);
  const int64_t m0 = tc.m0;
  for (int c = tid; c < BN; c += 64 * WAVES) {
    const int64_t r = w_row<BN, WN>(a, tc.tile_n, c);
    row_scale[c] = (a.scale && r < a.rows) ? a.scale[r] : 1.f;
  }

  const u32x4s xres = raw_rsrc(a.X, a.M * a.ldx * 2);
  const u32x4s wres = raw_rsrc(a.W, a.rows * a.K);
  int aoff[NA], boff[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = (wave * NA + i) * 8 + lane / 8;
    const int piece = (lane % 8) ^ ((row >> 1) & 7);
    const int64_t m = min(m0 + row, a.M - 1);
    aoff[i] = int((m * a.ldx + piece * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = (wave * NB + i) * 16 + lane / 4;
    const int q = (lane % 4) ^ ((row >> 2) & 3);
    const int64_t r = min(w_row<BN, WN>(a, tc.tile_n, row), a.rows - 1);
    boff[i] = int(r * a.K + q * 16);
  }
  auto issue = [&](uint8_t* A, uint8_t* B, int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; ++i) lds_load16<false>(xres, A + (wave * NA + i) * 1024, aoff[i], kt * kTileK * 2);
#pragma unroll
    for (int i = 0; i < NB; ++i) lds_load16<false>(wres, B + (wave * NB + i) * 1024, boff[i], kt * kTileK);
  };

  const int r32 = lane & 31, kg = lane >> 5;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int x = 0; x < TM; ++x)
#pragma unroll
    for (int y = 0; y < TN; ++y) acc[x][y] = f32x16{};

  // slice s (0, 1) of a stage: W codes of tile y, X fragment of half h, tile x
  bf16x8 fa[2][TM];
  u32x4 fw[2][TN];
  auto w_piece = [&](const uint8_t* B, int s, int y) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4*>(B + wswz(wn * WN + y * 32 + r32, 2 * s + kg) * 16);
  };
  auto a_piece = [&](const uint8_t* A, int s, int h, int x) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(A + swz(wm * (BM / 2) + x * 32 + r32, 4 * s + 2 * kg + h) * 16);
  };
  // The MFMAs of the current slice (W codes in set c), each followed by one
  // read of slice s_next of stage (A, B): first the W codes into set 1 - c,
  // then each X fragment right after its last MFMA.
  auto mma_read = [&](auto cc, const uint8_t* A, const uint8_t* B, int s_next) __attribute__((always_inline)) {
    constexpr int c = decltype(cc)::value;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 fb[TN];
#pragma unroll
      for (int y = 0; y < TN; ++y) fb[y] = fp8x8_to_bf16(fw[c][y][2 * h], fw[c][y][2 * h + 1]);
#pragma unroll
      for (int x = 0; x < TM; ++x) {
#pragma unroll
        for (int y = 0; y < TN; ++y) {
          acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[h][x], fb[y], acc[x][y], 0, 0, 0);
          const int i = (h * TM + x) * TN + y;
          if (h == 0 && i < TN) fw[1 - c][i] = w_piece(B, s_next, i);
          __builtin_amdgcn_sched_barrier(0x0006);
        }
        fa[h][x] = a_piece(A, s_next, h, x);
        __builtin_amdgcn_sched_barrier(0x0006);
      }
    }
  };

  constexpr int kLoads = NA + NB;
  const int nk = int(a.K / kTileK);
  issue(a0, b0, 0);
  if (nk > 1) issue(a1, b1, 1);
  if (nk > 1)
    wait_vm<kLoads>();
  else
    wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  if (nk > 2) issue(a2, b2, 2);
#pragma unroll
  for (int y = 0; y < TN; ++y) fw[0][y] = w_piece(b0, 0, y);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int x = 0; x < TM; ++x) fa[h][x] = a_piece(a0, 0, h, x);
  __builtin_amdgcn_sched_barrier(0);

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  // Step t: slice 0's MFMAs read slice 1; then, once this wave's reads of
  // stage t and its loads of step t + 1 are done, the barrier; the loads of
  // step t + 3 go into stage t; slice 1's MFMAs read slice 0 of step t + 1
  // (after the last step: stale fragments, never used).
  auto iter = [&](uint8_t* A, uint8_t* B, const uint8_t* An, const uint8_t* Bn, int kt) __attribute__((always_inline)) {
    mma_read(C0{}, A, B, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) {
      if (kt + 2 < nk)
        wait_vm_lds<kLoads>();
      else
        wait_vm_lds<0>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 3 < nk) issue(A, B, kt + 3);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma_read(C1{}, An, Bn, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  int kt = 0;
  for (; kt + kStages <= nk; kt += kStages) {
    iter(a0, b0, a1, b1, kt);
    iter(a1, b1, a2, b2, kt + 1);
    iter(a2, b2, a0, b0, kt + 2);
  }
  if (kt < nk) iter(a0, b0, a1, b1, kt);
  if (kt + 1 < nk) iter(a1, b1, a2, b2, kt + 1);
  wait_vm<0>();
  if (F32OUT ? epi_lds_ok_f32(a) : epi_lds_ok(a)) {
    __syncthreads();  // every wave is done with the stages
    constexpr int E = TM * TN * 32 * 32 * 2;
    uint8_t* region = epi_region<E, A_BYTES, B_BYTES, 3, WAVES>(wave, a0, a1, a2, b0, b1, b2);
    if constexpr (F32OUT)
      tile_epilogue_lds_t<BN, WN, TM, TN, true>(a, acc, m0, tc.tile_n, wm, wn, r32, kg, lane, region, row_scale,
                                                nullptr);
    else
      tile_epilogue_lds<BN, WN, TM, TN>(a, acc, m0, tc.tile_n, wm, wn, r32, kg, lane, region, row_scale, nullptr);
  } else {
    tile_epilogue<BN, WN, TM, TN>(a, acc, m0, tc.tile_n, wm, wn, r32, kg, row_scale);
  }
}

// ---------------------------------------------------------------------------
// FP8 weights and FP8 activations (codes of both operands, one fp32 scale per
// token in StreamArgs::xscale) in 64-K steps, for K a multiple of 64 but not
// of 128 (otherwise the double-step kernel below): both operands by
// buffer-to-LDS loads through a four-stage ring, three steps ahead.
//   * X stage: 256 rows x 64 B, W stage: BN rows x 64 B, both with piece q of
//     row r at r * 4 + (q ^ ((r >> 2) & 3)); a load instruction fills 16 rows;
//   * a step is one v_mfma_scale_f32_32x32x64_f8f6f4 per tile pair (E4M3 x
//     E4M3, no block scale): lane group g reads pieces 2g and 2g + 1
//     (K = 32g .. 32g + 31);
//   * per step: wait until this wave's loads of step t have landed, barrier,
//     issue the loads of step t + 3 into the stage that step t - 1 read,
//     multiply step t.
template <int BN, int WAVES>
__device__ inline void ring_tile_body(const StreamArgs& a, int64_t tile, int64_t ntiles) {
  constexpr int WGN = WAVES / 2;
  constexpr int WN = BN / WGN;
  constexpr int TM = 4;
  constexpr int TN = WN / 32;
  constexpr int BK = 64;                     // K per step: 64 bytes of every row
  constexpr int A_BYTES = kTileM * BK;       // 16 KB
  constexpr int B_BYTES = BN * BK;
  constexpr int NA = A_BYTES / 1024 / WAVES;  // 1 KB loads of X per wave per step
  constexpr int NB = B_BYTES / 1024 / WAVES;  // 1 KB loads of W per wave per step
  static_assert(TN >= 1 && NA >= 1 && NB >= 1 && NA * 1024 * WAVES == A_BYTES && NB * 1024 * WAVES == B_BYTES,
                "stage must split into whole 1 KB loads per wave");
  __shared__ __attribute__((aligned(1024))) uint8_t a0[A_BYTES], a1[A_BYTES], a2[A_BYTES], a3[A_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[B_BYTES], b1[B_BYTES], b2[B_BYTES], b3[B_BYTES];
  // first in LDS, for the same reason as in the FP8 kernel
  __shared__ __attribute__((aligned(4096))) float row_scale[BN];
  __shared__ float tok_scale[kTileM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const TileCoord tc = tile_coord<BN>(a, tile, ntiles);
  const int64_t m0 = tc.m0;
  for (int c = tid; c < BN; c += 64 * WAVES) {
    const int64_t r = w_row<BN, WN>(a, tc.tile_n, c);
    row_scale[c] = (a.scale && r < a.rows) ? a.scale[r] : 1.f;
  }
  for (int c = tid; c < kTileM; c += 64 * WAVES) tok_scale[c] = m0 + c < a.M ? a.xscale[m0 + c] : 0.f;

  const u32x4s xres = raw_rsrc(a.X, a.M * a.ldx);
  const u32x4s wres = raw_rsrc(a.W, a.rows * a.K);
  // Source offsets of this lane's pieces (step 0): a load fills rows
  // 16 * i .. 16 * i + 15 of the stage, lane l position l % 4 of row l / 4;
  // rows past the end are read from the last row and never stored.
  int aoff[NA], boff[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = (wave * NA + i) * 16 + lane / 4;
    const int q = (lane % 4) ^ ((row >> 2) & 3);
    const int64_t m = min(m0 + row, a.M - 1);
    aoff[i] = int(m * a.ldx + q * 16);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = (wave * NB + i) * 16 + lane / 4;
    const int q = (lane % 4) ^ ((row >> 2) & 3);
    const int64_t r = min(w_row<BN, WN>(a, tc.tile_n, row), a.rows - 1);
    boff[i] = int(r * a.K + q * 16);
  }
  auto issue = [&](uint8_t* A, uint8_t* B, int kt) {
#pragma unroll
    for (int i = 0; i < NA; ++i) lds_load16<false>(xres, A + (wave * NA + i) * 1024, aoff[i], kt * 64);
#pragma unroll
    for (int i = 0; i < NB; ++i) lds_load16<false>(wres, B + (wave * NB + i) * 1024, boff[i], kt * 64);
  };

  const int r32 = lane & 31, kg = lane >> 5;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int x = 0; x < TM; ++x)
#pragma unroll
    for (int y = 0; y < TN; ++y) acc[x][y] = f32x16{};

  auto compute = [&](const uint8_t* A, const uint8_t* B) {
    // 32 codes per lane: pieces 2g and 2g + 1 of its row
    i32x8 fa[TM], fb[TN];
    auto frag = [&](const uint8_t* base, int row) {
      const u32x4 lo = *reinterpret_cast<const u32x4*>(base + wswz(row, 2 * kg) * 16);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(base + wswz(row, 2 * kg + 1) * 16);
      return i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
    };
#pragma unroll
    for (int x = 0; x < TM; ++x) fa[x] = frag(A, wm * 128 + x * 32 + r32);
#pragma unroll
    for (int y = 0; y < TN; ++y) fb[y] = frag(B, wn * WN + y * 32 + r32);
#pragma unroll
    for (int x = 0; x < TM; ++x)
#pragma unroll
      for (int y = 0; y < TN; ++y)
        acc[x][y] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[x], fb[y], acc[x][y], 0, 0, 0, 0, 0, 0);
  };

  constexpr int kLoads = NA + NB;  // loads per wave per step
  const int nk = int(a.K / BK);
  // prologue: steps 0, 1 and 2 in flight
  issue(a0, b0, 0);
  if (nk > 1) issue(a1, b1, 1);
  if (nk > 2) issue(a2, b2, 2);

  // Step t uses stage t % 4; the loop is unrolled by the ring so every stage
  // is a fixed array.  A step opens with the wait for its own loads (those of
  // the next two steps may stay in flight) and a barrier, which also frees
  // the stage that step t - 1 read for the loads of step t + 3.
  auto step = [&](const uint8_t* A, const uint8_t* B, uint8_t* An, uint8_t* Bn, int kt) {
    if (kt + 2 < nk)
      wait_vm<2 * kLoads>();
    else if (kt + 1 < nk)
      wait_vm<kLoads>();
    else
      wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 3 < nk) issue(An, Bn, kt + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute(A, B);
    __builtin_amdgcn_sched_barrier(0);
  };
  // whole ring cycles without branches around the MFMAs, then the tail
  int kt = 0;
  for (; kt + 4 <= nk; kt += 4) {
    step(a0, b0, a3, b3, kt);
    step(a1, b1, a0, b0, kt + 1);
    step(a2, b2, a1, b1, kt + 2);
    step(a3, b3, a2, b2, kt + 3);
  }
  if (kt < nk) step(a0, b0, a3, b3, kt);
  if (kt + 1 < nk) step(a1, b1, a0, b0, kt + 1);
  if (kt + 2 < nk) step(a2, b2, a1, b1, kt + 2);
  wait_vm<0>();
  if (epi_lds_ok(a)) {
    __syncthreads();  // every wave is done with the stages
    // one 16 KB X stage per wave block (BN = 256: 16 KB W stages for waves 4 .. 7)
    constexpr int E = TM * TN * 32 * 32 * 2;
    static_assert(E == A_BYTES && (WAVES <= 4 || E == B_BYTES), "one stage per wave block");
    const int q = wave & 3;
    uint8_t* region = wave < 4 ? (q == 0 ? a0 : q == 1 ? a1 : q == 2 ? a2 : a3)
                               : (q == 0 ? b0 : q == 1 ? b1 : q == 2 ? b2 : b3);
    tile_epilogue_lds<BN, WN, TM, TN>(a, acc, m0, tc.tile_n, wm, wn, r32, kg, lane, region, row_scale, tok_scale);
  } else {
    tile_epilogue<BN, WN, TM, TN>(a, acc, m0, tc.tile_n, wm, wn, r32, kg, row_scale, tok_scale);
  }
}

// ---------------------------------------------------------------------------
// Both operands in double steps of 128 bytes per row (128 K of FP8 codes for
// FP8 weights with FP8 activations here, 64 K of BF16 for BF16 weights and
// activations in bf16_dstep_body below), so each buffer-to-LDS load fills 8
// whole 128-byte lines (1 KB) instead of 16 half lines: half the requests per
// byte of the 64-byte rows of the ring kernel above.  (Measured on MI355X:
// the 64-K kernel is bound by these loads -- with them removed it runs twice
// as fast, while removing its MFMAs or its fragment reads changes nothing --
// and the double steps take the FP8-activation MLP from 1.39 to 1.08 ms at
// 4096 tokens and from 5.50 to 4.08 ms at 16384; for BF16 the sharded-matmul
// GEMMs gain 8-11%.)  NST double stages in LDS (2 for 256-row tiles, 3 for
// 128-row ones), loads NST - 1 double steps ahead; the layout is the 128-byte
// row swizzle swz() of the FP8-weight kernel's X.  Within a double step, MFMA
// slice s (0, 1) takes K = 64s .. 64s + 63: lane group g reads pieces 4s + 2g
// and 4s + 2g + 1 of its row in both operands.  (The slice pipeline of the
// BF16 body, written out the same way here, needs 64 more registers than the
// eight waves have and spills: measured 9-12% slower.)
template <int BN, int WAVES, int NST, int BM = kTileM>
__device__ inline void f8f8_dstep_body(const StreamArgs& a, int64_t tile, int64_t ntiles) {
  constexpr int WGN = WAVES / 2;
  constexpr int WN = BN / WGN;
  constexpr int TM = BM / 64;  // two rows of waves along the tokens
  constexpr int TN = WN / 32;
  constexpr int DK = 128;                     // bytes (FP8 codes) of a row per double step
  constexpr int A_BYTES = BM * DK;             // 32 KB for 256 tokens
  constexpr int B_BYTES = BN * DK;
  constexpr int NA = A_BYTES / 1024 / WAVES;  // 1 KB loads of X per wave per double step
  constexpr int NB = B_BYTES / 1024 / WAVES;
  static_assert(TN >= 1 && NA >= 1 && NB >= 1 && NA * 1024 * WAVES == A_BYTES && NB * 1024 * WAVES == B_BYTES,
                "stage must split into whole 1 KB loads per wave");
  static_assert(NST == 2 || NST == 3, "two or three double stages");
  __shared__ __attribute__((aligned(1024))) uint8_t a0[A_BYTES], a1[A_BYTES], a2[NST > 2 ? A_BYTES : 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[B_BYTES], b1[B_BYTES], b2[NST > 2 ? B_BYTES : 1024];
  __shared__ __attribute__((aligned(4096))) float row_scale[BN];
  __shared__ float tok_scale[BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const TileCoord tc = tile_coord<BN, BM>(a, tile, ntiles);
  const int64_t m0 = tc.m0;
  for (int c = tid; c < BN; c += 64 * WAVES) {
    const int64_t r = w_row<BN, WN>(a, tc.tile_n, c);
    row_scale[c] = (a.scale && r < a.rows) ? a.scale[r] : 1.f;
  }
  for (int c = tid; c < BM; c += 64 * WAVES) tok_scale[c] = m0 + c < a.M ? a.xscale[m0 + c] : 0.f;

  const u32x4s xres = raw_rsrc(a.X, a.M * a.ldx);
  const u32x4s wres = raw_rsrc(a.W, a.rows * a.K);
  // a load fills rows 8i .. 8i + 7 of the stage: lane l writes slot l % 8 of
  // row l / 8, which holds piece (l % 8) ^ ((row >> 1) & 7) of that row
  int aoff[NA], boff[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = (wave * NA + i) * 8 + lane / 8;
    const int q = (lane % 8) ^ ((row >> 1) & 7);
    const int64_t m = min(m0 + row, a.M - 1);
    aoff[i] = int(m * a.ldx + q * 16);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = (wave * NB + i) * 8 + lane / 8;
    const int q = (lane % 8) ^ ((row >> 1) & 7);
    const int64_t r = min(w_row<BN, WN>(a, tc.tile_n, row), a.rows - 1);
    boff[i] = int(r * a.K + q * 16);
  }
  auto issue = [&](uint8_t* A, uint8_t* B, int kd) {
#pragma unroll
    for (int i = 0; i < NA; ++i) lds_load16<false>(xres, A + (wave * NA + i) * 1024, aoff[i], kd * DK);
#pragma unroll
    for (int i = 0; i < NB; ++i) lds_load16<false>(wres, B + (wave * NB + i) * 1024, boff[i], kd * DK);
  };

  const int r32 = lane & 31, kg = lane >> 5;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int x = 0; x < TM; ++x)
#pragma unroll
    for (int y = 0; y < TN; ++y) acc[x][y] = f32x16{};

  auto frag = [&](const uint8_t* base, int row, int s) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + swz(row, 4 * s + 2 * kg) * 16);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + swz(row, 4 * s + 2 * kg + 1) * 16);
    return i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
  };
  auto compute = [&](const uint8_t* A, const uint8_t* B) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      i32x8 fa[TM], fb[TN];
#pragma unroll
      for (int x = 0; x < TM; ++x) fa[x] = frag(A, wm * (BM / 2) + x * 32 + r32, s);
#pragma unroll
      for (int y = 0; y < TN; ++y) fb[y] = frag(B, wn * WN + y * 32 + r32, s);
#pragma unroll
      for (int x = 0; x < TM; ++x)
#pragma unroll
        for (int y = 0; y < TN; ++y)
          acc[x][y] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[x], fb[y], acc[x][y], 0, 0, 0, 0, 0, 0);
    }
  };

  constexpr int kLoads = NA + NB;  // loads per wave per double step
  const int nd = int(a.K / DK);
  // prologue: double steps 0 .. NST - 2 in flight
  issue(a0, b0, 0);
  if (NST > 2 && nd > 1) issue(a1, b1, 1);
  // Double step d uses stage d % NST.  It opens with the wait for this
  // wave's loads of step d (those of d + 1 may stay in flight with three
  // stages) and a barrier, which also frees the stage that step d - 1 read
  // for the loads of step d + NST - 1.
  auto step = [&](const uint8_t* A, const uint8_t* B, uint8_t* An, uint8_t* Bn, int kd) {
    if (NST > 2 && kd + 1 < nd)
      wait_vm<kLoads>();
    else
      wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (kd + NST - 1 < nd) issue(An, Bn, kd + NST - 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(A, B);
    __builtin_amdgcn_sched_barrier(0);
  };
  int kd = 0;
  if constexpr (NST == 2) {
    for (; kd + 2 <= nd; kd += 2) {
      step(a0, b0, a1, b1, kd);
      step(a1, b1, a0, b0, kd + 1);
    }
    if (kd < nd) step(a0, b0, a1, b1, kd);
  } else {
    for (; kd + 3 <= nd; kd += 3) {
      step(a0, b0, a2, b2, kd);
      step(a1, b1, a0, b0, kd + 1);
      step(a2, b2, a1, b1, kd + 2);
    }
    if (kd < nd) step(a0, b0, a2, b2, kd);
    if (kd + 1 < nd) step(a1, b1, a0, b0, kd + 1);
  }
  wait_vm<0>();
  if (epi_lds_ok(a)) {
    __syncthreads();  // every wave is done with the stages
    constexpr int E = TM * TN * 32 * 32 * 2;
    uint8_t* region = epi_region<E, A_BYTES, B_BYTES, NST, WAVES>(wave, a0, a1, a2, b0, b1, b2);
    tile_epilogue_lds<BN, WN, TM, TN>(a, acc, m0, tc.tile_n, wm, wn, r32, kg, lane, region, row_scale, tok_scale);
  } else {
    tile_epilogue<BN, WN, TM, TN>(a, acc, m0, tc.tile_n, wm, wn, r32, kg, row_scale, tok_scale);
  }
}

// BF16 weights and BF16 activations in double steps of 64 K (128-byte rows,
// as above), slice-pipelined: the double step's four 16-K MFMA slices (lane
// group g reads piece 2s + g of its row in slice s) are written out so that
// each MFMA is followed by its share of the next slice's fragment reads -- the
// W fragments into a second register set, each X fragment right after its
// last MFMA of the slice -- and scheduling barriers keep that order (MFMAs and
// LDS reads; address arithmetic moves freely).  The step's barrier sits before
// the last slice's MFMAs, whose fragments are already in registers; right
// after it the wave issues the loads of step d + NST into the stage it has
// just finished and reads slice 0 of step d + 1 while those MFMAs run.  Left
// to itself the compiler reads each slice's fragments just before its MFMAs
// and waits on them every two MFMAs (measured on MI355X: this order is 3-8%
// faster on the prefill and sharded-matmul GEMMs, and the LDS-staged
// epilogue another 4-9%).
template <int BN, int WAVES, int NST, bool F32OUT = false>
__device__ inline void bf16_dstep_body(const StreamArgs& a, int64_t tile, int64_t ntiles) {
  constexpr int BM = kTileM;
  constexpr int WGN = WAVES / 2;
  constexpr int WN = BN / WGN;
  constexpr int TM = BM / 64;  // two rows of waves along the tokens
  constexpr int TN = WN / 32;
  constexpr int DK = 128;       // bytes of a row per double step (64 K)
  constexpr int A_BYTES = BM * DK;
  constexpr int B_BYTES = BN * DK;
  constexpr int NA = A_BYTES / 1024 / WAVES;  // 1 KB loads of X per wave per double step
  constexpr int NB = B_BYTES / 1024 / WAVES;
  static_assert(TN >= 1 && NA >= 1 && NB >= 1 && NA * 1024 * WAVES == A_BYTES && NB * 1024 * WAVES == B_BYTES,
                "stage must split into whole 1 KB loads per wave");
  static_assert(NST == 2 || NST == 3, "two or three double stages");
  __shared__ __attribute__((aligned(1024))) uint8_t a0[A_BYTES], a1[A_BYTES], a2[NST > 2 ? A_BYTES : 1024];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[B_BYTES], b1[B_BYTES], b2[NST > 2 ? B_BYTES : 1024];
  __shared__ __attribute__((aligned(4096))) float row_scale[BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const TileCoord tc = tile_coord<BN, BM>(a, tile, ntiles);
  const int64_t m0 = tc.m0;
  for (int c = tid; c < BN; c += 64 * WAVES) {
    const int64_t r = w_row<BN, WN>(a, tc.tile_n, c);
    row_scale[c] = (a.scale && r < a.rows) ? a.scale[r] : 1.f;
  }

  const u32x4s xres = raw_rsrc(a.X, a.M * a.ldx * 2);
  const u32x4s wres = raw_rsrc(a.W, a.rows * a.K * 2);
  // a load fills rows 8i .. 8i + 7 of the stage: lane l writes slot l % 8 of
  // row l / 8, which holds piece (l % 8) ^ ((row >> 1) & 7) of that row
  int aoff[NA], boff[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = (wave * NA + i) * 8 + lane / 8;
    const int q = (lane % 8) ^ ((row >> 1) & 7);
    const int64_t m = min(m0 + row, a.M - 1);
    aoff[i] = int(m * a.ldx * 2 + q * 16);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = (wave * NB + i) * 8 + lane / 8;
    const int q = (lane % 8) ^ ((row >> 1) & 7);
    const int64_t r = min(w_row<BN, WN>(a, tc.tile_n, row), a.rows - 1);
    boff[i] = int(r * a.K * 2 + q * 16);
  }
  // (the lambdas are forced inline: out of line, the stage pointers would
  // lose their address space and the accumulators would live in memory)
  auto issue = [&](uint8_t* A, uint8_t* B, int kd) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NA; ++i) lds_load16<false>(xres, A + (wave * NA + i) * 1024, aoff[i], kd * DK);
#pragma unroll
    for (int i = 0; i < NB; ++i) lds_load16<false>(wres, B + (wave * NB + i) * 1024, boff[i], kd * DK);
  };

  const int r32 = lane & 31, kg = lane >> 5;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int x = 0; x < TM; ++x)
#pragma unroll
    for (int y = 0; y < TN; ++y) acc[x][y] = f32x16{};

  // X fragments in one set, W fragments in two (current, next slice)
  bf16x8 fa[TM], fb[2][TN];
  auto a_frag = [&](const uint8_t* A, int s, int x) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(A + swz(wm * (BM / 2) + x * 32 + r32, 2 * s + kg) * 16);
  };
  auto b_frag = [&](const uint8_t* B, int s, int y) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(B + swz(wn * WN + y * 32 + r32, 2 * s + kg) * 16);
  };
  // The MFMAs of the current slice (W fragments in set c, a compile-time
  // constant so that the sets stay in registers), reading slice s_next of
  // stage (A, B): W fragment y after MFMA y, X fragment x after its last MFMA.
  auto mma_read = [&](auto cc, const uint8_t* A, const uint8_t* B, int s_next) __attribute__((always_inline)) {
    constexpr int c = decltype(cc)::value;
#pragma unroll
    for (int x = 0; x < TM; ++x) {
#pragma unroll
      for (int y = 0; y < TN; ++y) {
        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[x], fb[c][y], acc[x][y], 0, 0, 0);
        const int i = x * TN + y;
        if (i < TN) fb[1 - c][i] = b_frag(B, s_next, i);
        __builtin_amdgcn_sched_barrier(0x0006);
      }
      fa[x] = a_frag(A, s_next, x);
      __builtin_amdgcn_sched_barrier(0x0006);
    }
  };

  constexpr int kLoads = NA + NB;  // loads per wave per double step
  const int nd = int(a.K * 2 / DK);
  // prologue: double steps 0 .. NST - 1 in flight, step 0 landed everywhere,
  // slice 0 of step 0 in registers
  issue(a0, b0, 0);
  if (nd > 1) issue(a1, b1, 1);
  if (NST > 2 && nd > 2) issue(a2, b2, 2);
  if (nd >= NST)
    wait_vm<(NST - 1) * kLoads>();
  else if (nd == 2)
    wait_vm<kLoads>();
  else
    wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int x = 0; x < TM; ++x) fa[x] = a_frag(a0, 0, x);
#pragma unroll
  for (int y = 0; y < TN; ++y) fb[0][y] = b_frag(b0, 0, y);
  __builtin_amdgcn_sched_barrier(0);

  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  // Double step d in stage (A, B); (An, Bn) holds step d + 1.  Slices 0..2
  // each read the next; then, once this wave's loads of step d + 1 have
  // landed (with three stages those of d + 2 may stay in flight) and its
  // reads of stage d are done, the barrier: every wave is past stage d (the
  // loads of step d + NST may overwrite it) and step d + 1 has landed
  // everywhere.  Slice 3 reads slice 0 of step d + 1 (after the last step:
  // stale fragments, never used -- no branch around the MFMAs, which would
  // merge two copies of the accumulators).
  auto step = [&](uint8_t* A, uint8_t* B, const uint8_t* An, const uint8_t* Bn, int kd) __attribute__((always_inline)) {
    mma_read(C0{}, A, B, 1);
    mma_read(C1{}, A, B, 2);
    mma_read(C0{}, A, B, 3);
    if (kd + 1 < nd) {
      if (NST > 2 && kd + 2 < nd)
        wait_vm_lds<kLoads>();
      else
        wait_vm_lds<0>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (kd + NST < nd) issue(A, B, kd + NST);
    }
    __builtin_amdgcn_sched_barrier(0);
    mma_read(C1{}, An, Bn, 0);
  };
  int kd = 0;
  if constexpr (NST == 2) {
    for (; kd + 2 <= nd; kd += 2) {
      step(a0, b0, a1, b1, kd);
      step(a1, b1, a0, b0, kd + 1);
    }
    if (kd < nd) step(a0, b0, a1, b1, kd);
  } else {
    for (; kd + 3 <= nd; kd += 3) {
      step(a0, b0, a1, b1, kd);
      step(a1, b1, a2, b2, kd + 1);
      step(a2, b2, a0, b0, kd + 2);
    }
    if (kd < nd) step(a0, b0, a1, b1, kd);
    if (kd + 1 < nd) step(a1, b1, a2, b2, kd + 1);
  }
  wait_vm<0>();
  if (F32OUT ? epi_lds_ok_f32(a) : epi_lds_ok(a)) {
    __syncthreads();  // every wave is done with the stages
    constexpr int E = TM * TN * 32 * 32 * 2;
    uint8_t* region = epi_region<E, A_BYTES, B_BYTES, NST, WAVES>(wave, a0, a1, a2, b0, b1, b2);
    if constexpr (F32OUT)
      tile_epilogue_lds_t<BN, WN, TM, TN, true>(a, acc, m0, tc.tile_n, wm, wn, r32, kg, lane, region, row_scale,
                                                nullptr);
    else
      tile_epilogue_lds<BN, WN, TM, TN>(a, acc, m0, tc.tile_n, wm, wn, r32, kg, lane, region, row_scale, nullptr);
  } else {
    tile_epilogue<BN, WN, TM, TN>(a, acc, m0, tc.tile_n, wm, wn, r32, kg, row_scale);
  }
}

template <int BN, int WAVES, int NST, int BM = kTileM>
__global__ __launch_bounds__(64 * WAVES, 1) void tile_gemm_f8f8d_kernel(StreamArgs a) {
  f8f8_dstep_body<BN, WAVES, NST, BM>(a, blockIdx.x, gridDim.x);
}

// (F32OUT: the instantiation for fp32 outputs, whose epilogue stages them
// through LDS in two halves; kept apart, the BF16-output kernels do not
// carry its registers -- measured 3% faster)
template <int BN, int WAVES, int NST, bool F32OUT = false>
__global__ __launch_bounds__(64 * WAVES, 1) void tile_gemm_bf16d_kernel(StreamArgs a) {
  bf16_dstep_body<BN, WAVES, NST, F32OUT>(a, blockIdx.x, gridDim.x);
}

template <int BN, int WAVES, int BM = kTileM, bool F32OUT = false>
__global__ __launch_bounds__(64 * WAVES, 1) void tile_gemm_fp8_kernel(StreamArgs a) {
  fp8_tile_body<BN, WAVES, BM, F32OUT>(a, blockIdx.x, gridDim.x);
}

// FP8 weights and FP8 activations in 64-K steps, for K a multiple of 64 but
// not of 128; otherwise tile_gemm_f8f8d_kernel
template <int BN, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void tile_gemm_f8f8_kernel(StreamArgs a) {
  ring_tile_body<BN, WAVES>(a, blockIdx.x, gridDim.x);
}

// Several GEMMs of one weight dtype in one launch (a layer's projections, the
// shards of a sharded product): workgroup x computes tile x - first[g] of
// problem g, the g with first[g] <= x < first[g + 1].
template <int BN, int WAVES, bool FP8, bool F32OUT = false>
__global__ __launch_bounds__(64 * WAVES, 1) void tile_group_kernel(TileGroup tg) {
  const int64_t x = blockIdx.x;
  int g = 0;
  while (g + 1 < tg.n && x >= tg.first[g + 1]) ++g;
  g = __builtin_amdgcn_readfirstlane(g);  // one problem per workgroup
  if constexpr (FP8)
    fp8_tile_body<BN, WAVES, kTileM, F32OUT>(tg.g[g], x - tg.first[g], tg.first[g + 1] - tg.first[g]);
  else
    bf16_dstep_body<BN, WAVES, BN == 256 ? 2 : 3, F32OUT>(tg.g[g], x - tg.first[g], tg.first[g + 1] - tg.first[g]);
}

int64_t tile_count(const StreamArgs& a, int bn, int bm = kTileM) {
  const bool silu_mode = a.mode == OUT_SILU_BF16;
  const int64_t tiles_m = (a.M + bm - 1) / bm;
  const int64_t cols = silu_mode ? a.inter : a.rows;
  const int64_t col_tile = silu_mode ? bn / 2 : bn;
  const int64_t tiles_n = (cols + col_tile - 1) / col_tile;
  return tiles_m * tiles_n;
}

template <int BN, int BM = kTileM>
dim3 tile_grid(const StreamArgs& a) {
  return dim3(unsigned(tile_count(a, BN, BM)));
}

template <int BN, int WAVES>
hipError_t launch_f8f8_ring(const StreamArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((tile_gemm_f8f8_kernel<BN, WAVES>), tile_grid<BN>(a), dim3(64 * WAVES), 0, stream, a);
  return hipGetLastError();
}

template <int BN, int WAVES, int NST>
hipError_t launch_bf16d(const StreamArgs& a, hipStream_t stream) {
  if (a.mode == OUT_F32)
    hipLaunchKernelGGL((tile_gemm_bf16d_kernel<BN, WAVES, NST, true>), tile_grid<BN>(a), dim3(64 * WAVES), 0, stream, a);
  else
    hipLaunchKernelGGL((tile_gemm_bf16d_kernel<BN, WAVES, NST>), tile_grid<BN>(a), dim3(64 * WAVES), 0, stream, a);
  return hipGetLastError();
}

template <int BN, int WAVES>
hipError_t launch_fp8(const StreamArgs& a, hipStream_t stream) {
  if (a.mode == OUT_F32)
    hipLaunchKernelGGL((tile_gemm_fp8_kernel<BN, WAVES, kTileM, true>), tile_grid<BN>(a), dim3(64 * WAVES), 0, stream, a);
  else
    hipLaunchKernelGGL((tile_gemm_fp8_kernel<BN, WAVES>), tile_grid<BN>(a), dim3(64 * WAVES), 0, stream, a);
  return hipGetLastError();
}

template <int BN, int WAVES, bool FP8>
hipError_t launch_group(const TileGroup& tg, hipStream_t stream) {
  // the fp32-output instantiation when every problem of the group writes fp32
  bool f32 = tg.n > 0;
  for (int i = 0; i < tg.n; ++i) f32 = f32 && tg.g[i].mode == OUT_F32;
  if (f32)
    hipLaunchKernelGGL((tile_group_kernel<BN, WAVES, FP8, true>), dim3(unsigned(tg.first[tg.n])), dim3(64 * WAVES), 0,
                       stream, tg);
  else
    hipLaunchKernelGGL((tile_group_kernel<BN, WAVES, FP8>), dim3(unsigned(tg.first[tg.n])), dim3(64 * WAVES), 0,
                       stream, tg);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_group(const StreamArgs* as, int n, int bn, bool fp8, hipStream_t stream) {
  if (n < 1 || n > kMaxGroup) return hipErrorInvalidValue;
  TileGroup tg{};
  tg.n = n;
  tg.first[0] = 0;
  for (int i = 0; i < n; ++i) {
    tg.g[i] = as[i];
    tg.first[i + 1] = tg.first[i] + tile_count(as[i], bn);
  }
  if (tg.first[n] == 0) return hipSuccess;
  if (tg.first[n] >= (INT64_C(1) << 31)) return hipErrorInvalidValue;
  if (bn != 256) return fp8 ? launch_group<128, 4, true>(tg, stream) : launch_group<128, 4, false>(tg, stream);
  // As launch_tile_gemm: where the last wave of 256-row tiles would be at
  // most half full, whole columns of those tiles (the last rows of the last
  // problems) move to 128-row tiles in a second launch.  The problems of a
  // group share M, so a column is tiles_m tiles.
  const int64_t tiles_m = (as[0].M + kTileM - 1) / kTileM;
  const int64_t rem = tg.first[n] % 256;
  bool same_m = true;
  for (int i = 0; i < n; ++i) same_m = same_m && as[i].M == as[0].M && as[i].mode != OUT_SILU_BF16;
  if (!same_m || tg.first[n] <= 256 || rem == 0 || rem > 128 || rem % tiles_m != 0)
    return fp8 ? launch_group<256, 8, true>(tg, stream) : launch_group<256, 8, false>(tg, stream);
  int64_t cols = rem / tiles_m;  // 256-row columns to move
  TileGroup tail{};
  const int64_t y_elem = as[0].mode == OUT_F32 ? 4 : 2;
  int nt = 0;
  for (int i = n - 1; i >= 0 && cols > 0; --i) {
    const int64_t tiles_n = (as[i].rows + 255) / 256;
    const int64_t take = cols < tiles_n ? cols : tiles_n;
    cols -= take;
    const int64_t rows1 = (tiles_n - take) * 256;
    StreamArgs t = as[i];
    t.W = as[i].W + rows1 * as[i].K * (fp8 ? 1 : 2);
    t.rows = as[i].rows - rows1;
    t.scale = as[i].scale ? as[i].scale + rows1 : nullptr;
    t.Y = static_cast<uint8_t*>(as[i].Y) + rows1 * y_elem;
    tail.g[nt++] = t;
    tg.g[i].rows = rows1;
  }
  tg.first[0] = 0;
  for (int i = 0; i < n; ++i) tg.first[i + 1] = tg.first[i] + (tg.g[i].rows > 0 ? tile_count(tg.g[i], 256) : 0);
  tail.n = nt;
  tail.first[0] = 0;
  for (int i = 0; i < nt; ++i) tail.first[i + 1] = tail.first[i] + tile_count(tail.g[i], 128);
  hipError_t e = fp8 ? launch_group<256, 8, true>(tg, stream) : launch_group<256, 8, false>(tg, stream);
  if (e != hipSuccess) return e;
  return fp8 ? launch_group<128, 4, true>(tail, stream) : launch_group<128, 4, false>(tail, stream);
}

// Where 128-token x 256-row tiles were chosen because 256 x 256 tiles fill
// less than two waves of workgroups, and the last wave of 256 x 256 tiles is
// at most half full: the weight rows whose 256 x 256 tiles make whole waves
// (the first columns of tiles).  The other columns then run as 128-token
// tiles, at most one more wave.  0 where this does not apply.
static int64_t whole_wave_rows(const StreamArgs& p) {
  if (p.mode == OUT_SILU_BF16) return 0;
  const int64_t tiles_m = (p.M + kTileM - 1) / kTileM;
  const int64_t tiles_n = (p.rows + 255) / 256;
  const int64_t rem = (tiles_m * tiles_n) % 256;
  if (tiles_m * tiles_n <= 256 || rem == 0 || rem > 128 || rem % tiles_m != 0) return 0;
  return (tiles_n - rem / tiles_m) * 256;
}

// p restricted to weight rows r0 ..: the weights, scales and output columns
// from row r0 on
static StreamArgs rows_from(const StreamArgs& p, int64_t r0, int64_t w_elem, int64_t y_elem) {
  StreamArgs q = p;
  q.W = p.W + r0 * p.K * w_elem;
  q.rows = p.rows - r0;
  q.scale = p.scale ? p.scale + r0 : nullptr;
  q.Y = static_cast<uint8_t*>(p.Y) + r0 * y_elem;
  return q;
}

hipError_t launch_tile_gemm(const StreamArgs& a, int bn, bool fp8, hipStream_t stream) {
  // The kernels address X through 32-bit buffer offsets: tokens go in parts
  // whose X spans less than 2 GiB (whole 256-token tiles).
  const bool f8x = a.xscale != nullptr;  // FP8 activations (FP8 weights too)
  const int64_t x_row = a.ldx * (f8x ? 1 : 2);
  int64_t part = ((INT64_C(1) << 31) - 1) / x_row / kTileM * kTileM;
  if (part < kTileM) return hipErrorInvalidValue;  // a 256-token tile alone would exceed 2 GiB
  const int64_t y_elem = a.mode == OUT_F32 ? 4 : 2;
  for (int64_t m0 = 0; m0 < a.M; m0 += part) {
    StreamArgs p = a;
    p.M = a.M - m0 < part ? a.M - m0 : part;
    p.X = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(a.X) + m0 * x_row);
    p.Y = static_cast<uint8_t*>(a.Y) + m0 * a.ldy * y_elem;
    if (f8x) {
      p.xscale = a.xscale + m0;
      hipError_t e;
      if (p.K % 128 == 0) {
        // 128-K double steps: whole 128-byte lines per load
        if (bn == 256)
          hipLaunchKernelGGL((tile_gemm_f8f8d_kernel<256, 8, 2>), tile_grid<256>(p), dim3(512), 0, stream, p);
        else if (tile_count(p, 256, 128) >= 512) {
          // 128 tokens x 256 weight rows, eight waves (as for FP8 weights),
          // after whole waves of 256 x 256 tiles where they fit
          const int64_t rows1 = whole_wave_rows(p);
          StreamArgs p2 = p;
          if (rows1 > 0) {
            StreamArgs p1 = p;
            p1.rows = rows1;
            hipLaunchKernelGGL((tile_gemm_f8f8d_kernel<256, 8, 2>), tile_grid<256>(p1), dim3(512), 0, stream, p1);
            p2 = rows_from(p, rows1, 1, y_elem);
          }
          if (hipPeekAtLastError() == hipSuccess)
            hipLaunchKernelGGL((tile_gemm_f8f8d_kernel<256, 8, 3, 128>), (tile_grid<256, 128>(p2)), dim3(512), 0,
                               stream, p2);
        } else
          hipLaunchKernelGGL((tile_gemm_f8f8d_kernel<128, 4, 3>), tile_grid<128>(p), dim3(256), 0, stream, p);
        e = hipGetLastError();
      } else {
        e = bn == 256 ? launch_f8f8_ring<256, 8>(p, stream) : launch_f8f8_ring<128, 4>(p, stream);
      }
      if (e != hipSuccess) return e;
      continue;
    }
    // 256-row tiles: 8 waves (two per SIMD, 128 x 64 each), so one wave's
    // waits on LDS and barriers are covered by the other's MFMAs
    hipError_t e;
    if (bn == 256) {
      // Whole waves of 256-row tiles over the 256 CUs.  Where the last wave
      // would be at most half full, its rows go to 128-row tiles in a second
      // launch instead (2048 x 8192 x 28672 BF16: 896 tiles, 3.5 waves; as
      // 768 + 256 half tiles 1137-1149 against 1095 TFLOP/s).
      int64_t rows1 = p.rows;
      if (p.mode != OUT_SILU_BF16) {
        const int64_t tiles_m = (p.M + kTileM - 1) / kTileM;
        const int64_t tiles_n = (p.rows + 255) / 256;
        const int64_t rem = (tiles_m * tiles_n) % 256;
        if (tiles_m * tiles_n > 256 && rem != 0 && rem <= 128) {
          int64_t n1 = tiles_n;
          while (n1 > 0 && (tiles_m * n1) % 256 != 0) --n1;
          if (n1 > 0) rows1 = n1 * 256;
        }
      }
      StreamArgs p1 = p;
      p1.rows = rows1;
      e = fp8 ? launch_fp8<256, 8>(p1, stream) : launch_bf16d<256, 8, 2>(p1, stream);
      if (e == hipSuccess && rows1 < p.rows) {
        const StreamArgs p2 = rows_from(p, rows1, fp8 ? 1 : 2, y_elem);
        e = fp8 ? launch_fp8<128, 4>(p2, stream) : launch_bf16d<128, 4, 3>(p2, stream);
      }
    } else if (fp8 && tile_count(p, 256, 128) >= 512) {
      // 128 tokens x 256 weight rows, eight waves of 64 x 64: per FLOP 20%
      // fewer bytes loaded into LDS than 256 x 128 (the BF16 X, twice the
      // bytes of the FP8 W, is the shorter side), and two waves per SIMD
      // (measured on the 4096-token down GEMM: 1065 against 1000 TFLOP/s).
      // Whole waves of 256 x 256 tiles first where they fit.
      const int64_t rows1 = whole_wave_rows(p);
      StreamArgs p2 = p;
      e = hipSuccess;
      if (rows1 > 0) {
        StreamArgs p1 = p;
        p1.rows = rows1;
        e = launch_fp8<256, 8>(p1, stream);
        p2 = rows_from(p, rows1, 1, y_elem);
      }
      if (e == hipSuccess) {
        if (p2.mode == OUT_F32)
          hipLaunchKernelGGL((tile_gemm_fp8_kernel<256, 8, 128, true>), (tile_grid<256, 128>(p2)), dim3(512), 0, stream,
                             p2);
        else
          hipLaunchKernelGGL((tile_gemm_fp8_kernel<256, 8, 128>), (tile_grid<256, 128>(p2)), dim3(512), 0, stream, p2);
        e = hipGetLastError();
      }
    } else
      e = fp8 ? launch_fp8<128, 4>(p, stream) : launch_bf16d<128, 4, 3>(p, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace swr
