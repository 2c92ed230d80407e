// Tiled MFMA GEMM for prefill-sized token counts on gfx950.
//
//   Y[m, o] = s[o] * sum_k X[m, k] * W[o, k]      (or the fused SiLU*up mode)
//
// At thousands of tokens the weights are reused by every token block and the
// product is bound by the matrix cores, so this is a classic LDS-tiled GEMM:
//   * a workgroup (4 waves, 2 x 2) computes a 256-token x BN-row tile of Y;
//     each wave a 128 x BN/2 sub-tile with v_mfma_f32_32x32x16_bf16 (tokens are
//     the MFMA rows, weight rows the MFMA columns, so a lane's outputs run
//     along a row of Y);
//   * each 64-K step of X (bf16) and W is staged in LDS, double buffered, the
//     next step's global loads in registers while the current one is
//     multiplied; FP8 weight codes are widened to BF16 once, on the way into
//     LDS (exact);
//   * LDS rows are 128 B of 16-byte pieces; piece p of row r is stored at
//     r * 8 + (p ^ ((r >> 1) & 7)), so the 32-row fragment reads of one MFMA
//     hit distinct banks;
//   * tiles are numbered so that each XCD (workgroups are dealt round-robin
//     to the 8 XCDs) works through a compact group of 4 token blocks x all
//     weight blocks, which keeps the X and W tiles of concurrently running
//     workgroups in that XCD's L2;
//   * in SiLU mode a workgroup owns gate rows J0..J0+BN/2 and the matching up
//     rows, laid out so that gate j and up j land in the same lane of
//     different MFMA tiles; the epilogue writes h = bf16(silu(g) * u).
#include "gemm_common.h"

namespace swr {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTileM = 256;
constexpr int kGroupM = 4;  // token blocks per XCD group

__device__ inline int swz(int row, int piece) { return row * 8 + (piece ^ ((row >> 1) & 7)); }

template <int BN, bool FP8, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 1) void tile_gemm_kernel(StreamArgs a) {
  constexpr int NT = 64 * WAVES;    // threads
  constexpr int WGN = WAVES / 2;    // waves along the weight rows (2 along the tokens)
  constexpr int WN = BN / WGN;      // weight rows per wave
  constexpr int TM = 4;             // 32-token MFMA tiles per wave (128 tokens)
  constexpr int TN = WN / 32;       // 32-row MFMA tiles per wave
  constexpr int A_BYTES = kTileM * kTileK * 2;
  constexpr int B_BYTES = BN * kTileK * 2;
  constexpr int NA = A_BYTES / 16 / NT;             // X pieces per thread per step
  constexpr int NB = FP8 ? BN * kTileK / 16 / NT     // fp8 pieces (16 codes) per thread
                         : B_BYTES / 16 / NT;        // bf16 pieces per thread
  static_assert(TN >= 1 && NA >= 1 && NB >= 1, "tile must split evenly over the workgroup");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (A_BYTES + B_BYTES)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const bool silu_mode = a.mode == OUT_SILU_BF16;

  // ---- tile numbering: XCD-contiguous ranges, grouped by token blocks
  const int64_t tiles_m = (a.M + kTileM - 1) / kTileM;
  const int64_t cols = silu_mode ? a.inter : a.rows;  // output columns
  const int64_t col_tile = silu_mode ? BN / 2 : BN;
  const int64_t tiles_n = (cols + col_tile - 1) / col_tile;
  const int64_t ntiles = int64_t(gridDim.x);
  const int64_t i = blockIdx.x;
  const int64_t t = (ntiles % 8 == 0) ? (i % 8) * (ntiles / 8) + i / 8 : i;
  const int64_t group = t / (kGroupM * tiles_n);
  const int64_t first_m = group * kGroupM;
  const int64_t gsize = min<int64_t>(tiles_m - first_m, kGroupM);
  const int64_t tile_m = first_m + (t % (kGroupM * tiles_n)) % gsize;
  const int64_t tile_n = (t % (kGroupM * tiles_n)) / gsize;

  // weight row held by local B row c (0 <= c < BN)
  auto w_row = [&](int c) -> int64_t {
    if (silu_mode) {
      const int half = c / WN;       // which wave column
      const int c2 = c % WN;         // within the wave: first half gate, second half up
      const int64_t j = tile_n * (BN / 2) + half * (WN / 2) + (c2 % (WN / 2));
      return c2 < WN / 2 ? j : a.inter + j;
    }
    return tile_n * BN + c;
  };

  // ---- global -> register staging addresses
  const int64_t m0 = tile_m * kTileM;
  const uint16_t* asrc[NA];
  int adst[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int v = j * NT + tid;
    const int row = v / 8, piece = v % 8;
    const int64_t m = min(m0 + row, a.M - 1);
    asrc[j] = a.X + m * a.ldx + piece * 8;
    adst[j] = swz(row, piece) * 16;
  }
  const uint8_t* bsrc[NB];
  int bdst[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int v = j * NT + tid;
    if (FP8) {
      const int row = v / 4, q = v % 4;  // 16 codes = bf16 pieces 2q, 2q+1
      int64_t r = w_row(row);
      r = min(r, a.rows - 1);
      bsrc[j] = a.W + r * a.K + q * 16;
      bdst[j] = swz(row, 2 * q) * 16;  // piece 2q+1 goes to swz(row, 2q+1)
    } else {
      const int row = v / 8, piece = v % 8;
      int64_t r = w_row(row);
      r = min(r, a.rows - 1);
      bsrc[j] = a.W + (r * a.K + piece * 8) * 2;
      bdst[j] = swz(row, piece) * 16;
    }
  }

  u32x4 ra[NA], rb[NB];
  auto load = [&](int kt) {
    const int64_t k0 = int64_t(kt) * kTileK;
#pragma unroll
    for (int j = 0; j < NA; ++j) ra[j] = *reinterpret_cast<const u32x4*>(asrc[j] + k0);
#pragma unroll
    for (int j = 0; j < NB; ++j) rb[j] = *reinterpret_cast<const u32x4*>(bsrc[j] + k0 * (FP8 ? 1 : 2));
  };
  auto store = [&](int buf) {
    uint8_t* A = lds + buf * (A_BYTES + B_BYTES);
    uint8_t* B = A + A_BYTES;
#pragma unroll
    for (int j = 0; j < NA; ++j) *reinterpret_cast<u32x4*>(A + adst[j]) = ra[j];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (FP8) {
        const int v = j * NT + tid;
        const int row = v / 4, q = v % 4;
        *reinterpret_cast<bf16x8*>(B + bdst[j]) = fp8x8_to_bf16(rb[j][0], rb[j][1]);
        *reinterpret_cast<bf16x8*>(B + swz(row, 2 * q + 1) * 16) = fp8x8_to_bf16(rb[j][2], rb[j][3]);
      } else {
        *reinterpret_cast<u32x4*>(B + bdst[j]) = rb[j];
      }
    }
  };

  // ---- fragment reads: k-step ks of buffer buf into F (A rows then B rows)
  const int r32 = lane & 31, kg = lane >> 5;
  f32x16 acc[TM][TN];
#pragma unroll
  for (int x = 0; x < TM; ++x)
#pragma unroll
    for (int y = 0; y < TN; ++y) acc[x][y] = f32x16{};

  bf16x8 F[2][TM + TN];  // two k-steps of fragments: the next one is read while the current one multiplies
  auto read_frags = [&](int buf, int ks, bf16x8(&f)[TM + TN]) {
    const uint8_t* A = lds + buf * (A_BYTES + B_BYTES);
    const uint8_t* B = A + A_BYTES;
    const int piece = ks * 2 + kg;
#pragma unroll
    for (int x = 0; x < TM; ++x) f[x] = *reinterpret_cast<const bf16x8*>(A + swz(wm * 128 + x * 32 + r32, piece) * 16);
#pragma unroll
    for (int y = 0; y < TN; ++y)
      f[TM + y] = *reinterpret_cast<const bf16x8*>(B + swz(wn * WN + y * 32 + r32, piece) * 16);
  };
  auto mfmas = [&](const bf16x8(&f)[TM + TN]) {
#pragma unroll
    for (int x = 0; x < TM; ++x)
#pragma unroll
      for (int y = 0; y < TN; ++y) acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[x], f[TM + y], acc[x][y], 0, 0, 0);
  };

  const int nk = int(a.K / kTileK);
  load(0);
  store(0);
  __syncthreads();
  read_frags(0, 0, F[0]);
  // Each k-step is a scheduling region of its own: the next k-step's LDS
  // fragment reads (into the other register set) interleave with this
  // k-step's MFMAs, and their wait lands at the start of the next region.
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    const int buf = kt & 1;
    if (more) load(kt + 1);  // global loads, in flight during the MFMAs below
#pragma unroll
    for (int ks = 0; ks < kTileK / 16; ++ks) {
      if (ks + 1 < kTileK / 16) read_frags(buf, ks + 1, F[(ks + 1) & 1]);
      mfmas(F[ks & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) store(buf ^ 1);  // the other buffer was last read before the previous barrier
    __syncthreads();
    if (more) read_frags(buf ^ 1, 0, F[0]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue: lane holds column c = l % 32 of each 32 x 32 tile, rows 8*(v/4) + 4*(l/32) + v%4
  const int tn_out = silu_mode ? TN / 2 : TN;
#pragma unroll
  for (int y = 0; y < tn_out; ++y) {
    const int c = wn * WN + y * 32 + r32;  // local B row
    const int64_t orow = w_row(c);
    int64_t ocol;  // output column
    float sc = 1.f, su = 1.f;
    bool col_ok;
    if (silu_mode) {
      ocol = orow;  // gate index j
      col_ok = ocol < a.inter;
      if (col_ok && a.scale) {
        sc = a.scale[ocol];
        su = a.scale[a.inter + ocol];
      }
    } else {
      ocol = orow;
      col_ok = ocol < a.rows;
      if (col_ok && a.scale) sc = a.scale[ocol];
    }
    if (!col_ok) continue;
#pragma unroll
    for (int x = 0; x < TM; ++x) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * 128 + x * 32 + 8 * (v / 4) + 4 * kg + (v % 4);
        if (m >= a.M) continue;
        float out = acc[x][y][v] * sc;
        if (silu_mode) {
          const float u = acc[x][y + TN / 2][v] * su;
          out = silu(out) * u;
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

template <int BN, bool FP8, int WAVES>
hipError_t launch_bn(const StreamArgs& a, hipStream_t stream) {
  const bool silu_mode = a.mode == OUT_SILU_BF16;
  const int64_t tiles_m = (a.M + kTileM - 1) / kTileM;
  const int64_t cols = silu_mode ? a.inter : a.rows;
  const int64_t col_tile = silu_mode ? BN / 2 : BN;
  const int64_t tiles_n = (cols + col_tile - 1) / col_tile;
  hipLaunchKernelGGL((tile_gemm_kernel<BN, FP8, WAVES>), dim3(unsigned(tiles_m * tiles_n)), dim3(64 * WAVES), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_gemm(const StreamArgs& a, int bn, bool fp8, hipStream_t stream) {
  // 256-row tiles: 8 waves (two per SIMD, 128 x 64 each), so one wave's
  // waits on LDS and barriers are covered by the other's MFMAs
  if (bn == 256) return fp8 ? launch_bn<256, true, 8>(a, stream) : launch_bn<256, false, 8>(a, stream);
  return fp8 ? launch_bn<128, true, 4>(a, stream) : launch_bn<128, false, 4>(a, stream);
}

}  // namespace swr
