// Device-side pieces shared by the GEMM kernels (streaming and tiled).
#pragma once

#include "swr_internal.h"

namespace swr {

// Arguments of every GEMM kernel (plain pointers and sizes).
struct StreamArgs {
  const uint8_t* W;
  const float* scale;
  const uint16_t* X;
  int64_t ldx;
  int64_t M;
  int64_t rows;
  int64_t K;
  int64_t kper;   // K per workgroup split
  int64_t inter;  // I in SILU mode
  int64_t rb;     // output rows per row block (gate rows in SILU mode), a multiple of 4
  void* Y;
  int64_t ldy;
  float* partial;  // [ksplit][M][rows] when ksplit > 1
  const float* xscale;  // tiled kernels, FP8 activations: one scale per token (X holds E4M3FN codes)
  int mode;
  int ksplit;
};

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kStepK = 64;    // K elements per wave step (stream kernel)
constexpr int kStageK = 256;  // K elements per stage (staged kernel)
constexpr int kTileK = 64;    // K elements per tile (tiled prefill kernel)


__device__ inline bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0];
  r[1] = a[1];
  r[2] = b[0];
  r[3] = b[1];
  r[4] = c[0];
  r[5] = c[1];
  r[6] = d[0];
  r[7] = d[1];
  return r;
}

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw buffer resource (base, no stride, num_records bytes) in scalar registers.
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
__device__ inline u32x4s raw_rsrc(const void* base, int64_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  // the same in every lane: kept in scalar registers (the loads take it there)
  u32x4s r;
  r[0] = __builtin_amdgcn_readfirstlane(uint32_t(p));
  r[1] = __builtin_amdgcn_readfirstlane(uint32_t(p >> 32) & 0xFFFFu);  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(uint32_t(bytes));
  r[3] = 0x00020000u;
  return r;
}

// One 16-byte buffer-to-LDS load per lane: lane l's bytes land at lds + 16*l
// (the wave-uniform base goes in M0).  Written as assembly so that the
// compiler adds no waits of its own for it: this kernel orders these loads
// itself (wait_vm before each barrier).  NT selects the streaming hint.  The
// LDS base is an M0 operand of the statement ("{m0}"), so the compiler itself
// writes M0 before it and knows what M0 holds.
template <bool NT>
__device__ inline void lds_load16(const u32x4s& res, uint8_t* lds, int voffset, int soffset) {
  // the base is the same in every lane of the wave
  const uint32_t base = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>((lds_ptr_t)lds)));
  if constexpr (NT)
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds"
                 :
                 : "v"(voffset), "s"(res), "s"(soffset), "{m0}"(base)
                 : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voffset), "s"(res), "s"(soffset), "{m0}"(base)
                 : "memory");
}

template <int N>
__device__ inline void wait_vm() {
  // s_waitcnt with vmcnt = N and the other counters at their maximum
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int N>
__device__ inline void wait_vm_lds() {
  // s_waitcnt with vmcnt = N, lgkmcnt = 0 (every LDS access of the wave done)
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}


__device__ inline float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ inline uint16_t bf16_bits(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }

}  // namespace

// Tiled MFMA GEMM for prefill-sized M (gemm_tile.hip).  bn is 256 or 128.
hipError_t launch_tile_gemm(const StreamArgs& a, int bn, bool fp8, hipStream_t stream);

// n tiled GEMMs of one weight dtype (BF16 activations, no SiLU mode, each
// X under 2 GiB) in one launch of the bn-row tile kernel.
struct TileGroup {
  StreamArgs g[kMaxGroup];
  int64_t first[kMaxGroup + 1];  // first tile of each problem; first[n] tiles in all
  int n;
};
hipError_t launch_tile_group(const StreamArgs* as, int n, int bn, bool fp8, hipStream_t stream);

}  // namespace swr
