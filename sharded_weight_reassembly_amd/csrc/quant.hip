// Per-token E4M3FN quantisation of BF16 activations on gfx950 (the FP8-
// activation option of the prefill GEMMs; the pages keep activations in BF16).
//
//   s[m]    = amax_k |x[m, k]| / 448          (binary32; 1 for an all-zero row)
//   q[m, k] = E4M3FN(x[m, k] / s[m])          (binary32 quotient, round to
//                                              nearest, ties to even, magnitudes
//                                              above 448 saturate to 448)
//
// One workgroup per row: a first pass over the row finds the largest
// magnitude (wave shuffles, then LDS across the waves), a second pass reads
// the row again (from L2) and writes 8 codes per 16 bytes of BF16.  The
// division is the compiler's correctly rounded binary32 division, so the
// codes are a function of the row alone.
#include "swr_internal.h"

namespace swr {
namespace {

constexpr int kQThreads = 256;

__device__ inline float bf16_value(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// E4M3FN code of a binary32 value: nearest finite value, ties to the even
// code, saturating at 448.  Below 2^-6 the step is 2^-9 (subnormals; the
// value 2^-6 itself is code 8, the first normal); from 2^e (e >= -6) the step
// is 2^(e-3), and a mantissa that rounds up to 16 carries into the exponent.
__device__ inline uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 31) << 7;
  const float a = fminf(fabsf(y), 448.0f);
  uint32_t c;
  if (a < 0.015625f) {
    c = uint32_t(rintf(a * 512.0f));
  } else {
    const int e = ilogbf(a);
    c = uint32_t((e + 7) << 3) + uint32_t(rintf(ldexpf(a, 3 - e))) - 8u;
  }
  return c | sign;
}

__global__ __launch_bounds__(kQThreads) void quantize_rows_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                                  int64_t K, uint8_t* __restrict__ Q, int64_t ldq,
                                                                  float* __restrict__ S) {
  const int64_t m = blockIdx.x;
  const uint16_t* x = X + m * ldx;
  uint8_t* q = Q + m * ldq;
  const int64_t nv = K / 8;  // whole 16-byte pieces; the rest is a short tail

  float amax = 0.f;
  for (int64_t i = threadIdx.x; i < nv; i += kQThreads) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(x + i * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(bf16_value(v[j] & 0xFFFFu)));
      amax = fmaxf(amax, fabsf(bf16_value(v[j] >> 16)));
    }
  }
  for (int64_t k = nv * 8 + threadIdx.x; k < K; k += kQThreads) amax = fmaxf(amax, fabsf(bf16_value(x[k])));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  __shared__ float wave_max[kQThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  float a = wave_max[0];
#pragma unroll
  for (int w = 1; w < kQThreads / 64; ++w) a = fmaxf(a, wave_max[w]);
  const float s = a > 0.f ? a / 448.0f : 1.0f;
  if (threadIdx.x == 0) S[m] = s;

  for (int64_t i = threadIdx.x; i < nv; i += kQThreads) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(x + i * 8);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = e4m3_code(bf16_value(v[j] & 0xFFFFu) / s);
      const uint32_t hi = e4m3_code(bf16_value(v[j] >> 16) / s);
      w[j / 2] |= (lo | (hi << 8)) << (16 * (j % 2));
    }
    *reinterpret_cast<uint2*>(q + i * 8) = make_uint2(w[0], w[1]);
  }
  for (int64_t k = nv * 8 + threadIdx.x; k < K; k += kQThreads) q[k] = uint8_t(e4m3_code(bf16_value(x[k]) / s));
}

}  // namespace

hipError_t launch_quantize_rows(const void* X, int64_t ldx, int64_t M, int64_t K, void* Q, int64_t ldq, float* S,
                                hipStream_t stream) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3(unsigned(M)), dim3(kQThreads), 0, stream,
                     static_cast<const uint16_t*>(X), ldx, K, static_cast<uint8_t*>(Q), ldq, S);
  return hipGetLastError();
}

}  // namespace swr

using swr::aligned;
using swr::fail;

extern "C" int swr_quantize_rows_e4m3(const void* X, int64_t ldx, int64_t M, int64_t K, void* Q, int64_t ldq,
                                      float* S, hipStream_t stream) {
  const char* fn = "swr_quantize_rows_e4m3";
  if (!X || !Q || !S) return fail(SWR_E_INVALID, "%s: null pointer", fn);
  if (M < 0 || K < 1 || M > (INT64_C(1) << 31) - 1 || ldx < K || ldq < K)
    return fail(SWR_E_SHAPE, "%s: M=%lld K=%lld ldx=%lld ldq=%lld", fn, (long long)M, (long long)K, (long long)ldx,
                (long long)ldq);
  if (!aligned(X, 16) || ldx % 8 != 0 || !aligned(Q, 8) || ldq % 8 != 0 || !aligned(S, 4))
    return fail(SWR_E_ALIGN, "%s: X rows must be 16-byte aligned, Q rows 8-byte aligned", fn);
  const hipError_t e = swr::launch_quantize_rows(X, ldx, M, K, Q, ldq, S, stream);
  if (e != hipSuccess) return swr::hip_fail(e, "quantize rows: launch");
  swr::clear_error();
  return SWR_OK;
}
