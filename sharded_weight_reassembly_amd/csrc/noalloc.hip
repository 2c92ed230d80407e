// swr_mlp_forward_noalloc: the shared-expert MLP of swr_mlp_forward with its
// scratch (h and any split-K partial sums) in a fixed device array of this
// library instead of a caller-provided workspace, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops).
//
// The array lives in every GPU the library runs on until the process ends.
// Its address differs per device and is not the host symbol's address: it is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and only that looked-up pointer is handed to the kernels.
// Nothing in the scratch has to start at zero: the gate_up launch writes all
// of h before the down launch reads it, and every split-K partial is written
// before the finalize kernel adds it.
#include <mutex>

#include "swr_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[SWR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// The scratch array's device address on the current device (looked up on the
// first call for that device).
int scratch_for_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return swr::hip_fail(e, "swr_mlp_forward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return swr::fail(SWR_E_INVALID, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return swr::hip_fail(e, "swr_mlp_forward_noalloc: hipGetSymbolAddress");
    if (!p || !swr::aligned(p, 256))
      return swr::fail(SWR_E_HIP, "%s: scratch address %p of device %d is not 256-byte aligned", fn, p, dev);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SWR_OK;
}

}  // namespace

extern "C" int swr_mlp_forward_noalloc(const void* W_gate_up, const float* s_gu, const void* W_down,
                                       const float* s_d, int32_t dtype, int64_t H, int64_t I, const void* X,
                                       int64_t M, void* Y, hipStream_t stream) {
  const char* fn = "swr_mlp_forward_noalloc";
  if (!W_gate_up || !W_down || !X || !Y) return swr::fail(SWR_E_INVALID, "%s: null pointer", fn);
  // sizes first: a call the fixed scratch cannot serve is refused before any
  // HIP call
  const int64_t need = swr_mlp_workspace_bytes(M, H, I, dtype);
  if (need < 0) return int(need);
  if (need > SWR_NOALLOC_SCRATCH_BYTES)
    return swr::fail(SWR_E_CAPACITY, "%s: M=%lld, H=%lld, I=%lld need %lld bytes of scratch, more than the %lld "
                     "this entry point holds; use swr_mlp_forward with a workspace",
                     fn, (long long)M, (long long)H, (long long)I, (long long)need,
                     (long long)SWR_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (int rc = scratch_for_current_device(fn, &ws)) return rc;
  return swr::mlp_impl(fn, W_gate_up, s_gu, W_down, s_d, dtype, H, I, X, M, Y, false, ws,
                       SWR_NOALLOC_SCRATCH_BYTES, stream);
}
