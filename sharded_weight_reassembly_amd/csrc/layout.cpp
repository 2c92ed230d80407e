// Flat layout planning (host only) and the library's error reporting.
//
// weight_sharding (zdszero.github.io), section "one AllGather per layer: flat
// layout", steps 1-2: items laid end to end in order, each on a 16-byte
// boundary, the total padded to a multiple of 16*N, and N equal chunks.
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "swr_internal.h"

namespace swr {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

int hip_fail(hipError_t e, const char* what) {
  return fail(SWR_E_HIP, "%s: %s (%d)", what, hipGetErrorString(e), static_cast<int>(e));
}

}  // namespace swr

extern "C" const char* swr_last_error(void) { return swr::g_last_error.c_str(); }

extern "C" const char* swr_version(void) { return "swr 0.1 gfx950"; }

static int64_t elem_bytes(int32_t dtype) {
  switch (dtype) {
    case SWR_BF16:
      return 2;
    case SWR_FP8_E4M3FN:
      return 1;
    default:
      return 0;
  }
}

extern "C" int swr_plan_layer(const swr_weight_desc* w, int32_t n_weights, int32_t n_chunks,
                              swr_view_desc* views_out, swr_layout* layout_out) {
  using swr::fail;
  if (!w || !views_out || !layout_out) return fail(SWR_E_INVALID, "swr_plan_layer: null pointer");
  if (n_weights < 1 || n_weights > SWR_MAX_WEIGHTS)
    return fail(SWR_E_INVALID, "swr_plan_layer: n_weights=%d outside [1, %d]", n_weights, SWR_MAX_WEIGHTS);
  if (n_chunks < 1 || n_chunks > SWR_MAX_CHUNKS)
    return fail(SWR_E_INVALID, "swr_plan_layer: n_chunks=%d outside [1, %d]", n_chunks, SWR_MAX_CHUNKS);
  const int64_t kLimit = INT64_C(1) << 52;  // keeps every sum below exact-int64 overflow
  int64_t end = 0;
  for (int j = 0; j < n_weights; ++j) {
    const int64_t eb = elem_bytes(w[j].dtype);
    if (eb == 0) return fail(SWR_E_INVALID, "swr_plan_layer: weight %d has unknown dtype %d", j, w[j].dtype);
    if (w[j].reserved != 0) return fail(SWR_E_INVALID, "swr_plan_layer: weight %d reserved field not 0", j);
    if (w[j].out_features < 1 || w[j].in_features < 1)
      return fail(SWR_E_SHAPE, "swr_plan_layer: weight %d has shape [%lld x %lld]", j,
                  (long long)w[j].out_features, (long long)w[j].in_features);
    if (w[j].out_features > kLimit / w[j].in_features || w[j].out_features * w[j].in_features > kLimit / eb)
      return fail(SWR_E_SHAPE, "swr_plan_layer: weight %d is too large", j);
    const int64_t start = (end + SWR_ITEM_ALIGN - 1) / SWR_ITEM_ALIGN * SWR_ITEM_ALIGN;
    const int64_t size = w[j].out_features * w[j].in_features * eb;
    if (start > kLimit - size) return fail(SWR_E_SHAPE, "swr_plan_layer: layer is too large");
    views_out[j].offset = start;
    views_out[j].nbytes = size;
    views_out[j].out_features = w[j].out_features;
    views_out[j].in_features = w[j].in_features;
    views_out[j].dtype = w[j].dtype;
    views_out[j].reserved = 0;
    end = start + size;
  }
  const int64_t unit = int64_t(SWR_ITEM_ALIGN) * n_chunks;
  const int64_t total = (end + unit - 1) / unit * unit;
  layout_out->payload_bytes = end;
  layout_out->total_bytes = total;
  layout_out->chunk_bytes = total / n_chunks;
  layout_out->n_weights = n_weights;
  layout_out->n_chunks = n_chunks;
  swr::clear_error();
  return SWR_OK;
}
