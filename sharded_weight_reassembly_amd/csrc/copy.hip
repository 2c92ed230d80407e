// Byte-moving kernels of the path: the one-time pack into flat chunks, the
// per-layer reassembly of the chunks into a workspace slot, and the fixed-order
// sum of split-contraction partials.  All three are HBM-bound streams of
// 16-byte vectors; none of them does arithmetic on weight values.
#include <algorithm>

#include "swr_internal.h"

namespace swr {
namespace {

constexpr int kThreads = 256;

// ----------------------------------------------------------------- reassembly
//
// weight_sharding, flat layout step 3: after the gather every rank holds the
// whole T, i.e. slot[i*C, (i+1)*C) = chunk_i.  Grid: (blocks per chunk, N).
// Each workgroup copies one 32 KiB span of one chunk in a single round of
// 16-byte loads (8 per thread, all in flight) and stores; many
// short-lived workgroups keep more bytes in flight per CU than long loops
// (measured on MI355X: 6.45 TB/s of read+write against 5.5 TB/s for
// 64-128 KiB spans).
//
// The slot is written for the GEMMs that read it next.  Workgroups are
// dispatched in grid order, so chunk y of the grid is chunk N-1-y of T: the
// front of the slot, where a layer's first weights sit, is written last.
// The stores carry no streaming hint, so those most recent lines are still
// in the 256 MB last-level cache when the first GEMM starts, and their
// write-back to HBM overlaps that GEMM.  Measured on the shared-expert
// decode stack (8 layers of 264 MB): 1.8-2.8% less wall time per forward at
// every token count than streaming stores in chunk order; streaming stores
// in reverse order gained nothing, cached stores in chunk order lost 1.5%
// at 64 tokens.  The chunks are read once per gather: their loads stream.
constexpr int kCopyUnroll = 8;
constexpr int64_t kCopySpanVecs = 256 * kCopyUnroll;  // 32 KiB per workgroup

__global__ __launch_bounds__(kThreads) void reassemble_kernel(ChunkPtrs chunks, u32x4* __restrict__ slot,
                                                              int64_t chunk_vecs, int64_t span_vecs) {
  const int c = int(gridDim.y) - 1 - int(blockIdx.y);
  const u32x4* __restrict__ src = static_cast<const u32x4*>(chunks.p[c]);
  u32x4* __restrict__ dst = slot + int64_t(c) * chunk_vecs;
  const int64_t step = int64_t(kThreads) * kCopyUnroll;
  // one span per workgroup when the grid covers the chunk; a smaller grid walks the spans
  for (int64_t begin = int64_t(blockIdx.x) * span_vecs; begin < chunk_vecs; begin += int64_t(gridDim.x) * span_vecs) {
    const int64_t end = min(begin + span_vecs, chunk_vecs);
    int64_t i = begin + threadIdx.x;
    // full tiles: every vector of the tile is in range
    for (; i + (kCopyUnroll - 1) * kThreads < end; i += step) {
      u32x4 v[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) dst[i + u * kThreads] = v[u];
    }
    for (; i < end; i += kThreads) dst[i] = src[i];
  }
}

// --------------------------------------------------------------------- pack
//
// weight_sharding, flat layout steps 1-2 and the loading section's one-time
// re-layout: every 16-byte vector of T is taken from the weight whose byte
// range covers it (or is zero padding) and written to chunk p / C at p % C.
// Item offsets and C are multiples of 16, so a vector never spans two items
// or two chunks; only an item's last vector can be partly padding.
__global__ __launch_bounds__(kThreads) void pack_kernel(PackPlan plan) {
  const int64_t nvec = plan.total_bytes / 16;
  for (int64_t v = int64_t(blockIdx.x) * kThreads + threadIdx.x; v < nvec;
       v += int64_t(gridDim.x) * kThreads) {
    const int64_t p = v * 16;
    // largest j with off[j] <= p (offsets are increasing)
    int lo = 0, hi = plan.n_weights - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (plan.off[mid] <= p)
        lo = mid;
      else
        hi = mid - 1;
    }
    uint4 out = make_uint4(0, 0, 0, 0);
    const int64_t rel = p - plan.off[lo];
    if (rel >= 0 && rel < plan.size[lo]) {
      const uint8_t* s = static_cast<const uint8_t*>(plan.src[lo]) + rel;
      if (rel + 16 <= plan.size[lo]) {
        out = *reinterpret_cast<const uint4*>(s);
      } else {
        uint8_t b[16];
        const int64_t n = plan.size[lo] - rel;
#pragma unroll
        for (int t = 0; t < 16; ++t) b[t] = (t < n) ? s[t] : uint8_t(0);
        out = *reinterpret_cast<const uint4*>(b);
      }
    }
    const int64_t ci = p / plan.chunk_bytes;
    uint8_t* dst = static_cast<uint8_t*>(plan.chunk[ci]) + (p - ci * plan.chunk_bytes);
    *reinterpret_cast<uint4*>(dst) = out;
  }
}

// ----------------------------------------------------- row-shard re-layout
//
// weight_sharding, loading section: the one-time re-layout from a tensor-
// parallel loader's row shards into the flat chunks.  One launch per weight
// writes T[begin, end): the weight's bytes (each 16-byte vector gathered from
// the rank shard that holds its row) and the zero padding up to the next item.
// Rank r's shard holds, for each sub-block b of a merged weight in order, the
// rows [r*R_b/N, (r+1)*R_b/N) of that sub-block.
__device__ inline const uint8_t* shard_byte(const RedistArgs& a, int64_t rel) {
  if (a.replicated) return a.src[0] + rel;
  const int64_t row = rel / a.row_bytes;
  const int64_t cb = rel - row * a.row_bytes;
  int b = 0;
  while (b + 1 < a.n_sub && row >= a.sub_start[b + 1]) ++b;
  const int64_t per = (a.sub_start[b + 1] - a.sub_start[b]) / a.n;
  const int64_t rr = row - a.sub_start[b];
  const int64_t q = rr / per;
  return a.src[q] + (a.sub_first[b] + (rr - q * per)) * a.row_bytes + cb;
}

__global__ __launch_bounds__(kThreads) void redistribute_kernel(RedistArgs a) {
  for (int64_t p = a.begin + (int64_t(blockIdx.x) * kThreads + threadIdx.x) * 16; p < a.end;
       p += int64_t(gridDim.x) * kThreads * 16) {
    const int64_t rel = p - a.off;
    uint4 out = make_uint4(0, 0, 0, 0);
    // bytes before the item (the first launch starts at 0) and after it are padding
    if (rel >= 0 && rel < a.size) {
      const uint8_t* s0 = shard_byte(a, rel);
      const bool one_row = (rel / a.row_bytes) == ((rel + 15) / a.row_bytes);
      if (rel + 16 <= a.size && (a.replicated || one_row) && (reinterpret_cast<uintptr_t>(s0) & 15) == 0) {
        out = *reinterpret_cast<const uint4*>(s0);
      } else {
        uint8_t b[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) b[t] = rel + t < a.size ? *shard_byte(a, rel + t) : uint8_t(0);
        out = *reinterpret_cast<const uint4*>(b);
      }
    }
    const int64_t ci = p / a.chunk_bytes;
    *reinterpret_cast<uint4*>(static_cast<uint8_t*>(a.chunk[ci]) + (p - ci * a.chunk_bytes)) = out;
  }
}

// ------------------------------------------------------------- sum partials
//
// Sharded-matrices notes, local matmul case 3: split-contraction partials add
// up to the full product.  Added in fp32 in shard order 0..n-1.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const __bf16 ha = static_cast<__bf16>(a);
  const __bf16 hb = static_cast<__bf16>(b);
  return uint32_t(__builtin_bit_cast(uint16_t, ha)) | (uint32_t(__builtin_bit_cast(uint16_t, hb)) << 16);
}

// One thread per 4 consecutive outputs.  The n partial vectors are loaded in
// batches of 8 independent loads (all in flight at once) and added in shard
// order, so the sum is the same as a plain left-to-right loop.
__global__ __launch_bounds__(kThreads) void sum_partials_kernel(PartPtrs parts, int n, int64_t count,
                                                                void* __restrict__ out, int out_bf16) {
  constexpr int kBatch = 8;
  const int64_t nvec = count / 4;
  for (int64_t v = int64_t(blockIdx.x) * kThreads + threadIdx.x; v < nvec;
       v += int64_t(gridDim.x) * kThreads) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < n; j0 += kBatch) {
      f32x4 p[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        p[u] = j0 + u < n ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(parts.p[j0 + u]) + v)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (j0 + u < n) acc = (j0 + u == 0) ? p[u] : acc + p[u];
    }
    if (out_bf16) {
      uint2 o = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
      reinterpret_cast<uint2*>(out)[v] = o;
    } else {
      reinterpret_cast<f32x4*>(out)[v] = acc;
    }
  }
  // scalar tail (count % 4 elements), done by the first workgroup
  if (blockIdx.x == 0) {
    const int64_t i = nvec * 4 + threadIdx.x;
    if (i < count) {
      float acc = parts.p[0][i];
      for (int j = 1; j < n; ++j) acc += parts.p[j][i];
      if (out_bf16)
        reinterpret_cast<__bf16*>(out)[i] = static_cast<__bf16>(acc);
      else
        reinterpret_cast<float*>(out)[i] = acc;
    }
  }
}

int grid_for(int64_t work_items, int per_block_items) {
  int64_t g = (work_items + per_block_items - 1) / per_block_items;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return int(g);
}

}  // namespace

// lds_bytes: LDS each workgroup reserves and never touches (see
// swr_planner_set_gather_lds); it only limits how many share a CU.
hipError_t launch_reassemble(const ChunkPtrs& chunks, int n_chunks, int64_t chunk_bytes, void* slot,
                             unsigned lds_bytes, hipStream_t stream) {
  const int64_t chunk_vecs = chunk_bytes / 16;
  const int64_t span = kCopySpanVecs;
  int64_t blocks = (chunk_vecs + span - 1) / span;
  if (blocks < 1) blocks = 1;
  const dim3 grid = dim3(unsigned(blocks), unsigned(n_chunks));
  hipLaunchKernelGGL(reassemble_kernel, grid, dim3(kThreads), lds_bytes, stream, chunks, static_cast<u32x4*>(slot),
                     chunk_vecs, span);
  return hipGetLastError();
}

hipError_t launch_pack(const PackPlan& plan, hipStream_t stream) {
  const int grid = grid_for(plan.total_bytes / 16, kThreads * 4);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(kThreads), 0, stream, plan);
  return hipGetLastError();
}

hipError_t launch_redistribute(const RedistArgs& a, hipStream_t stream) {
  const int grid = grid_for((a.end - a.begin) / 16, kThreads * 4);
  hipLaunchKernelGGL(redistribute_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_sum_partials(const PartPtrs& parts, int n, int64_t count, void* out, bool out_bf16,
                               hipStream_t stream) {
  const int grid = grid_for(count / 4 + 1, kThreads);
  hipLaunchKernelGGL(sum_partials_kernel, dim3(grid), dim3(kThreads), 0, stream, parts, n, count, out,
                     out_bf16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace swr

// ====================================================================== C ABI

using swr::aligned;
using swr::fail;

namespace {

// A view lies inside the payload, 16-byte aligned, after the previous one
// (prev_end >= 0, 0 <= payload); no sum here can overflow.
bool view_fits(const swr_view_desc& v, int64_t prev_end, int64_t payload) {
  return v.offset % 16 == 0 && v.offset >= prev_end && v.offset <= payload && v.nbytes > 0 &&
         v.nbytes <= payload - v.offset;
}

}  // namespace

extern "C" int swr_pack_layer(const swr_layout* layout, const swr_view_desc* views,
                              const void* const* src_dev, void* const* chunk_dev, hipStream_t stream) {
  if (!layout || !views || !src_dev || !chunk_dev) return fail(SWR_E_INVALID, "swr_pack_layer: null pointer");
  const int nw = layout->n_weights, nc = layout->n_chunks;
  if (nw < 1 || nw > SWR_MAX_WEIGHTS || nc < 1 || nc > SWR_MAX_CHUNKS)
    return fail(SWR_E_INVALID, "swr_pack_layer: n_weights=%d n_chunks=%d out of range", nw, nc);
  if (layout->total_bytes <= 0 || layout->total_bytes % (16 * int64_t(nc)) != 0 ||
      layout->chunk_bytes != layout->total_bytes / nc)
    return fail(SWR_E_INVALID, "swr_pack_layer: inconsistent layout (|T|=%lld, C=%lld, N=%d)",
                (long long)layout->total_bytes, (long long)layout->chunk_bytes, nc);
  if (layout->payload_bytes < 0 || layout->payload_bytes > layout->total_bytes)
    return fail(SWR_E_INVALID, "swr_pack_layer: payload outside [0, |T|]");
  swr::PackPlan plan{};
  int64_t prev_end = 0;
  for (int j = 0; j < nw; ++j) {
    const swr_view_desc& v = views[j];
    if (!view_fits(v, prev_end, layout->payload_bytes))
      return fail(SWR_E_INVALID, "swr_pack_layer: view %d (offset %lld, %lld bytes) does not fit the layout", j,
                  (long long)v.offset, (long long)v.nbytes);
    if (!src_dev[j]) return fail(SWR_E_INVALID, "swr_pack_layer: src_dev[%d] is null", j);
    if (!aligned(src_dev[j], 16)) return fail(SWR_E_ALIGN, "swr_pack_layer: src_dev[%d] not 16-byte aligned", j);
    plan.src[j] = src_dev[j];
    plan.off[j] = v.offset;
    plan.size[j] = v.nbytes;
    prev_end = v.offset + v.nbytes;
  }
  for (int i = 0; i < nc; ++i) {
    if (!chunk_dev[i]) return fail(SWR_E_INVALID, "swr_pack_layer: chunk_dev[%d] is null", i);
    if (!aligned(chunk_dev[i], 16)) return fail(SWR_E_ALIGN, "swr_pack_layer: chunk_dev[%d] not 16-byte aligned", i);
    plan.chunk[i] = chunk_dev[i];
  }
  plan.chunk_bytes = layout->chunk_bytes;
  plan.total_bytes = layout->total_bytes;
  plan.n_weights = nw;
  plan.n_chunks = nc;
  const hipError_t e = swr::launch_pack(plan, stream);
  if (e != hipSuccess) return swr::hip_fail(e, "swr_pack_layer: launch");
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_redistribute_row_shards(const swr_layout* layout, const swr_view_desc* views,
                                           const swr_row_shards* shards, void* const* chunk_dev,
                                           hipStream_t stream) {
  const char* fn = "swr_redistribute_row_shards";
  if (!layout || !views || !shards || !chunk_dev) return fail(SWR_E_INVALID, "%s: null pointer", fn);
  const int nw = layout->n_weights, nc = layout->n_chunks;
  if (nw < 1 || nw > SWR_MAX_WEIGHTS || nc < 1 || nc > SWR_MAX_CHUNKS)
    return fail(SWR_E_INVALID, "%s: n_weights=%d n_chunks=%d out of range", fn, nw, nc);
  if (layout->total_bytes <= 0 || layout->total_bytes % (16 * int64_t(nc)) != 0 ||
      layout->chunk_bytes != layout->total_bytes / nc || layout->payload_bytes < 0 ||
      layout->payload_bytes > layout->total_bytes)
    return fail(SWR_E_INVALID, "%s: inconsistent layout", fn);
  for (int i = 0; i < nc; ++i) {
    if (!chunk_dev[i]) return fail(SWR_E_INVALID, "%s: chunk_dev[%d] is null", fn, i);
    if (!aligned(chunk_dev[i], 16)) return fail(SWR_E_ALIGN, "%s: chunk_dev[%d] not 16-byte aligned", fn, i);
  }
  // every check before the first launch
  int64_t prev_end = 0;
  for (int j = 0; j < nw; ++j) {
    const swr_view_desc& v = views[j];
    const swr_row_shards& sh = shards[j];
    const int64_t elem = v.dtype == SWR_FP8_E4M3FN ? 1 : 2;
    int64_t item = 0;
    if (!view_fits(v, prev_end, layout->payload_bytes) || v.out_features < 1 || v.in_features < 1 ||
        __builtin_mul_overflow(v.out_features, v.in_features, &item) || __builtin_mul_overflow(item, elem, &item) ||
        item != v.nbytes)
      return fail(SWR_E_INVALID, "%s: view %d does not fit the layout", fn, j);
    prev_end = v.offset + v.nbytes;
    if (sh.replicated) {
      if (!sh.src[0]) return fail(SWR_E_INVALID, "%s: weight %d: src[0] is null", fn, j);
      if (!aligned(sh.src[0], 16)) return fail(SWR_E_ALIGN, "%s: weight %d: src[0] not 16-byte aligned", fn, j);
      continue;
    }
    if (sh.n_sub < 1 || sh.n_sub > SWR_MAX_SUB)
      return fail(SWR_E_INVALID, "%s: weight %d: n_sub=%d outside [1, %d]", fn, j, sh.n_sub, SWR_MAX_SUB);
    int64_t rows = 0;
    for (int b = 0; b < sh.n_sub; ++b) {
      if (sh.sub_rows[b] < 0 || sh.sub_rows[b] % nc != 0)
        return fail(SWR_E_SHAPE, "%s: weight %d: sub-block %d has %lld rows, not a multiple of N=%d", fn, j, b,
                    (long long)sh.sub_rows[b], nc);
      rows += sh.sub_rows[b];
    }
    if (rows != v.out_features)
      return fail(SWR_E_SHAPE, "%s: weight %d: sub-blocks hold %lld rows, the weight %lld", fn, j, (long long)rows,
                  (long long)v.out_features);
    for (int r = 0; r < nc; ++r) {
      if (!sh.src[r]) return fail(SWR_E_INVALID, "%s: weight %d: src[%d] is null", fn, j, r);
      if (!aligned(sh.src[r], 16)) return fail(SWR_E_ALIGN, "%s: weight %d: src[%d] not 16-byte aligned", fn, j, r);
    }
  }
  // launch j writes T[begin, end): from the item's offset (0 for the first
  // item, so that any bytes before it are written as zero padding, as
  // swr_pack_layer does) to the next item's offset or |T|
  for (int j = 0; j < nw; ++j) {
    const swr_view_desc& v = views[j];
    const swr_row_shards& sh = shards[j];
    swr::RedistArgs a{};
    a.begin = j == 0 ? 0 : v.offset;
    a.end = j + 1 < nw ? views[j + 1].offset : layout->total_bytes;
    a.off = v.offset;
    a.size = v.nbytes;
    a.row_bytes = v.nbytes / v.out_features;
    a.chunk_bytes = layout->chunk_bytes;
    a.n = nc;
    a.replicated = sh.replicated ? 1 : 0;
    a.n_sub = sh.replicated ? 1 : sh.n_sub;
    int64_t start = 0, first = 0;
    for (int b = 0; b < a.n_sub; ++b) {
      a.sub_start[b] = start;
      a.sub_first[b] = first;
      const int64_t rb = sh.replicated ? v.out_features : sh.sub_rows[b];
      start += rb;
      first += rb / nc;
    }
    a.sub_start[a.n_sub] = start;
    for (int r = 0; r < (sh.replicated ? 1 : nc); ++r) a.src[r] = static_cast<const uint8_t*>(sh.src[r]);
    for (int i = 0; i < nc; ++i) a.chunk[i] = chunk_dev[i];
    const hipError_t e = swr::launch_redistribute(a, stream);
    if (e != hipSuccess) return swr::hip_fail(e, "swr_redistribute_row_shards: launch");
  }
  swr::clear_error();
  return SWR_OK;
}

namespace {

// Shared by both gather entry points: every argument is checked before the
// gate wait, the copy and the ready record are enqueued on `side`.
int reassemble(const char* fn, const void* const* chunk_dev, int32_t n_chunks, int64_t chunk_bytes, void* slot,
               int64_t slot_bytes, int32_t self_rank, hipStream_t side, hipEvent_t gate, hipEvent_t ready,
               int64_t* remote_bytes, bool dma, unsigned lds_bytes) {
  if (!chunk_dev || !slot) return fail(SWR_E_INVALID, "%s: null pointer", fn);
  if (n_chunks < 1 || n_chunks > SWR_MAX_CHUNKS)
    return fail(SWR_E_INVALID, "%s: n_chunks=%d outside [1, %d]", fn, n_chunks, SWR_MAX_CHUNKS);
  if (chunk_bytes <= 0 || chunk_bytes % 16 != 0)
    return fail(SWR_E_ALIGN, "%s: chunk_bytes=%lld is not a positive multiple of 16", fn, (long long)chunk_bytes);
  if (self_rank < 0 || self_rank >= n_chunks)
    return fail(SWR_E_INVALID, "%s: self_rank=%d outside [0, %d)", fn, self_rank, n_chunks);
  // (divided, not multiplied: no overflow for any chunk_bytes)
  if (chunk_bytes > slot_bytes / n_chunks)
    return fail(SWR_E_CAPACITY, "%s: slot holds %lld bytes, layer needs %d chunks of %lld", fn,
                (long long)slot_bytes, n_chunks, (long long)chunk_bytes);
  if (!aligned(slot, 16)) return fail(SWR_E_ALIGN, "%s: slot not 16-byte aligned", fn);
  swr::ChunkPtrs ptrs{};
  for (int i = 0; i < n_chunks; ++i) {
    if (!chunk_dev[i]) return fail(SWR_E_INVALID, "%s: chunk_dev[%d] is null", fn, i);
    if (!aligned(chunk_dev[i], 16)) return fail(SWR_E_ALIGN, "%s: chunk_dev[%d] not 16-byte aligned", fn, i);
    ptrs.p[i] = chunk_dev[i];
  }
  hipError_t e;
  if (gate) {
    e = hipStreamWaitEvent(side, gate, 0);
    if (e != hipSuccess) return swr::hip_fail(e, "reassembly: wait gate");
  }
  if (dma) {
    // the DMA engines, no compute units: one device-to-device copy per chunk
    for (int i = 0; i < n_chunks; ++i) {
      e = hipMemcpyAsync(static_cast<uint8_t*>(slot) + int64_t(i) * chunk_bytes, chunk_dev[i], size_t(chunk_bytes),
                         hipMemcpyDeviceToDeviceNoCU, side);
      if (e != hipSuccess) return swr::hip_fail(e, "reassembly: DMA copy");
    }
  } else {
    e = swr::launch_reassemble(ptrs, n_chunks, chunk_bytes, slot, lds_bytes, side);
    if (e != hipSuccess) return swr::hip_fail(e, "reassembly: launch");
  }
  if (ready) {
    e = hipEventRecord(ready, side);
    if (e != hipSuccess) return swr::hip_fail(e, "reassembly: record ready");
  }
  if (remote_bytes) *remote_bytes += int64_t(n_chunks - 1) * chunk_bytes;
  swr::clear_error();
  return SWR_OK;
}

}  // namespace

extern "C" int swr_reassemble_into_slot(const void* const* chunk_dev, int32_t n_chunks, int64_t chunk_bytes,
                                        void* slot, int64_t slot_bytes, int32_t self_rank, hipStream_t side,
                                        hipEvent_t gate, hipEvent_t ready, int64_t* remote_bytes) {
  return reassemble("swr_reassemble_into_slot", chunk_dev, n_chunks, chunk_bytes, slot, slot_bytes, self_rank, side,
                    gate, ready, remote_bytes, false, 0);
}

namespace swr {
int reassemble_reserving(const void* const* chunk_dev, int32_t n_chunks, int64_t chunk_bytes, void* slot,
                         int64_t slot_bytes, int32_t self_rank, hipStream_t side, hipEvent_t gate, hipEvent_t ready,
                         int64_t* remote_bytes, unsigned lds_bytes) {
  return reassemble("swr_reassemble_into_slot", chunk_dev, n_chunks, chunk_bytes, slot, slot_bytes, self_rank, side,
                    gate, ready, remote_bytes, false, lds_bytes);
}
}  // namespace swr

extern "C" int swr_reassemble_into_slot_dma(const void* const* chunk_dev, int32_t n_chunks, int64_t chunk_bytes,
                                            void* slot, int64_t slot_bytes, int32_t self_rank, hipStream_t side,
                                            hipEvent_t gate, hipEvent_t ready, int64_t* remote_bytes) {
  return reassemble("swr_reassemble_into_slot_dma", chunk_dev, n_chunks, chunk_bytes, slot, slot_bytes, self_rank,
                    side, gate, ready, remote_bytes, true, 0);
}

extern "C" int swr_sum_partials(const float* const* parts, int32_t n, int64_t count, void* out, int32_t out_bf16,
                                hipStream_t stream) {
  if (!parts || !out) return fail(SWR_E_INVALID, "swr_sum_partials: null pointer");
  if (n < 1 || n > SWR_MAX_CHUNKS) return fail(SWR_E_INVALID, "swr_sum_partials: n=%d outside [1, 64]", n);
  if (count < 0) return fail(SWR_E_INVALID, "swr_sum_partials: negative count");
  if (!aligned(out, 16)) return fail(SWR_E_ALIGN, "swr_sum_partials: out not 16-byte aligned");
  swr::PartPtrs ptrs{};
  for (int j = 0; j < n; ++j) {
    if (!parts[j]) return fail(SWR_E_INVALID, "swr_sum_partials: parts[%d] is null", j);
    if (!aligned(parts[j], 16)) return fail(SWR_E_ALIGN, "swr_sum_partials: parts[%d] not 16-byte aligned", j);
    ptrs.p[j] = parts[j];
  }
  if (count == 0) {
    swr::clear_error();
    return SWR_OK;
  }
  const hipError_t e = swr::launch_sum_partials(ptrs, n, count, out, out_bf16 != 0, stream);
  if (e != hipSuccess) return swr::hip_fail(e, "swr_sum_partials: launch");
  swr::clear_error();
  return SWR_OK;
}
