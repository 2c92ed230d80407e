// Lookahead / ping-pong planner (weight_sharding, zdszero.github.io):
//   * section "lookahead and ping-pong slot": the gather of layer l+1 runs on a
//     side stream while layer l computes; layer l+1 waits on the gather's
//     ready event; two slots alternate by layer, so the gather of l+1 first
//     waits for the done event of l-1, the last reader of that slot;
//   * section "implementation in SGLang": reset(), pre_dispatch(start), and
//     per layer maybe_dispatch(i+1), the layer, update_done_event(i);
//   * section "CUDA graph and the draft model": the compute stream waits at
//     most once per layer (wait_ready_once) and the sequence is fixed at init.
// A gather with no earlier layer in the forward is gated by a forward-start
// event recorded by reset() on the compute stream.
//
// Cyclic mode (the same layers run forward after forward, an even number of
// them): like the draft model's first-layer prefetch in the CUDA-graph
// section, maybe_dispatch(end) gathers the next forward's first layer into
// slot 0 -- free once done(end - 2) is recorded, since the last layer reads
// slot 1 -- so the next forward starts without an exposed gather.
//
// First layer on a dedicated stream (the CUDA-graph section's draft-model
// prefetch, outside the captured graph): the forward does not gather its
// first layer; its compute stream waits (an external wait, a node of a
// captured graph) for ready(start), which swr_planner_prefetch_first records
// on the dedicated stream after gathering layer start into slot 0; that
// gather waits for the "free" event the forward records (external record)
// once slot 0's last reader is done.
//
// Gates: the gather of l+1 waits for done(l-1) (the pages' gate), for the
// compute stream to begin layer l, or for done(l) ("after": no overlap; on
// one GPU the gather and the GEMMs share one HBM, and a slot read right after
// it was written is partly still in the last-level cache).  With one queue
// (compute == side) the waits between the two roles are implied by queue
// order and are not enqueued; the trace still lists them.
#include <vector>

#include "swr_internal.h"

using swr::fail;

struct swr_planner {
  int32_t start = 0, end = 0;
  hipStream_t compute = nullptr, side = nullptr;
  void* slot[2] = {nullptr, nullptr};
  int64_t slot_bytes = 0;

  struct Layer {
    std::vector<const void*> chunks;
    int64_t chunk_bytes = 0;
  };
  std::vector<Layer> layers;
  hipEvent_t start_evt = nullptr;
  std::vector<hipEvent_t> ready, done;
  // optional timing events around each gather's copy (after the gate wait):
  // a ring of event pairs, one pair per timed dispatch
  std::vector<hipEvent_t> t0, t1;
  int64_t timed_dispatches = 0;
  // and around each layer's compute on the compute stream: c0 recorded when
  // the layer begins (after its ready wait, the last packet before its
  // kernels), c1 after its done record
  std::vector<hipEvent_t> c0, c1;
  int64_t timed_layers = 0;
  // while set, dispatches and layers record no timing events (the rings keep
  // what they hold)
  bool timing_paused = false;
  std::vector<int64_t> layer_slot;  // ring slot of each layer's c0 in this forward

  // gather engine: 0 the copy kernel, 1 the DMA engines
  int32_t engine = 0;
  // LDS each copy workgroup of the planner's gathers reserves (0: none)
  int32_t gather_lds = 0;

  // gate mode SWR_GATE_BEGIN: each gather of layer l+1 waits for the compute
  // stream to begin layer l (after its ready(l) wait) instead of done(l-1);
  // the gather is enqueued by wait_ready_once(l).  SWR_GATE_AFTER: it waits
  // for done(l) and is enqueued by update_done_event(l).
  bool gate_begin = false;
  bool gate_after = false;
  std::vector<hipEvent_t> begin;
  int32_t pending = -1;       // layer whose gather waits for the next begin (or done) record
  bool pending_next = false;  // the next forward's first layer waits likewise

  // cyclic first-layer prefetch
  bool cyclic = false;
  bool next_prefetched = false;  // the next forward's first layer is already gathered

  // first layer gathered on a dedicated stream outside the forward
  hipStream_t pf = nullptr;
  hipEvent_t first_ready = nullptr;  // recorded on pf after the first-layer gather
  hipEvent_t slot0_free = nullptr;   // recorded (external) after slot 0's last reader
  int64_t pf_issued = 0;             // first-layer gathers enqueued on pf

  // per-forward state
  bool reset_called = false;
  std::vector<uint8_t> dispatched, waited, finished;

  int64_t remote_bytes = 0;
  int64_t gathers = 0;
  std::vector<int32_t> trace;

  bool one_queue() const { return compute == side; }
  bool first_external() const { return pf != nullptr; }
  int32_t last_slot0_reader() const { return start + ((end - 1 - start) & ~1); }
  int idx(int32_t layer) const { return layer - start; }
  bool in_range(int32_t layer) const { return layer >= start && layer < end; }
  int slot_of(int32_t layer) const { return (layer - start) & 1; }
  void log(int32_t op, int32_t stream, int32_t layer, int32_t slot_id) {
    trace.push_back(op);
    trace.push_back(stream);
    trace.push_back(layer);
    trace.push_back(slot_id);
  }
};

namespace {

// True while `s` is capturing a graph.  The external record/wait flags make
// graph nodes during a capture and are not used outside one.
hipError_t capturing(hipStream_t s, bool* out) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(s, &st);
  *out = st == hipStreamCaptureStatusActive;
  return e;
}

// Records `ev` on `s`; while `s` captures a graph, as an event-record node of
// that graph after the stream's current capture dependencies, so that every
// replay records it (HIP refuses hipEventRecordExternal under capture).
hipError_t record_visible(hipEvent_t ev, hipStream_t s) {
  bool cap = false;
  hipError_t e = capturing(s, &cap);
  if (e != hipSuccess || !cap) return e == hipSuccess ? hipEventRecord(ev, s) : e;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  unsigned long long id = 0;
  hipGraph_t graph = nullptr;
  const hipGraphNode_t* deps = nullptr;
  size_t ndeps = 0;
  e = hipStreamGetCaptureInfo_v2(s, &st, &id, &graph, &deps, &ndeps);
  if (e != hipSuccess) return e;
  hipGraphNode_t node = nullptr;
  e = hipGraphAddEventRecordNode(&node, graph, deps, ndeps, ev);
  if (e != hipSuccess) return e;
  return hipStreamUpdateCaptureDependencies(s, &node, 1, hipStreamSetCaptureDependencies);
}

void destroy_events(swr_planner* p) {
  if (p->start_evt) (void)hipEventDestroy(p->start_evt);
  if (p->first_ready) (void)hipEventDestroy(p->first_ready);
  if (p->slot0_free) (void)hipEventDestroy(p->slot0_free);
  for (hipEvent_t e : p->ready)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->done)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->begin)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->t0)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->t1)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->c0)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->c1)
    if (e) (void)hipEventDestroy(e);
}

// Side stream: gate, gather of `layer` into its slot, ready record.  With
// `for_next`, the gather is the next forward's first layer (cyclic mode): its
// slot's last reader in this forward is layer end - 2.  `begin_layer` >= 0
// (gate SWR_GATE_BEGIN) gates it on the begin record of that layer;
// `after_layer` >= 0 (gate SWR_GATE_AFTER) on done(after_layer).
int dispatch(swr_planner* p, int32_t layer, bool for_next = false, int32_t begin_layer = -1,
             int32_t after_layer = -1) {
  const int i = p->idx(layer);
  const swr_planner::Layer& L = p->layers[i];
  if (L.chunks.empty()) return fail(SWR_E_SEQUENCE, "planner: layer %d has no chunks (swr_planner_set_layer)", layer);
  hipEvent_t gate;
  const bool by_begin = begin_layer >= 0;
  const int32_t prev = after_layer >= 0 ? after_layer
                       : (for_next ? p->end - 2 : layer - 2);  // last reader of the slot this gather overwrites
  if (by_begin) {
    gate = p->begin[p->idx(begin_layer)];  // recorded on the compute stream after done(prev)
  } else if (prev >= p->start) {
    if (!p->finished[p->idx(prev)])
      return fail(SWR_E_SEQUENCE, "planner: gather of layer %d needs done(%d), which was not recorded", layer, prev);
    gate = p->done[p->idx(prev)];
  } else {
    gate = p->start_evt;
  }
  const int s = p->slot_of(layer);
  int64_t remote = 0;
  int rc;
  const unsigned lds = unsigned(p->gather_lds);
  auto gather = [p, lds](const void* const* chunks, int32_t n, int64_t c, void* slot, int64_t slot_bytes, int32_t rank,
                         hipStream_t side, hipEvent_t g, hipEvent_t ready, int64_t* remote_bytes) {
    if (p->engine == SWR_ENGINE_DMA)
      return swr_reassemble_into_slot_dma(chunks, n, c, slot, slot_bytes, rank, side, g, ready, remote_bytes);
    return swr::reassemble_reserving(chunks, n, c, slot, slot_bytes, rank, side, g, ready, remote_bytes, lds);
  };
  // one queue: the gate precedes the gather and the gather precedes its
  // reader in queue order already, so neither the gate wait nor the ready
  // record is enqueued
  hipEvent_t wait_on = p->one_queue() ? nullptr : gate;
  hipEvent_t ready = p->one_queue() ? nullptr : p->ready[i];
  if (p->t0.empty() || p->timing_paused) {
    rc = gather(L.chunks.data(), int32_t(L.chunks.size()), L.chunk_bytes, p->slot[s], p->slot_bytes, 0, p->side,
                wait_on, ready, &remote);
  } else {
    // same sequence with timing records between the gate wait and the ready record
    const size_t r = size_t(p->timed_dispatches % int64_t(p->t0.size()));
    hipError_t e = wait_on ? hipStreamWaitEvent(p->side, wait_on, 0) : hipSuccess;
    if (e != hipSuccess) return swr::hip_fail(e, "planner: wait gate");
    e = hipEventRecord(p->t0[r], p->side);
    if (e != hipSuccess) return swr::hip_fail(e, "planner: record timing start");
    rc = gather(L.chunks.data(), int32_t(L.chunks.size()), L.chunk_bytes, p->slot[s], p->slot_bytes, 0, p->side,
                nullptr, nullptr, &remote);
    if (rc == SWR_OK) {
      e = hipEventRecord(p->t1[r], p->side);
      if (e == hipSuccess && ready) e = hipEventRecord(ready, p->side);
      if (e != hipSuccess) return swr::hip_fail(e, "planner: record timing end / ready");
      p->timed_dispatches += 1;
    }
  }
  if (rc != SWR_OK) return rc;
  if (by_begin)
    p->log(SWR_OP_WAIT_BEGIN, SWR_STREAM_SIDE, begin_layer, -1);
  else if (prev >= p->start)
    p->log(SWR_OP_WAIT_DONE, SWR_STREAM_SIDE, prev, -1);
  else
    p->log(SWR_OP_WAIT_START, SWR_STREAM_SIDE, -1, -1);
  p->log(for_next ? SWR_OP_COPY_NEXT : SWR_OP_COPY, SWR_STREAM_SIDE, layer, s);
  p->log(SWR_OP_RECORD_READY, SWR_STREAM_SIDE, layer, -1);
  if (for_next)
    p->next_prefetched = true;
  else
    p->dispatched[i] = 1;
  p->remote_bytes += remote;
  p->gathers += 1;
  return SWR_OK;
}

}  // namespace

extern "C" int swr_planner_create(int32_t start, int32_t end, hipStream_t compute, hipStream_t side, void* slot_a,
                                  void* slot_b, int64_t slot_bytes, swr_planner** out) {
  if (!out || !slot_a || !slot_b) return fail(SWR_E_INVALID, "swr_planner_create: null pointer");
  *out = nullptr;
  if (end <= start || start < 0) return fail(SWR_E_INVALID, "swr_planner_create: empty range [%d, %d)", start, end);
  if (end - start > (1 << 20)) return fail(SWR_E_INVALID, "swr_planner_create: too many layers");
  if (slot_bytes <= 0) return fail(SWR_E_INVALID, "swr_planner_create: slot_bytes must be positive");
  if (!swr::aligned(slot_a, 16) || !swr::aligned(slot_b, 16))
    return fail(SWR_E_ALIGN, "swr_planner_create: slots must be 16-byte aligned");
  swr_planner* p = new swr_planner();
  p->start = start;
  p->end = end;
  p->compute = compute;
  p->side = side;
  p->slot[0] = slot_a;
  p->slot[1] = slot_b;
  p->slot_bytes = slot_bytes;
  const int n = end - start;
  p->layers.resize(n);
  p->ready.assign(n, nullptr);
  p->done.assign(n, nullptr);
  p->begin.assign(n, nullptr);
  p->layer_slot.assign(n, -1);
  p->dispatched.assign(n, 0);
  p->waited.assign(n, 0);
  p->finished.assign(n, 0);
  hipError_t e = hipEventCreateWithFlags(&p->start_evt, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->first_ready, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&p->slot0_free, hipEventDisableTiming);
  for (int i = 0; e == hipSuccess && i < n; ++i) {
    e = hipEventCreateWithFlags(&p->ready[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->done[i], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->begin[i], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    destroy_events(p);
    delete p;
    return swr::hip_fail(e, "swr_planner_create: hipEventCreate");
  }
  *out = p;
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_set_layer(swr_planner* p, int32_t layer, const void* const* chunk_dev, int32_t n_chunks,
                                     int64_t chunk_bytes) {
  if (!p || !chunk_dev) return fail(SWR_E_INVALID, "swr_planner_set_layer: null pointer");
  if (!p->in_range(layer))
    return fail(SWR_E_INVALID, "swr_planner_set_layer: layer %d outside [%d, %d)", layer, p->start, p->end);
  if (n_chunks < 1 || n_chunks > SWR_MAX_CHUNKS)
    return fail(SWR_E_INVALID, "swr_planner_set_layer: n_chunks=%d outside [1, 64]", n_chunks);
  if (chunk_bytes <= 0 || chunk_bytes % 16)
    return fail(SWR_E_ALIGN, "swr_planner_set_layer: chunk_bytes must be a positive multiple of 16");
  if (chunk_bytes > p->slot_bytes / n_chunks)
    return fail(SWR_E_CAPACITY, "swr_planner_set_layer: layer %d needs %d chunks of %lld bytes, slots hold %lld",
                layer, n_chunks, (long long)chunk_bytes, (long long)p->slot_bytes);
  for (int i = 0; i < n_chunks; ++i) {
    if (!chunk_dev[i]) return fail(SWR_E_INVALID, "swr_planner_set_layer: chunk %d is null", i);
    if (!swr::aligned(chunk_dev[i], 16)) return fail(SWR_E_ALIGN, "swr_planner_set_layer: chunk %d misaligned", i);
  }
  swr_planner::Layer& L = p->layers[p->idx(layer)];
  L.chunks.assign(chunk_dev, chunk_dev + n_chunks);
  L.chunk_bytes = chunk_bytes;
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_reset(swr_planner* p) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_reset: null pointer");
  // (one queue: the forward-start point is implied by queue order)
  const hipError_t e = p->one_queue() ? hipSuccess : hipEventRecord(p->start_evt, p->compute);
  if (e != hipSuccess) return swr::hip_fail(e, "swr_planner_reset: record start");
  std::fill(p->dispatched.begin(), p->dispatched.end(), 0);
  std::fill(p->waited.begin(), p->waited.end(), 0);
  std::fill(p->finished.begin(), p->finished.end(), 0);
  if (p->next_prefetched) {  // gathered by the previous forward
    p->dispatched[0] = 1;
    p->next_prefetched = false;
  }
  p->pending = -1;
  p->pending_next = false;
  p->trace.clear();
  p->log(SWR_OP_RECORD_START, SWR_STREAM_COMPUTE, -1, -1);
  p->reset_called = true;
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_pre_dispatch(swr_planner* p, int32_t layer) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_pre_dispatch: null pointer");
  if (!p->reset_called) return fail(SWR_E_SEQUENCE, "swr_planner_pre_dispatch: call swr_planner_reset first");
  if (layer != p->start)
    return fail(SWR_E_SEQUENCE, "swr_planner_pre_dispatch: layer %d is not the first layer %d", layer, p->start);
  if (p->dispatched[0]) {
    if (p->cyclic) {  // already gathered by the previous forward
      swr::clear_error();
      return SWR_OK;
    }
    return fail(SWR_E_SEQUENCE, "swr_planner_pre_dispatch: already dispatched");
  }
  if (p->first_external()) {
    // gathered on the dedicated stream (swr_planner_prefetch_first)
    if (p->pf_issued == 0)
      return fail(SWR_E_SEQUENCE, "swr_planner_pre_dispatch: call swr_planner_prefetch_first before the first forward");
    p->dispatched[0] = 1;
    swr::clear_error();
    return SWR_OK;
  }
  const int rc = dispatch(p, layer);
  if (rc == SWR_OK) swr::clear_error();
  return rc;
}

extern "C" int swr_planner_maybe_dispatch(swr_planner* p, int32_t layer) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_maybe_dispatch: null pointer");
  if (layer == p->end && p->cyclic && p->reset_called && !p->next_prefetched) {
    if (!p->dispatched[p->idx(p->end - 1)])
      return fail(SWR_E_SEQUENCE, "swr_planner_maybe_dispatch: next forward before layer %d", p->end - 1);
    if (p->gate_begin || p->gate_after) {  // enqueued by wait_ready_once / update_done_event(end - 1)
      p->pending_next = true;
      swr::clear_error();
      return SWR_OK;
    }
    const int rc = dispatch(p, p->start, true);
    if (rc == SWR_OK) swr::clear_error();
    return rc;
  }
  if (!p->in_range(layer)) {
    swr::clear_error();
    return SWR_OK;
  }
  if (!p->reset_called) return fail(SWR_E_SEQUENCE, "swr_planner_maybe_dispatch: call swr_planner_reset first");
  if (p->dispatched[p->idx(layer)])
    return fail(SWR_E_SEQUENCE, "swr_planner_maybe_dispatch: layer %d already dispatched in this forward", layer);
  if (layer > p->start && !p->dispatched[p->idx(layer - 1)])
    return fail(SWR_E_SEQUENCE, "swr_planner_maybe_dispatch: layer %d before layer %d", layer, layer - 1);
  if ((p->gate_begin || p->gate_after) && layer > p->start) {
    // enqueued by wait_ready_once(layer - 1) (begin) or update_done_event(layer - 1) (after)
    if (p->pending >= 0)
      return fail(SWR_E_SEQUENCE, "swr_planner_maybe_dispatch: layer %d is still pending", p->pending);
    p->pending = layer;
    swr::clear_error();
    return SWR_OK;
  }
  const int rc = dispatch(p, layer);
  if (rc == SWR_OK) swr::clear_error();
  return rc;
}

extern "C" int swr_planner_wait_ready_once(swr_planner* p, int32_t layer, void** slot_out) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_wait_ready_once: null pointer");
  if (!p->in_range(layer))
    return fail(SWR_E_INVALID, "swr_planner_wait_ready_once: layer %d outside [%d, %d)", layer, p->start, p->end);
  const int i = p->idx(layer);
  if (!p->dispatched[i]) return fail(SWR_E_SEQUENCE, "swr_planner_wait_ready_once: layer %d not dispatched", layer);
  if (!p->waited[i]) {
    hipError_t e;
    if (p->first_external() && layer == p->start) {
      // the dedicated stream's gather; while capturing, an external wait (a
      // node of the graph, so every replay waits again)
      bool cap = false;
      e = capturing(p->compute, &cap);
      if (e == hipSuccess) e = hipStreamWaitEvent(p->compute, p->first_ready, cap ? hipEventWaitExternal : 0);
    } else {
      // one queue: the gather precedes this point in queue order already
      e = p->one_queue() ? hipSuccess : hipStreamWaitEvent(p->compute, p->ready[i], 0);
    }
    if (e != hipSuccess) return swr::hip_fail(e, "swr_planner_wait_ready_once: wait");
    p->waited[i] = 1;
    p->log(SWR_OP_WAIT_READY, SWR_STREAM_COMPUTE, layer, p->slot_of(layer));
    const bool next_due = p->pending == layer + 1;
    const bool first_due = p->pending_next && layer == p->end - 1;
    const bool gate_due = p->gate_begin && (next_due || first_due);
    // the begin records: the gate of the pending gather in SWR_GATE_BEGIN
    // mode (two queues only), and the layer's timing start when layers are
    // timed
    if (gate_due && !p->one_queue()) {
      const hipError_t eb = hipEventRecord(p->begin[i], p->compute);
      if (eb != hipSuccess) return swr::hip_fail(eb, "swr_planner_wait_ready_once: record begin");
    }
    if (!p->c0.empty() && !p->timing_paused) {
      const int64_t r = p->timed_layers % int64_t(p->c0.size());
      p->layer_slot[i] = r;
      const hipError_t eb = hipEventRecord(p->c0[size_t(r)], p->compute);
      if (eb != hipSuccess) return swr::hip_fail(eb, "swr_planner_wait_ready_once: record timing start");
    }
    if (gate_due) {
      p->log(SWR_OP_RECORD_BEGIN, SWR_STREAM_COMPUTE, layer, -1);
      int rc;
      if (next_due) {
        p->pending = -1;
        rc = dispatch(p, layer + 1, false, layer);
      } else {
        p->pending_next = false;
        rc = dispatch(p, p->start, true, layer);
      }
      if (rc != SWR_OK) return rc;
    }
  }
  if (slot_out) *slot_out = p->slot[p->slot_of(layer)];
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_update_done_event(swr_planner* p, int32_t layer) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_update_done_event: null pointer");
  if (!p->in_range(layer))
    return fail(SWR_E_INVALID, "swr_planner_update_done_event: layer %d outside [%d, %d)", layer, p->start, p->end);
  const int i = p->idx(layer);
  if (!p->waited[i])
    return fail(SWR_E_SEQUENCE, "swr_planner_update_done_event: layer %d did not wait for its weights", layer);
  hipError_t e = p->one_queue() ? hipSuccess : hipEventRecord(p->done[i], p->compute);
  if (e != hipSuccess) return swr::hip_fail(e, "swr_planner_update_done_event: record");
  if (!p->c1.empty() && p->layer_slot[i] >= 0) {
    e = hipEventRecord(p->c1[size_t(p->layer_slot[i])], p->compute);
    if (e != hipSuccess) return swr::hip_fail(e, "swr_planner_update_done_event: record timing end");
    p->layer_slot[i] = -1;
    p->timed_layers += 1;
  }
  p->finished[i] = 1;
  p->log(SWR_OP_RECORD_DONE, SWR_STREAM_COMPUTE, layer, -1);
  if (p->first_external() && layer == p->last_slot0_reader()) {
    // slot 0 is free for the next forward's first layer (while capturing, a
    // record node of the graph, so that every replay records it)
    e = record_visible(p->slot0_free, p->compute);
    if (e != hipSuccess) return swr::hip_fail(e, "swr_planner_update_done_event: record free");
    p->log(SWR_OP_RECORD_FREE, SWR_STREAM_COMPUTE, layer, 0);
  }
  if (p->gate_after) {
    // the pending gather of layer + 1 (or of the next forward's first layer)
    // waits for done(layer), just recorded
    int rc = SWR_OK;
    if (p->pending == layer + 1) {
      p->pending = -1;
      rc = dispatch(p, layer + 1, false, -1, layer);
    } else if (p->pending_next && layer == p->end - 1) {
      p->pending_next = false;
      rc = dispatch(p, p->start, true, -1, layer);
    }
    if (rc != SWR_OK) return rc;
  }
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_set_cyclic(swr_planner* p, int32_t enabled) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_set_cyclic: null pointer");
  if (enabled && ((p->end - p->start) % 2 != 0 || p->end - p->start < 2))
    return fail(SWR_E_INVALID, "swr_planner_set_cyclic: needs an even number of layers (have %d)", p->end - p->start);
  if (enabled && p->first_external())
    return fail(SWR_E_INVALID, "swr_planner_set_cyclic: the first layer is gathered on a dedicated stream");
  p->cyclic = enabled != 0;
  if (!p->cyclic) p->next_prefetched = false;
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_set_first_prefetch(swr_planner* p, hipStream_t stream) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_set_first_prefetch: null pointer");
  if (stream && stream == p->compute)
    return fail(SWR_E_INVALID, "swr_planner_set_first_prefetch: the prefetch stream must not be the compute stream");
  if (stream && p->cyclic)
    return fail(SWR_E_INVALID, "swr_planner_set_first_prefetch: cyclic mode gathers the first layer already");
  if (p->reset_called && p->dispatched[0] && !p->finished[p->idx(p->end - 1)])
    return fail(SWR_E_SEQUENCE, "swr_planner_set_first_prefetch: a forward is in progress");
  p->pf = stream;
  p->pf_issued = 0;
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_prefetch_first(swr_planner* p) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_prefetch_first: null pointer");
  if (!p->first_external())
    return fail(SWR_E_SEQUENCE, "swr_planner_prefetch_first: no prefetch stream (swr_planner_set_first_prefetch)");
  const swr_planner::Layer& L = p->layers[0];
  if (L.chunks.empty())
    return fail(SWR_E_SEQUENCE, "swr_planner_prefetch_first: layer %d has no chunks (swr_planner_set_layer)", p->start);
  // slot 0's last reader in the latest forward; before any forward the event
  // was never recorded and the wait orders nothing
  hipError_t e = hipStreamWaitEvent(p->pf, p->slot0_free, 0);
  if (e != hipSuccess) return swr::hip_fail(e, "swr_planner_prefetch_first: wait free");
  int64_t remote = 0;
  int rc;
  if (p->engine == SWR_ENGINE_DMA)
    rc = swr_reassemble_into_slot_dma(L.chunks.data(), int32_t(L.chunks.size()), L.chunk_bytes, p->slot[0],
                                      p->slot_bytes, 0, p->pf, nullptr, p->first_ready, &remote);
  else
    rc = swr::reassemble_reserving(L.chunks.data(), int32_t(L.chunks.size()), L.chunk_bytes, p->slot[0],
                                   p->slot_bytes, 0, p->pf, nullptr, p->first_ready, &remote,
                                   unsigned(p->gather_lds));
  if (rc != SWR_OK) return rc;
  p->log(SWR_OP_WAIT_FREE, SWR_STREAM_PREFETCH, p->last_slot0_reader(), -1);
  p->log(SWR_OP_COPY_NEXT, SWR_STREAM_PREFETCH, p->start, 0);
  p->log(SWR_OP_RECORD_READY, SWR_STREAM_PREFETCH, p->start, -1);
  p->remote_bytes += remote;
  p->gathers += 1;
  p->pf_issued += 1;
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_set_gate(swr_planner* p, int32_t gate) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_set_gate: null pointer");
  if (gate != SWR_GATE_DONE && gate != SWR_GATE_BEGIN && gate != SWR_GATE_AFTER)
    return fail(SWR_E_INVALID, "swr_planner_set_gate: unknown gate %d", gate);
  if (p->pending >= 0 || p->pending_next)
    return fail(SWR_E_SEQUENCE, "swr_planner_set_gate: a gather is still pending");
  p->gate_begin = gate == SWR_GATE_BEGIN;
  p->gate_after = gate == SWR_GATE_AFTER;
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_set_copy_engine(swr_planner* p, int32_t engine) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_set_copy_engine: null pointer");
  if (engine != SWR_ENGINE_KERNEL && engine != SWR_ENGINE_DMA)
    return fail(SWR_E_INVALID, "swr_planner_set_copy_engine: unknown engine %d", engine);
  p->engine = engine;
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_set_gather_lds(swr_planner* p, int32_t bytes) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_set_gather_lds: null pointer");
  if (bytes < 0 || bytes > SWR_MAX_GATHER_LDS)
    return fail(SWR_E_INVALID, "swr_planner_set_gather_lds: %d bytes outside [0, %d]", bytes, SWR_MAX_GATHER_LDS);
  p->gather_lds = bytes;
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_set_timing(swr_planner* p, int32_t capacity) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_set_timing: null pointer");
  if (capacity < 0 || capacity > (1 << 16))
    return fail(SWR_E_INVALID, "swr_planner_set_timing: capacity %d outside [0, 65536]", capacity);
  for (hipEvent_t e : p->t0)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->t1)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->c0)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->c1)
    if (e) (void)hipEventDestroy(e);
  p->t0.assign(capacity, nullptr);
  p->t1.assign(capacity, nullptr);
  p->c0.assign(capacity, nullptr);
  p->c1.assign(capacity, nullptr);
  std::fill(p->layer_slot.begin(), p->layer_slot.end(), -1);
  p->timed_dispatches = 0;
  p->timed_layers = 0;
  hipError_t e = hipSuccess;
  // Timing events carry no system-scope fence: they only mark time, and on
  // MI355X a fenced record costs about 2.5 us between two kernels (its cache
  // writeback) against under 1 us without it.
  const unsigned tf = hipEventDisableSystemFence;
  for (int i = 0; e == hipSuccess && i < capacity; ++i) {
    e = hipEventCreateWithFlags(&p->t0[i], tf);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->t1[i], tf);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->c0[i], tf);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->c1[i], tf);
  }
  if (e != hipSuccess) {
    for (auto* v : {&p->t0, &p->t1, &p->c0, &p->c1}) {
      for (hipEvent_t x : *v)
        if (x) (void)hipEventDestroy(x);
      v->clear();
    }
    return swr::hip_fail(e, "swr_planner_set_timing: hipEventCreate");
  }
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_pause_timing(swr_planner* p, int32_t paused) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_pause_timing: null pointer");
  p->timing_paused = paused != 0;
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_gather_times(const swr_planner* p, float* ms, int32_t cap, int32_t* n) {
  if (!p || !n || (cap > 0 && !ms)) return fail(SWR_E_INVALID, "swr_planner_gather_times: null pointer");
  const int64_t ring = int64_t(p->t0.size());
  const int64_t avail = p->timed_dispatches < ring ? p->timed_dispatches : ring;
  const int64_t count = avail < cap ? avail : cap;
  *n = int32_t(count);
  const int64_t first = p->timed_dispatches - avail;  // oldest dispatch still in the ring
  for (int64_t k = 0; k < count; ++k) {
    const size_t r = size_t((first + k) % ring);
    const hipError_t e = hipEventElapsedTime(&ms[k], p->t0[r], p->t1[r]);
    if (e != hipSuccess) return swr::hip_fail(e, "swr_planner_gather_times: hipEventElapsedTime");
  }
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_layer_times(const swr_planner* p, float* ms, int32_t cap, int32_t* n) {
  if (!p || !n || (cap > 0 && !ms)) return fail(SWR_E_INVALID, "swr_planner_layer_times: null pointer");
  const int64_t ring = int64_t(p->c0.size());
  const int64_t avail = p->timed_layers < ring ? p->timed_layers : ring;
  const int64_t count = avail < cap ? avail : cap;
  *n = int32_t(count);
  const int64_t first = p->timed_layers - avail;
  for (int64_t k = 0; k < count; ++k) {
    const size_t r = size_t((first + k) % ring);
    const hipError_t e = hipEventElapsedTime(&ms[k], p->c0[r], p->c1[r]);
    if (e != hipSuccess) return swr::hip_fail(e, "swr_planner_layer_times: hipEventElapsedTime");
  }
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_counters(const swr_planner* p, int64_t* remote_bytes, int64_t* gathers) {
  if (!p) return fail(SWR_E_INVALID, "swr_planner_counters: null pointer");
  if (remote_bytes) *remote_bytes = p->remote_bytes;
  if (gathers) *gathers = p->gathers;
  swr::clear_error();
  return SWR_OK;
}

extern "C" int swr_planner_trace(const swr_planner* p, int32_t* ops, int32_t cap, int32_t* n) {
  if (!p || !n) return fail(SWR_E_INVALID, "swr_planner_trace: null pointer");
  const int32_t count = int32_t(p->trace.size() / 4);
  *n = count;
  if (ops) {
    const int32_t m = count < cap ? count : cap;
    for (int32_t i = 0; i < 4 * m; ++i) ops[i] = p->trace[i];
  }
  swr::clear_error();
  return SWR_OK;
}

extern "C" void swr_planner_destroy(swr_planner* p) {
  if (!p) return;
  destroy_events(p);
  delete p;
}
