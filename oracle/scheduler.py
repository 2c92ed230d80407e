"""Lookahead gather with two ping-pong slots -- oracle (test infrastructure only).

Weight-sharding page (zdszero.github.io):
* section "lookahead and ping-pong slot": while layer l computes, the gather
  of layer l+1 is issued on a side stream; layer l+1 waits for that gather's
  completion event before it computes; full weights live in only two slots
  that alternate by layer, so the gather of l+1 overwrites the slot layer l-1
  used and must first wait for l-1's compute to finish (the gate event);
* section "implementation in SGLang": the model loop is reset(),
  pre_dispatch(start), then per layer maybe_dispatch(i+1), the layer's
  forward, update_done_event(i);
* section "CUDA graph and the draft model": after one launch the current
  stream waits at most once (wait_ready_once), and the sequence is fixed.

Readings where the page is silent: the first dispatched layer uses slot 0,
i.e. layer l uses slot (l - start) mod 2; a gather with no previous layer in
this forward is gated by a forward-start event that reset() records on the
compute stream (it covers the previous forward's readers).

Cyclic forwards (the same layers run again and again, with an even number of
layers): the draft-model part of the page's CUDA-graph section moves a first
layer's gather out of the loop so that it overlaps other work.  Here
maybe_dispatch(end) gathers the *next* forward's first layer into slot 0 --
free once done(end - 2) is recorded, since the last layer uses slot 1 -- and
the next forward skips its own pre_dispatch gather.

Gate "begin" (a one-GPU variant, same dependencies): the gather of layer
l+1 waits for an event recorded on the compute stream right after that
stream's wait for ready(l) -- the moment layer l begins.  That point follows
done(l-1) on the compute stream, and the gather of l precedes the gather of
l+1 on the side stream, so the gather may start exactly when the page's gate
allows; it is enqueued after the compute stream's ready wait instead of
before it.

Gate "after" (a one-GPU schedule, same slots and ready/done events): the
gather of layer l+1 waits for done(l), the layer that runs just before it,
and is enqueued when that done event is recorded.  On one GPU the gather
and the GEMMs draw on the same HBM, so running them one after the other (and
reading each slot right after it was written) can beat running them side by
side; the gate is the page's done gate moved one layer later, which orders
the gather after both earlier readers of its slot.

First-layer prefetch on a dedicated stream (the page's CUDA-graph section:
the draft model's layer-0 gather runs outside the captured graph, on its own
stream, overlapping the main model's last layers, and the graph waits for
it).  Here the forward (which may be captured) does not gather its first
layer: its compute stream waits for ready(start) recorded by a prefetch made
outside it, and it records a "free" event once slot 0's last reader in the
forward, layer l0 = the last layer with (l - start) even, is done.  The
prefetch, on stream "prefetch", waits for that event, gathers layer start
into slot 0 for the next forward and records ready(start).

An op is a tuple (name, stream, layer, slot) with names
  record_start  wait_start  wait_done  copy  copy_next  record_ready
  wait_ready  record_done  record_begin  wait_begin  record_free  wait_free
and layer/slot -1 where they do not apply; ``copy_next`` is a gather made in
one forward for the next one.  ``check_trace`` is an independent
happens-before checker: it does not reuse ``expected_trace``.
"""
from __future__ import annotations

COMPUTE, SIDE, PREFETCH = "compute", "side", "prefetch"


def slot_of(layer: int, start: int) -> int:
    return (layer - start) % 2


def last_slot0_reader(start: int, end: int) -> int:
    """The last layer of [start, end) that reads slot 0."""
    return start + ((end - 1 - start) & ~1)


def prefetch_first_ops(start: int, end: int) -> list[tuple]:
    """The dedicated-stream gather of the next forward's first layer."""
    return [("wait_free", PREFETCH, last_slot0_reader(start, end), -1), ("copy_next", PREFETCH, start, 0),
            ("record_ready", PREFETCH, start, -1)]


def expected_trace(start: int, end: int, prefetched: bool = False, prefetch_next: bool = False,
                   gate: str = "done", first_external: bool = False) -> list[tuple]:
    """Launch/wait sequence of one forward over layers [start, end).

    prefetched: the previous forward already gathered layer `start` (cyclic mode);
    prefetch_next: this forward gathers the next forward's layer `start`;
    gate: "done" (the page's gate), "begin" or "after";
    first_external: layer `start` comes from a dedicated-stream prefetch made
    outside the forward (prefetch_first_ops), and the forward records the
    "free" event after its last reader of slot 0."""
    ops: list[tuple] = [("record_start", COMPUTE, -1, -1)]
    if end <= start:
        return ops
    if first_external:
        if prefetched or prefetch_next:
            raise ValueError("the dedicated first-layer prefetch replaces the cyclic one")
        inner = expected_trace(start, end, prefetched=True, gate=gate)
        l0 = last_slot0_reader(start, end)
        out = []
        for op in inner:
            out.append(op)
            if op == ("record_done", COMPUTE, l0, -1):
                out.append(("record_free", COMPUTE, l0, 0))
        return out
    if prefetch_next and ((end - start) % 2 or end - start < 2):
        raise ValueError("cyclic prefetch needs an even number of layers")
    if gate not in ("done", "begin", "after"):
        raise ValueError("gate is 'done', 'begin' or 'after'")
    if gate == "after":
        if not prefetched:
            ops += [("wait_start", SIDE, -1, -1), ("copy", SIDE, start, 0), ("record_ready", SIDE, start, -1)]
        for layer in range(start, end):
            ops.append(("wait_ready", COMPUTE, layer, slot_of(layer, start)))
            ops.append(("record_done", COMPUTE, layer, -1))
            if layer + 1 < end:
                ops += [("wait_done", SIDE, layer, -1), ("copy", SIDE, layer + 1, slot_of(layer + 1, start)),
                        ("record_ready", SIDE, layer + 1, -1)]
            elif prefetch_next:
                ops += [("wait_done", SIDE, layer, -1), ("copy_next", SIDE, start, 0),
                        ("record_ready", SIDE, start, -1)]
        return ops
    if gate == "begin":
        if not prefetched:
            ops += [("wait_start", SIDE, -1, -1), ("copy", SIDE, start, 0), ("record_ready", SIDE, start, -1)]
        for layer in range(start, end):
            ops.append(("wait_ready", COMPUTE, layer, slot_of(layer, start)))
            nxt = layer + 1 < end
            if nxt or prefetch_next:
                ops.append(("record_begin", COMPUTE, layer, -1))
                ops.append(("wait_begin", SIDE, layer, -1))
                if nxt:
                    ops.append(("copy", SIDE, layer + 1, slot_of(layer + 1, start)))
                    ops.append(("record_ready", SIDE, layer + 1, -1))
                else:
                    ops.append(("copy_next", SIDE, start, 0))
                    ops.append(("record_ready", SIDE, start, -1))
            ops.append(("record_done", COMPUTE, layer, -1))
        return ops

    def dispatch(layer: int) -> None:
        prev = layer - 2  # the last reader of the slot this gather overwrites
        if prev >= start:
            ops.append(("wait_done", SIDE, prev, -1))
        else:
            ops.append(("wait_start", SIDE, -1, -1))
        ops.append(("copy", SIDE, layer, slot_of(layer, start)))
        ops.append(("record_ready", SIDE, layer, -1))

    if not prefetched:
        dispatch(start)  # pre_dispatch(start)
    for layer in range(start, end):
        if layer + 1 < end:
            dispatch(layer + 1)  # maybe_dispatch(layer + 1)
        elif prefetch_next:
            # maybe_dispatch(end): the next forward's first layer into slot 0,
            # whose last reader in this forward is layer end - 2
            ops.append(("wait_done", SIDE, end - 2, -1))
            ops.append(("copy_next", SIDE, start, 0))
            ops.append(("record_ready", SIDE, start, -1))
        ops.append(("wait_ready", COMPUTE, layer, slot_of(layer, start)))
        ops.append(("record_done", COMPUTE, layer, -1))
    return ops


def _event(op: tuple):
    name, _, layer, _ = op
    if name in ("record_start", "wait_start"):
        return ("start",)
    if name in ("record_ready", "wait_ready"):
        return ("ready", layer)
    if name in ("record_done", "wait_done"):
        return ("done", layer)
    if name in ("record_begin", "wait_begin"):
        return ("begin", layer)
    if name in ("record_free", "wait_free"):
        return ("free",)
    return None


def check_trace(forwards: list[list[tuple]]) -> list[str]:
    """Check the data-race and data-flow properties of one or more forwards
    enqueued back to back.  Returns a list of violations (empty if clean).

    Model: each stream runs its ops in order; ``wait_*`` on a stream orders
    everything after it behind the latest ``record_*`` of the same event
    enqueued before the wait (a wait with no earlier record orders nothing).
    Layer l's compute reads its slot between its ``wait_ready`` and its
    ``record_done`` on the compute stream.  Violations reported:
      * a copy and a compute on the same slot that are not ordered;
      * a compute whose latest ordered copy into its slot is not its layer's;
      * a layer whose compute stream waited for ready more than once or never.
    """
    nodes: list[tuple] = []  # (kind, stream, layer, slot, forward)
    edges: dict[int, set[int]] = {}
    last_on_stream: dict[str, int] = {}
    last_record: dict[tuple, int] = {}
    problems: list[str] = []

    def add(kind, stream, layer, slot, fwd):
        idx = len(nodes)
        nodes.append((kind, stream, layer, slot, fwd))
        edges[idx] = set()
        if stream in last_on_stream:
            edges[last_on_stream[stream]].add(idx)
        last_on_stream[stream] = idx
        return idx

    for f, ops in enumerate(forwards):
        waits: dict[int, int] = {}
        reading: dict[int, int] = {}
        for op in ops:
            name, stream, layer, slot = op
            ev = _event(op)
            if name == "record_done":
                # the layer's compute runs on the compute stream right before its done record
                if layer in reading:
                    add("compute", stream, layer, reading[layer], f)
                else:
                    problems.append(f"forward {f}: layer {layer} computed without waiting for ready")
            if name.startswith("record"):
                last_record[ev] = add(name, stream, layer, slot, f)
            elif name.startswith("wait"):
                idx = add(name, stream, layer, slot, f)
                if ev in last_record:
                    edges[last_record[ev]].add(idx)
                if name == "wait_ready":
                    waits[layer] = waits.get(layer, 0) + 1
                    reading[layer] = slot
            elif name == "copy":
                add("copy", stream, layer, slot, f)
            elif name == "copy_next":
                add("copy", stream, layer, slot, f + 1)  # feeds the next forward
            else:
                problems.append(f"unknown op {op}")
        for layer, n in waits.items():
            if n != 1:
                problems.append(f"forward {f}: layer {layer} waited for ready {n} times")

    # transitive closure by DFS from each node (traces are small)
    reach: list[set[int]] = []
    for s in range(len(nodes)):
        seen, stack = set(), [s]
        while stack:
            u = stack.pop()
            for v in edges[u]:
                if v not in seen:
                    seen.add(v)
                    stack.append(v)
        reach.append(seen)

    def before(a: int, b: int) -> bool:
        return b in reach[a]

    copies = [i for i, n in enumerate(nodes) if n[0] == "copy"]
    computes = [i for i, n in enumerate(nodes) if n[0] == "compute"]
    for c in computes:
        _, _, layer, slot, f = nodes[c]
        ordered_writes = []
        for w in copies:
            if nodes[w][3] != slot:
                continue
            if before(w, c):
                ordered_writes.append(w)
            elif not before(c, w):
                wl, wf = nodes[w][2], nodes[w][4]
                problems.append(
                    f"race: copy of layer {wl} (forward {wf}) into slot {slot} is unordered with "
                    f"the compute of layer {layer} (forward {f})")
        latest = [w for w in ordered_writes if not any(before(w, o) for o in ordered_writes if o != w)]
        if len(latest) != 1 or nodes[latest[0]][2] != layer or nodes[latest[0]][4] != f:
            problems.append(f"forward {f}: layer {layer} does not read its own weights from slot {slot}")
    return problems
