"""GPU checks of the lookahead / ping-pong planner (weight_sharding,
zdszero.github.io, sections on lookahead and ping-pong slots, on the SGLang
implementation and on CUDA graphs).

* The planner's recorded launch/wait sequence equals the oracle's model and
  passes the oracle's happens-before checker.
* A pipelined forward over several layers, with each layer's compute delayed
  on the compute stream, produces every layer's oracle output: if a gather
  overwrote a slot still being read, some layer would read another layer's
  weights.
"""
import numpy as np
import pytest
import torch

import sharded_weight_reassembly_amd as swr
import synth
from oracle import accounting, gemm
from oracle import layout as olayout
from oracle import scheduler as osch

from gpu_util import DEV, assert_close_rows, bf16, note, u8, values

pytestmark = pytest.mark.gpu

GATE_NAMES = {swr.GATE_DONE: "done", swr.GATE_BEGIN: "begin", swr.GATE_AFTER: "after"}


def _layers(wl, n_layers, n_chunks):
    layers = []
    for layer in range(n_layers):
        ws = wl.layer_weights(layer)
        shp = [(o, i, d) for _, o, i, d in wl.weights]
        views, lay = swr.plan_layer(shp, n_chunks)
        chunks = [torch.empty(lay["chunk_bytes"], dtype=torch.uint8, device=DEV) for _ in range(n_chunks)]
        swr.pack_layer(lay, views, [u8(w.raw()) for w in ws], chunks)
        layers.append(dict(ws=ws, views=views, lay=lay, chunks=chunks))
    torch.cuda.synchronize()
    return layers


def _forward(planner, layers, start, x_dev, outs, ws_buf, delay=None):
    wl = synth.TINY
    planner.reset()
    planner.pre_dispatch(start)
    for i in range(start, start + len(layers)):
        planner.maybe_dispatch(i + 1)
        base = planner.wait_ready_once(i)
        assert planner.wait_ready_once(i) == base  # second call: no new wait
        if delay is not None:
            delay()  # keeps the compute stream busy so an ungated gather would overlap
        L = layers[i - start]
        swr.mlp_forward(base + L["views"][0]["offset"], None, base + L["views"][1]["offset"], None, "bf16",
                        wl.hidden, wl.intermediate, x_dev, outs[i - start], ws_buf)
        planner.update_done_event(i)


@pytest.mark.parametrize("start,n_layers", [(0, 1), (0, 2), (1, 5)])
def test_trace_matches_model_and_outputs_match_oracle(start, n_layers):
    note(f"planner start={start} layers={n_layers}")
    wl = synth.TINY
    layers = _layers(wl, n_layers, wl.n_chunks)
    total = layers[0]["lay"]["total_bytes"]
    slot_a = torch.empty(total, dtype=torch.uint8, device=DEV)
    slot_b = torch.empty(total, dtype=torch.uint8, device=DEV)
    compute = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    p = swr.Planner(start, start + n_layers, compute, side, slot_a, slot_b)
    for i, L in enumerate(layers):
        p.set_layer(start + i, L["chunks"], L["lay"]["chunk_bytes"])
    x = synth.activations(synth.seed_for(1, 0, 50), 4, wl.hidden)
    xd = bf16(x)
    outs = [torch.empty((4, wl.hidden), dtype=torch.bfloat16, device=DEV) for _ in layers]
    wsb = torch.empty(swr.mlp_workspace_bytes(4, wl.hidden, wl.intermediate, "bf16"), dtype=torch.uint8, device=DEV)
    a = torch.randn(2048, 2048, device=DEV)

    def delay():
        for _ in range(4):
            torch.mm(a, a)

    traces = []
    for _ in range(3):  # back-to-back forwards reuse the slots
        _forward(p, layers, start, xd, outs, wsb, delay)
        traces.append(p.trace())
    torch.cuda.synchronize()
    expected = osch.expected_trace(start, start + n_layers)
    for t in traces:
        assert t == expected
    assert osch.check_trace(traces) == []
    for i, L in enumerate(layers):
        ws = L["ws"]
        _, _, ref = gemm.mlp_f64(x, ws[0].raw(), None, ws[1].raw(), None, "bf16", wl.hidden, wl.intermediate)
        assert_close_rows(values(outs[i]), ref, what=f"layer {start + i}")
    remote, gathers = p.counters()
    assert gathers == 3 * n_layers
    assert remote == 3 * n_layers * accounting.transfer_bytes(total, wl.n_chunks)
    p.close()


def test_sequence_errors():
    wl = synth.TINY
    layers = _layers(wl, 2, wl.n_chunks)
    total = layers[0]["lay"]["total_bytes"]
    slot_a = torch.empty(total, dtype=torch.uint8, device=DEV)
    slot_b = torch.empty(total, dtype=torch.uint8, device=DEV)
    p = swr.Planner(0, 2, torch.cuda.current_stream(), torch.cuda.Stream(), slot_a, slot_b)
    with pytest.raises(swr.SwrError) as e:
        p.pre_dispatch(0)  # before reset
    assert e.value.code == swr.E_SEQUENCE
    p.reset()
    with pytest.raises(swr.SwrError) as e:
        p.pre_dispatch(0)  # layer 0 has no chunks yet
    assert e.value.code == swr.E_SEQUENCE
    for i, L in enumerate(layers):
        p.set_layer(i, L["chunks"], L["lay"]["chunk_bytes"])
    p.reset()
    with pytest.raises(swr.SwrError) as e:
        p.wait_ready_once(1)  # not dispatched
    assert e.value.code == swr.E_SEQUENCE
    p.pre_dispatch(0)
    with pytest.raises(swr.SwrError) as e:
        p.update_done_event(0)  # did not wait
    assert e.value.code == swr.E_SEQUENCE
    p.maybe_dispatch(2)  # outside the range: no-op
    with pytest.raises(swr.SwrError) as e:
        p.set_layer(0, layers[0]["chunks"], 1 << 40)
    assert e.value.code == swr.E_CAPACITY
    with pytest.raises(swr.SwrError) as e:
        # N * C wraps to 0 in int64: still refused
        p.set_layer(0, layers[0]["chunks"][:4], 1 << 62)
    assert e.value.code == swr.E_CAPACITY
    torch.cuda.synchronize()
    p.close()


@pytest.mark.parametrize("start,n_layers", [(0, 2), (1, 4)])
def test_cyclic_prefetch_on_gpu(start, n_layers):
    """Cyclic mode: each forward gathers the next forward's first layer during its
    last layer; traces equal the oracle's model, outputs equal the oracle's."""
    note(f"planner cyclic start={start} layers={n_layers}")
    wl = synth.TINY
    layers = _layers(wl, n_layers, wl.n_chunks)
    total = layers[0]["lay"]["total_bytes"]
    slot_a = torch.empty(total, dtype=torch.uint8, device=DEV)
    slot_b = torch.empty(total, dtype=torch.uint8, device=DEV)
    p = swr.Planner(start, start + n_layers, torch.cuda.current_stream(), torch.cuda.Stream(), slot_a, slot_b)
    for i, L in enumerate(layers):
        p.set_layer(start + i, L["chunks"], L["lay"]["chunk_bytes"])
    p.set_cyclic(True)
    x = synth.activations(synth.seed_for(1, 0, 50), 4, wl.hidden)
    xd = bf16(x)
    wsb = torch.empty(swr.mlp_workspace_bytes(4, wl.hidden, wl.intermediate, "bf16"), dtype=torch.uint8, device=DEV)
    a = torch.randn(2048, 2048, device=DEV)

    def delay():
        for _ in range(4):
            torch.mm(a, a)

    traces, outs_all = [], []
    for _ in range(4):
        outs = [torch.empty((4, wl.hidden), dtype=torch.bfloat16, device=DEV) for _ in layers]
        _forward(p, layers, start, xd, outs, wsb, delay)
        traces.append(p.trace())
        outs_all.append(outs)
    torch.cuda.synchronize()
    end = start + n_layers
    assert traces[0] == osch.expected_trace(start, end, prefetched=False, prefetch_next=True)
    for t in traces[1:]:
        assert t == osch.expected_trace(start, end, prefetched=True, prefetch_next=True)
    assert osch.check_trace(traces) == []
    for outs in outs_all:
        for i, L in enumerate(layers):
            ws = L["ws"]
            _, _, ref = gemm.mlp_f64(x, ws[0].raw(), None, ws[1].raw(), None, "bf16", wl.hidden, wl.intermediate)
            assert_close_rows(values(outs[i]), ref, what=f"cyclic layer {start + i}")
    _, gathers = p.counters()
    assert gathers == 4 * n_layers + 1  # one per layer per forward, plus the last forward's early gather
    p.set_cyclic(False)
    p.close()


def test_cyclic_needs_even_layers():
    wl = synth.TINY
    layers = _layers(wl, 1, wl.n_chunks)
    total = layers[0]["lay"]["total_bytes"]
    slot = torch.empty(total, dtype=torch.uint8, device=DEV)
    p = swr.Planner(0, 3, torch.cuda.current_stream(), torch.cuda.Stream(), slot, torch.empty_like(slot))
    with pytest.raises(swr.SwrError) as e:
        p.set_cyclic(True)
    assert e.value.code == swr.E_INVALID
    p.close()


@pytest.mark.parametrize("start,n_layers,cyclic", [(0, 3, False), (1, 4, True)])
def test_dma_engine_planner(start, n_layers, cyclic):
    """The planner with the DMA-engine gather: same launch/wait sequence as the
    copy kernel, and every layer's outputs equal the oracle's."""
    note(f"planner dma engine start={start} layers={n_layers} cyclic={cyclic}")
    wl = synth.TINY
    layers = _layers(wl, n_layers, wl.n_chunks)
    total = layers[0]["lay"]["total_bytes"]
    slot_a = torch.empty(total, dtype=torch.uint8, device=DEV)
    slot_b = torch.empty(total, dtype=torch.uint8, device=DEV)
    p = swr.Planner(start, start + n_layers, torch.cuda.current_stream(), torch.cuda.Stream(), slot_a, slot_b)
    for i, L in enumerate(layers):
        p.set_layer(start + i, L["chunks"], L["lay"]["chunk_bytes"])
    p.set_copy_engine(swr.ENGINE_DMA)
    with pytest.raises(swr.SwrError) as e:
        p.set_copy_engine(7)
    assert e.value.code == swr.E_INVALID
    if cyclic:
        p.set_cyclic(True)
    x = synth.activations(synth.seed_for(1, 0, 50), 4, wl.hidden)
    xd = bf16(x)
    wsb = torch.empty(swr.mlp_workspace_bytes(4, wl.hidden, wl.intermediate, "bf16"), dtype=torch.uint8, device=DEV)
    a = torch.randn(2048, 2048, device=DEV)

    def delay():
        for _ in range(4):
            torch.mm(a, a)

    traces, outs_all = [], []
    for _ in range(3):
        outs = [torch.empty((4, wl.hidden), dtype=torch.bfloat16, device=DEV) for _ in layers]
        _forward(p, layers, start, xd, outs, wsb, delay)
        traces.append(p.trace())
        outs_all.append(outs)
    torch.cuda.synchronize()
    end = start + n_layers
    if cyclic:
        assert traces[0] == osch.expected_trace(start, end, prefetched=False, prefetch_next=True)
        assert all(t == osch.expected_trace(start, end, prefetched=True, prefetch_next=True) for t in traces[1:])
    else:
        assert all(t == osch.expected_trace(start, end) for t in traces)
    assert osch.check_trace(traces) == []
    for outs in outs_all:
        for i, L in enumerate(layers):
            ws = L["ws"]
            _, _, ref = gemm.mlp_f64(x, ws[0].raw(), None, ws[1].raw(), None, "bf16", wl.hidden, wl.intermediate)
            assert_close_rows(values(outs[i]), ref, what=f"dma layer {start + i}")
    p.set_cyclic(False)
    p.close()


@pytest.mark.parametrize("gather_lds,gate", [(57344, swr.GATE_DONE), (32768, swr.GATE_BEGIN), (65536, swr.GATE_DONE)])
def test_gather_lds_reservation(gather_lds, gate):
    """Copy workgroups that reserve LDS (fewer per CU): the same launch/wait
    sequence, slots bit-exact to the flat buffer, outputs equal to the oracle;
    reservations outside [0, 64 KiB] are refused."""
    note(f"planner gather_lds={gather_lds} gate={gate}")
    wl = synth.TINY
    n_layers = 4
    layers = _layers(wl, n_layers, wl.n_chunks)
    total = layers[0]["lay"]["total_bytes"]
    slot_a = torch.empty(total, dtype=torch.uint8, device=DEV)
    slot_b = torch.empty(total, dtype=torch.uint8, device=DEV)
    p = swr.Planner(0, n_layers, torch.cuda.current_stream(), torch.cuda.Stream(), slot_a, slot_b)
    for i, L in enumerate(layers):
        p.set_layer(i, L["chunks"], L["lay"]["chunk_bytes"])
    for bad in (-1, 65537):
        with pytest.raises(swr.SwrError) as e:
            p.set_gather_lds(bad)
        assert e.value.code == swr.E_INVALID
    p.set_gather_lds(gather_lds)
    p.set_gate(gate)
    x = synth.activations(synth.seed_for(1, 0, 50), 4, wl.hidden)
    xd = bf16(x)
    wsb = torch.empty(swr.mlp_workspace_bytes(4, wl.hidden, wl.intermediate, "bf16"), dtype=torch.uint8, device=DEV)
    traces = []
    for _ in range(2):
        outs = [torch.empty((4, wl.hidden), dtype=torch.bfloat16, device=DEV) for _ in layers]
        _forward(p, layers, 0, xd, outs, wsb)
        traces.append(p.trace())
        torch.cuda.synchronize()
        for i, L in enumerate(layers):
            ws = L["ws"]
            _, _, ref = gemm.mlp_f64(x, ws[0].raw(), None, ws[1].raw(), None, "bf16", wl.hidden, wl.intermediate)
            assert_close_rows(values(outs[i]), ref, what=f"gather_lds={gather_lds} layer {i}")
    g = "begin" if gate == swr.GATE_BEGIN else "done"
    assert all(t == osch.expected_trace(0, n_layers, gate=g) for t in traces)
    assert osch.check_trace(traces) == []
    # the last layer's slot holds the oracle's flat buffer bit for bit
    last = slot_b if (n_layers - 1) % 2 else slot_a
    plan = olayout.plan_layer([(o, i, d) for _, o, i, d in wl.weights], wl.n_chunks)
    t_ref, _ = olayout.pack_layer(plan, [w.raw() for w in layers[-1]["ws"]])
    assert np.array_equal(last.cpu().numpy(), t_ref)
    p.close()


@pytest.mark.parametrize("engine,gate,gather_lds,one_queue", [(swr.ENGINE_KERNEL, swr.GATE_DONE, 0, False),
                                                              (swr.ENGINE_DMA, swr.GATE_DONE, 0, False),
                                                              (swr.ENGINE_KERNEL, swr.GATE_BEGIN, 0, False),
                                                              (swr.ENGINE_KERNEL, swr.GATE_DONE, 57344, False),
                                                              (swr.ENGINE_KERNEL, swr.GATE_AFTER, 0, False),
                                                              (swr.ENGINE_KERNEL, swr.GATE_AFTER, 0, True)])
def test_forward_captured_in_a_graph(engine, gate, gather_lds, one_queue):
    """weight_sharding, CUDA graph section: the launch/wait sequence is fixed,
    so one forward (gathers on the side stream, MLPs on the compute stream)
    can be captured once and replayed.  Between replays both slots and every
    output are overwritten with garbage by eager work; each replay must
    gather again and reproduce the oracle's outputs."""
    note(f"graph capture engine={engine} gate={gate} gather_lds={gather_lds} one_queue={one_queue}")
    wl = synth.TINY
    n_layers = 4
    layers = _layers(wl, n_layers, wl.n_chunks)
    total = layers[0]["lay"]["total_bytes"]
    slot_a = torch.empty(total, dtype=torch.uint8, device=DEV)
    slot_b = torch.empty(total, dtype=torch.uint8, device=DEV)
    compute = torch.cuda.Stream()
    side = compute if one_queue else torch.cuda.Stream()
    p = swr.Planner(0, n_layers, compute, side, slot_a, slot_b)
    for i, L in enumerate(layers):
        p.set_layer(i, L["chunks"], L["lay"]["chunk_bytes"])
    p.set_copy_engine(engine)
    p.set_gate(gate)
    p.set_gather_lds(gather_lds)
    x = synth.activations(synth.seed_for(1, 0, 50), 4, wl.hidden)
    xd = bf16(x)
    outs = [torch.empty((4, wl.hidden), dtype=torch.bfloat16, device=DEV) for _ in layers]
    wsb = torch.empty(swr.mlp_workspace_bytes(4, wl.hidden, wl.intermediate, "bf16"), dtype=torch.uint8, device=DEV)
    refs = []
    for L in layers:
        ws = L["ws"]
        refs.append(gemm.mlp_f64(x, ws[0].raw(), None, ws[1].raw(), None, "bf16", wl.hidden, wl.intermediate)[2])
    with torch.cuda.stream(compute):
        _forward(p, layers, 0, xd, outs, wsb)  # eager warm-up on the same streams
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=compute):
        _forward(p, layers, 0, xd, outs, wsb)
    # the captured sequence is the model's
    assert p.trace() == osch.expected_trace(0, n_layers, gate=GATE_NAMES[gate])
    torch.cuda.synchronize()
    for rep in range(4):
        slot_a.fill_(0xFF)  # 0xFFFF as bf16 is NaN: a replay that skipped a gather would show it
        slot_b.fill_(0xFF)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(n_layers):
            assert_close_rows(values(outs[i]), refs[i], what=f"graph replay {rep} layer {i}")
    p.close()


@pytest.mark.parametrize("start,n_layers,cyclic", [(0, 3, False), (1, 4, True), (0, 2, False)])
def test_begin_gate_on_gpu(start, n_layers, cyclic):
    """SWR_GATE_BEGIN: each gather after the first waits for the compute stream
    to begin the previous layer.  The trace equals the oracle's model of that
    gate, passes the happens-before checker, and every layer's outputs equal
    the oracle's with the compute stream delayed."""
    note(f"planner begin gate start={start} layers={n_layers} cyclic={cyclic}")
    wl = synth.TINY
    layers = _layers(wl, n_layers, wl.n_chunks)
    total = layers[0]["lay"]["total_bytes"]
    slot_a = torch.empty(total, dtype=torch.uint8, device=DEV)
    slot_b = torch.empty(total, dtype=torch.uint8, device=DEV)
    p = swr.Planner(start, start + n_layers, torch.cuda.current_stream(), torch.cuda.Stream(), slot_a, slot_b)
    for i, L in enumerate(layers):
        p.set_layer(start + i, L["chunks"], L["lay"]["chunk_bytes"])
    p.set_gate(swr.GATE_BEGIN)
    with pytest.raises(swr.SwrError) as e:
        p.set_gate(5)
    assert e.value.code == swr.E_INVALID
    if cyclic:
        p.set_cyclic(True)
    p.set_timing(64)  # the begin record doubles as the layer's timing start
    x = synth.activations(synth.seed_for(1, 0, 50), 4, wl.hidden)
    xd = bf16(x)
    wsb = torch.empty(swr.mlp_workspace_bytes(4, wl.hidden, wl.intermediate, "bf16"), dtype=torch.uint8, device=DEV)
    a = torch.randn(2048, 2048, device=DEV)

    def delay():
        for _ in range(4):
            torch.mm(a, a)

    traces, outs_all = [], []
    for _ in range(3):
        outs = [torch.empty((4, wl.hidden), dtype=torch.bfloat16, device=DEV) for _ in layers]
        _forward(p, layers, start, xd, outs, wsb, delay)
        traces.append(p.trace())
        outs_all.append(outs)
    torch.cuda.synchronize()
    end = start + n_layers
    if cyclic:
        assert traces[0] == osch.expected_trace(start, end, prefetch_next=True, gate="begin")
        assert all(t == osch.expected_trace(start, end, prefetched=True, prefetch_next=True, gate="begin")
                   for t in traces[1:])
    else:
        assert all(t == osch.expected_trace(start, end, gate="begin") for t in traces)
    assert osch.check_trace(traces) == []
    for outs in outs_all:
        for i, L in enumerate(layers):
            ws = L["ws"]
            _, _, ref = gemm.mlp_f64(x, ws[0].raw(), None, ws[1].raw(), None, "bf16", wl.hidden, wl.intermediate)
            assert_close_rows(values(outs[i]), ref, what=f"begin gate layer {start + i}")
    times = p.layer_times()
    assert len(times) == 3 * n_layers and all(t > 0 for t in times)
    assert len(p.gather_times()) == (3 * n_layers + 1 if cyclic else 3 * n_layers)
    p.set_timing(0)
    p.set_cyclic(False)
    p.close()


def test_set_gate_refused_while_a_gather_is_pending():
    wl = synth.TINY
    layers = _layers(wl, 2, wl.n_chunks)
    total = layers[0]["lay"]["total_bytes"]
    slot = torch.empty(total, dtype=torch.uint8, device=DEV)
    p = swr.Planner(0, 2, torch.cuda.current_stream(), torch.cuda.Stream(), slot, torch.empty_like(slot))
    for i, L in enumerate(layers):
        p.set_layer(i, L["chunks"], L["lay"]["chunk_bytes"])
    p.set_gate(swr.GATE_BEGIN)
    p.reset()
    p.pre_dispatch(0)
    p.maybe_dispatch(1)  # pending until wait_ready_once(0)
    with pytest.raises(swr.SwrError) as e:
        p.set_gate(swr.GATE_DONE)
    assert e.value.code == swr.E_SEQUENCE
    p.wait_ready_once(0)
    p.update_done_event(0)
    p.wait_ready_once(1)
    p.update_done_event(1)
    p.set_gate(swr.GATE_DONE)
    torch.cuda.synchronize()
    p.close()


@pytest.mark.parametrize("start,n_layers,cyclic,one_queue", [(0, 3, False, False), (1, 4, True, False),
                                                             (0, 2, True, True), (1, 5, False, True)])
def test_after_gate_on_gpu(start, n_layers, cyclic, one_queue):
    """SWR_GATE_AFTER: the gather of layer l+1 waits for done(l) and is enqueued
    by update_done_event(l); with one queue (compute == side) the waits are
    implied by queue order.  The trace equals the oracle's model of that gate,
    passes the happens-before checker, and every layer's outputs equal the
    oracle's with the compute stream delayed; the slots hold the oracle's T."""
    note(f"planner after gate start={start} layers={n_layers} cyclic={cyclic} one_queue={one_queue}")
    wl = synth.TINY
    layers = _layers(wl, n_layers, wl.n_chunks)
    total = layers[0]["lay"]["total_bytes"]
    slot_a = torch.empty(total, dtype=torch.uint8, device=DEV)
    slot_b = torch.empty(total, dtype=torch.uint8, device=DEV)
    compute = torch.cuda.current_stream()
    side = compute if one_queue else torch.cuda.Stream()
    p = swr.Planner(start, start + n_layers, compute, side, slot_a, slot_b)
    for i, L in enumerate(layers):
        p.set_layer(start + i, L["chunks"], L["lay"]["chunk_bytes"])
    p.set_gate(swr.GATE_AFTER)
    if cyclic:
        p.set_cyclic(True)
    p.set_timing(64)
    x = synth.activations(synth.seed_for(1, 0, 50), 4, wl.hidden)
    xd = bf16(x)
    wsb = torch.empty(swr.mlp_workspace_bytes(4, wl.hidden, wl.intermediate, "bf16"), dtype=torch.uint8, device=DEV)
    a = torch.randn(2048, 2048, device=DEV)

    def delay():
        for _ in range(4):
            torch.mm(a, a)

    traces, outs_all = [], []
    for f in range(3):
        # the second forward runs with timing paused: it records no timing events
        p.pause_timing(f == 1)
        outs = [torch.empty((4, wl.hidden), dtype=torch.bfloat16, device=DEV) for _ in layers]
        _forward(p, layers, start, xd, outs, wsb, delay)
        traces.append(p.trace())
        outs_all.append(outs)
    p.pause_timing(False)
    torch.cuda.synchronize()
    end = start + n_layers
    if cyclic:
        assert traces[0] == osch.expected_trace(start, end, prefetch_next=True, gate="after")
        assert all(t == osch.expected_trace(start, end, prefetched=True, prefetch_next=True, gate="after")
                   for t in traces[1:])
    else:
        assert all(t == osch.expected_trace(start, end, gate="after") for t in traces)
    assert osch.check_trace(traces) == []
    for outs in outs_all:
        for i, L in enumerate(layers):
            ws = L["ws"]
            _, _, ref = gemm.mlp_f64(x, ws[0].raw(), None, ws[1].raw(), None, "bf16", wl.hidden, wl.intermediate)
            assert_close_rows(values(outs[i]), ref, what=f"after gate layer {start + i}")
    # timed: the layers of forwards 0 and 2, and the gathers dispatched during
    # them (in cyclic mode forward 0 also gathers its own first layer)
    times = p.layer_times()
    assert len(times) == 2 * n_layers and all(t > 0 for t in times)
    assert len(p.gather_times()) == (2 * n_layers + 1 if cyclic else 2 * n_layers)
    # the last layer's slot holds the oracle's flat buffer bit for bit
    last = slot_b if (n_layers - 1) % 2 else slot_a
    plan = olayout.plan_layer([(o, i, d) for _, o, i, d in wl.weights], wl.n_chunks)
    if not cyclic:
        t_ref, _ = olayout.pack_layer(plan, [w.raw() for w in layers[-1]["ws"]])
        assert np.array_equal(last.cpu().numpy(), t_ref)
    p.set_timing(0)
    p.set_cyclic(False)
    p.close()


@pytest.mark.parametrize("gate,one_queue,engine", [(swr.GATE_DONE, False, swr.ENGINE_KERNEL),
                                                   (swr.GATE_AFTER, True, swr.ENGINE_KERNEL),
                                                   (swr.GATE_BEGIN, False, swr.ENGINE_KERNEL),
                                                   (swr.GATE_DONE, False, swr.ENGINE_DMA)])
def test_first_layer_prefetch_outside_a_graph(gate, one_queue, engine):
    """weight_sharding, CUDA graph section: the first layer is gathered on a
    dedicated stream outside the captured forward, overlapping the previous
    replay's last layers, and the graph waits for it.  The eager sequence
    equals the oracle's model (prologue prefetch, then forward + prefetch) and
    passes its race checker; then one forward is captured and replayed, each
    replay's prefetch for the next enqueued right behind it while the replay
    (with its layers delayed) still runs.  Every replay's outputs equal the
    oracle's; slot 1 and the outputs are clobbered between replays."""
    note(f"first-layer prefetch stream gate={gate} one_queue={one_queue} engine={engine}")
    wl = synth.TINY
    n_layers = 4
    layers = _layers(wl, n_layers, wl.n_chunks)
    total = layers[0]["lay"]["total_bytes"]
    slot_a = torch.empty(total, dtype=torch.uint8, device=DEV)
    slot_b = torch.empty(total, dtype=torch.uint8, device=DEV)
    compute = torch.cuda.Stream()
    side = compute if one_queue else torch.cuda.Stream()
    pf = torch.cuda.Stream()
    p = swr.Planner(0, n_layers, compute, side, slot_a, slot_b)
    for i, L in enumerate(layers):
        p.set_layer(i, L["chunks"], L["lay"]["chunk_bytes"])
    p.set_gate(gate)
    p.set_copy_engine(engine)
    with pytest.raises(swr.SwrError) as e:
        p.set_first_prefetch(compute)
    assert e.value.code == swr.E_INVALID
    p.set_first_prefetch(pf)
    with pytest.raises(swr.SwrError) as e:
        p.set_cyclic(True)
    assert e.value.code == swr.E_INVALID
    p.reset()
    with pytest.raises(swr.SwrError) as e:
        p.pre_dispatch(0)  # no prefetch yet
    assert e.value.code == swr.E_SEQUENCE
    x = synth.activations(synth.seed_for(1, 0, 50), 4, wl.hidden)
    xd = bf16(x)
    outs = [torch.full((4, wl.hidden), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in layers]
    wsb = torch.empty(swr.mlp_workspace_bytes(4, wl.hidden, wl.intermediate, "bf16"), dtype=torch.uint8, device=DEV)
    refs = [gemm.mlp_f64(x, L["ws"][0].raw(), None, L["ws"][1].raw(), None, "bf16", wl.hidden, wl.intermediate)[2]
            for L in layers]
    a = torch.randn(2048, 2048, device=DEV)

    def delay():
        for _ in range(2):
            torch.mm(a, a)

    g = GATE_NAMES[gate]
    # eager: prologue prefetch, then forward + the next forward's prefetch
    traces = []
    p.prefetch_first()
    traces.append(p.trace())
    with torch.cuda.stream(compute):
        for _ in range(2):
            _forward(p, layers, 0, xd, outs, wsb, delay)
            p.prefetch_first()
            traces.append(p.trace())
    torch.cuda.synchronize()
    want = osch.expected_trace(0, n_layers, gate=g, first_external=True) + osch.prefetch_first_ops(0, n_layers)
    # (the refused pre_dispatch above came after a reset, which the prologue trace begins with)
    assert traces[0] == [("record_start", "compute", -1, -1)] + osch.prefetch_first_ops(0, n_layers)
    assert all(t == want for t in traces[1:])
    assert osch.check_trace(traces) == []
    for i in range(n_layers):
        assert_close_rows(values(outs[i]), refs[i], what=f"eager prefetch layer {i}")
    # captured: the forward (without its first gather) as a graph; the prefetch outside it
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=compute):
        _forward(p, layers, 0, xd, outs, wsb, delay)
    assert p.trace() == osch.expected_trace(0, n_layers, gate=g, first_external=True)
    torch.cuda.synchronize()
    for rep in range(4):
        graph.replay()
        p.prefetch_first()  # for the next replay, while this one still runs
        torch.cuda.synchronize()
        for i in range(n_layers):
            assert_close_rows(values(outs[i]), refs[i], what=f"replay {rep} layer {i}")
        slot_b.fill_(0xFF)  # slot 0 now holds the next replay's first layer
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
    _, gathers = p.counters()
    # prologue prefetch; two eager forwards (n - 1 gathers + a prefetch each); the
    # gathers enqueued while capturing; one prefetch per replay
    assert gathers == 1 + 2 * n_layers + (n_layers - 1) + 4
    p.set_first_prefetch(None)
    p.close()
