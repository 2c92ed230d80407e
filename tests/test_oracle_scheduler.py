"""Pins for the lookahead / ping-pong launch sequence (weight-sharding page,
sections on lookahead and ping-pong slots, on the SGLang implementation and
on CUDA graphs).  The happens-before checker is independent of the sequence
generator; mistakes planted in the sequence must be caught by it."""
import pytest

from oracle import scheduler as sch


@pytest.mark.parametrize("start,end", [(0, 1), (0, 2), (1, 5), (1, 93), (3, 11)])
def test_expected_trace_is_race_free(start, end):
    t = sch.expected_trace(start, end)
    assert sch.check_trace([t]) == []
    assert sch.check_trace([t, t, t]) == []  # back-to-back forwards


def test_slots_alternate_and_two_suffice():
    t = sch.expected_trace(1, 9)
    copies = [(op[2], op[3]) for op in t if op[0] == "copy"]
    assert copies == [(layer, (layer - 1) % 2) for layer in range(1, 9)]
    assert {s for _, s in copies} == {0, 1}
    waits = [op for op in t if op[0] == "wait_ready"]
    assert [w[2] for w in waits] == list(range(1, 9))


def test_gate_waits_for_layer_two_back():
    t = sch.expected_trace(0, 6)
    for i, op in enumerate(t):
        if op[0] == "copy" and op[2] >= 2:
            assert t[i - 1] == ("wait_done", "side", op[2] - 2, -1)


def test_missing_gate_is_a_race():
    t = [op for op in sch.expected_trace(0, 4) if op[0] != "wait_done"]
    problems = sch.check_trace([t])
    assert any("race" in p for p in problems)


def test_missing_ready_wait_is_caught():
    t = sch.expected_trace(0, 4)
    bad = [op for op in t if not (op[0] == "wait_ready" and op[2] == 2)]
    assert sch.check_trace([bad])


def test_double_ready_wait_is_caught():
    t = sch.expected_trace(0, 3)
    i = t.index(("wait_ready", "compute", 1, 1))
    bad = t[:i + 1] + [t[i]] + t[i + 1:]
    assert any("2 times" in p for p in sch.check_trace([bad]))


def test_next_forward_needs_start_event():
    # Without the start record, the next forward's first gathers race with the
    # previous forward's last computes on the same slots.
    t = sch.expected_trace(0, 4)
    no_start = [op for op in t if op[0] != "record_start"]
    assert sch.check_trace([t, no_start])


def test_wrong_slot_is_caught():
    t = sch.expected_trace(0, 4)
    bad = [(n, s, layer, 1 - slot) if (n == "wait_ready" and layer == 3) else (n, s, layer, slot)
           for n, s, layer, slot in t]
    assert sch.check_trace([bad])


def test_empty_range():
    assert sch.expected_trace(5, 5) == [("record_start", "compute", -1, -1)]


@pytest.mark.parametrize("start,end", [(0, 2), (1, 9), (0, 16)])
def test_cyclic_prefetch_is_race_free(start, end):
    first = sch.expected_trace(start, end, prefetched=False, prefetch_next=True)
    mid = sch.expected_trace(start, end, prefetched=True, prefetch_next=True)
    last = sch.expected_trace(start, end, prefetched=True, prefetch_next=False)
    assert sch.check_trace([first, mid, mid, last]) == []
    # the next forward issues no gather of its first layer
    assert not any(op[0] == "copy" and op[2] == start for op in mid)


def test_cyclic_prefetch_needs_its_gate_and_even_layers():
    first = sch.expected_trace(0, 4, prefetch_next=True)
    mid = sch.expected_trace(0, 4, prefetched=True)
    i = first.index(("copy_next", "side", 0, 0))
    no_gate = first[:i - 1] + first[i:]
    assert any("race" in p for p in sch.check_trace([no_gate, mid]))
    # a forward that believes its first layer was prefetched when it was not
    assert sch.check_trace([sch.expected_trace(0, 4), mid])
    with pytest.raises(ValueError):
        sch.expected_trace(0, 3, prefetch_next=True)


@pytest.mark.parametrize("start,end", [(0, 1), (0, 2), (1, 5), (3, 11)])
def test_begin_gate_is_race_free(start, end):
    t = sch.expected_trace(start, end, gate="begin")
    assert sch.check_trace([t, t, t]) == []
    # the same gathers and slots as the page's gate, in the same order
    copies = lambda tr: [op for op in tr if op[0] in ("copy", "copy_next")]
    assert copies(t) == copies(sch.expected_trace(start, end))


@pytest.mark.parametrize("start,end", [(0, 2), (1, 9)])
def test_begin_gate_cyclic_is_race_free(start, end):
    first = sch.expected_trace(start, end, prefetch_next=True, gate="begin")
    mid = sch.expected_trace(start, end, prefetched=True, prefetch_next=True, gate="begin")
    last = sch.expected_trace(start, end, prefetched=True, gate="begin")
    assert sch.check_trace([first, mid, mid, last]) == []


def test_begin_gate_mistakes_are_caught():
    t = sch.expected_trace(0, 6, gate="begin")
    no_wait = [op for op in t if op[0] != "wait_begin"]
    assert any("race" in p for p in sch.check_trace([no_wait]))
    # gating the gather of l+1 on the begin of l-1 lets it overwrite the slot layer l-1 still reads
    early = [("wait_begin", s, layer - 1, x) if (n == "wait_begin" and layer >= 1) else (n, s, layer, x)
             for n, s, layer, x in t]
    assert any("race" in p for p in sch.check_trace([early]))
    with pytest.raises(ValueError):
        sch.expected_trace(0, 4, gate="ready")


@pytest.mark.parametrize("start,end", [(0, 1), (0, 2), (1, 5), (3, 11)])
def test_after_gate_is_race_free(start, end):
    t = sch.expected_trace(start, end, gate="after")
    assert sch.check_trace([t, t, t]) == []
    # the same gathers into the same slots as the page's gate, in the same order
    copies = lambda tr: [op for op in tr if op[0] in ("copy", "copy_next")]
    assert copies(t) == copies(sch.expected_trace(start, end))
    # each gather after the first follows the done record of the layer before it
    for i, op in enumerate(t):
        if op[0] == "copy" and op[2] > start:
            assert t[i - 1] == ("wait_done", "side", op[2] - 1, -1)
            assert t[i - 2] == ("record_done", "compute", op[2] - 1, -1)


@pytest.mark.parametrize("start,end", [(0, 2), (1, 9)])
def test_after_gate_cyclic_is_race_free(start, end):
    first = sch.expected_trace(start, end, prefetch_next=True, gate="after")
    mid = sch.expected_trace(start, end, prefetched=True, prefetch_next=True, gate="after")
    last = sch.expected_trace(start, end, prefetched=True, gate="after")
    assert sch.check_trace([first, mid, mid, last]) == []
    assert first[-3:] == [("wait_done", "side", end - 1, -1), ("copy_next", "side", start, 0),
                          ("record_ready", "side", start, -1)]


def test_after_gate_mistakes_are_caught():
    t = sch.expected_trace(0, 6, gate="after")
    no_wait = [op for op in t if op[0] != "wait_done"]
    assert any("race" in p for p in sch.check_trace([no_wait]))
    # a layer that does not wait for its gather reads whatever the slot holds
    no_ready = [op for op in t if op != ("wait_ready", "compute", 3, 1)]
    assert sch.check_trace([no_ready])



@pytest.mark.parametrize("gate", ["done", "begin", "after"])
@pytest.mark.parametrize("start,end", [(0, 1), (0, 2), (1, 4), (0, 5), (3, 11)])
def test_dedicated_first_prefetch_is_race_free(gate, start, end):
    """The first layer gathered on its own stream outside the forward: a
    prologue prefetch, then forwards each followed by the prefetch for the next."""
    fwd = sch.expected_trace(start, end, gate=gate, first_external=True)
    pf = sch.prefetch_first_ops(start, end)
    assert sch.check_trace([pf, fwd + pf, fwd + pf, fwd]) == []
    # the forward itself gathers every layer but its first, into the same slots
    copies = [op for op in fwd if op[0] == "copy"]
    assert [(op[2], op[3]) for op in copies] == [(layer, (layer - start) % 2) for layer in range(start + 1, end)]
    l0 = sch.last_slot0_reader(start, end)
    assert (l0 - start) % 2 == 0 and l0 + 2 >= end
    assert fwd[fwd.index(("record_done", "compute", l0, -1)) + 1] == ("record_free", "compute", l0, 0)


def test_dedicated_first_prefetch_mistakes_are_caught():
    fwd = sch.expected_trace(0, 4, first_external=True)
    pf = sch.prefetch_first_ops(0, 4)
    # the prefetch without its gate overwrites slot 0 while layer 2 reads it
    no_wait = [op for op in pf if op[0] != "wait_free"]
    assert any("race" in p for p in sch.check_trace([pf, fwd + no_wait, fwd]))
    # a forward that never records the free event gives the prefetch nothing to wait for
    no_free = [op for op in fwd if op[0] != "record_free"]
    assert any("race" in p for p in sch.check_trace([pf, no_free + pf, fwd]))
    # freeing slot 0 after layer 0 instead of its last reader, layer 2
    early = [("record_free", "compute", 0, 0) if op[0] == "record_free" else op for op in fwd]
    early.remove(("record_free", "compute", 0, 0))
    early.insert(early.index(("record_done", "compute", 0, -1)) + 1, ("record_free", "compute", 0, 0))
    assert any("race" in p for p in sch.check_trace([pf, early + pf, fwd]))
    # a forward that does not wait for the prefetch reads whatever slot 0 holds
    no_ready = [op for op in fwd if op != ("wait_ready", "compute", 0, 0)]
    assert sch.check_trace([pf, no_ready])
    with pytest.raises(ValueError):
        sch.expected_trace(0, 4, first_external=True, prefetch_next=True)
