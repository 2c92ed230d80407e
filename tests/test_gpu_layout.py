"""GPU parity: pack, reassembly and views are bit-exact against the oracle.

weight_sharding (zdszero.github.io), flat layout steps 1-4: T holds the
weights at 16-byte aligned offsets with zero padding, chunk i is
T[i*C:(i+1)*C], the gathered slot equals T and every view equals the bytes
of its weight.
"""
import numpy as np
import pytest
import torch

import sharded_weight_reassembly_amd as swr
import synth
from oracle import layout as olayout

from gpu_util import DEV, note, u8

pytestmark = pytest.mark.gpu


def _pack_and_gather(ws_shapes, weights, n, stream=None):
    views, lay = swr.plan_layer([(o, i, d) for (o, i, d) in ws_shapes], n)
    src = [u8(w.raw()) for w in weights]
    c = lay["chunk_bytes"]
    # chunk buffers prefilled with garbage: pack must write every byte, padding included
    chunks = [torch.full((c,), 0xA5, dtype=torch.uint8, device=DEV) for _ in range(n)]
    swr.pack_layer(lay, views, src, chunks, stream=stream)
    slot = torch.full((lay["total_bytes"] + 4096,), 0x5A, dtype=torch.uint8, device=DEV)
    remote = swr.reassemble_into_slot(chunks, c, slot, stream=stream)
    torch.cuda.synchronize()
    return views, lay, chunks, slot, remote


CASES = [
    (synth.TINY.weights, 4),
    (synth.TINY_PADDED.weights, 4),
    (synth.TINY_PADDED.weights, 3),
    (synth.TINY_PADDED.weights, 16),
    ([("a", 1, 1, synth.FP8)], 1),
    ([("a", 7, 3, synth.FP8), ("b", 5, 9, synth.BF16), ("c", 1, 1, synth.FP8), ("d", 33, 17, synth.BF16)], 5),
    ([("a", 7, 3, synth.FP8)] * 64, 64),
]


@pytest.mark.parametrize("shapes,n", CASES)
def test_pack_reassemble_bit_exact(shapes, n):
    note(f"pack/reassemble shapes={[(o, i, d) for _, o, i, d in shapes][:4]} n={n}")
    ws = [synth.weight(synth.seed_for(11, 0, t), o, i, d) for t, (_, o, i, d) in enumerate(shapes)]
    shp = [(o, i, d) for _, o, i, d in shapes]
    views, lay, chunks, slot, remote = _pack_and_gather(shp, ws, n)
    plan = olayout.plan_layer(shp, n)
    t_ref, chunks_ref = olayout.pack_layer(plan, [w.raw() for w in ws])
    for i in range(n):
        assert np.array_equal(chunks[i].cpu().numpy(), chunks_ref[i]), f"chunk {i}"
    got = slot.cpu().numpy()
    assert np.array_equal(got[:lay["total_bytes"]], t_ref)
    assert (got[lay["total_bytes"]:] == 0x5A).all(), "copy wrote past |T|"
    assert remote == olayout.remote_bytes(plan)
    for j, w in enumerate(ws):
        v = swr.view(slot, views[j])
        assert v.data_ptr() == slot.data_ptr() + views[j]["offset"]  # zero copy
        assert np.array_equal(v.contiguous().view(torch.uint8).cpu().numpy().reshape(-1), w.raw())


def test_self_rank_and_repeated_gathers():
    note("self_rank/repeat")
    shp = [(o, i, d) for _, o, i, d in synth.TINY.weights]
    ws = synth.TINY.layer_weights(0)
    views, lay, chunks, slot, remote = _pack_and_gather(shp, ws, 4)
    c = lay["chunk_bytes"]
    for r in range(4):
        assert swr.reassemble_into_slot(chunks, c, slot, self_rank=r) == 3 * c
    torch.cuda.synchronize()
    ref = torch.cat(chunks)
    assert torch.equal(slot[:lay["total_bytes"]], ref)


def test_gate_and_ready_events():
    note("gate/ready events")
    shp = [(o, i, d) for _, o, i, d in synth.TINY.weights]
    ws = synth.TINY.layer_weights(0)
    views, lay, chunks, slot, _ = _pack_and_gather(shp, ws, 4)
    side = torch.cuda.Stream()
    gate, ready = torch.cuda.Event(), torch.cuda.Event()
    slot2 = torch.zeros_like(slot)
    gate.record(torch.cuda.current_stream())
    swr.reassemble_into_slot(chunks, lay["chunk_bytes"], slot2, stream=side, gate=gate, ready=ready)
    torch.cuda.current_stream().wait_event(ready)
    assert torch.equal(slot2, slot.masked_fill(torch.arange(slot.numel(), device=DEV) >= lay["total_bytes"], 0))


def test_full_size_shared_expert_layer():
    """One 264 MB shared-expert layer at N=16, bit-exact against the oracle's T."""
    wl = synth.SHARED_EXPERT_DECODE
    note("full-size pack/reassemble 264 MB N=16")
    ws = wl.layer_weights(0)
    shp = [(o, i, d) for _, o, i, d in wl.weights]
    views, lay, chunks, slot, remote = _pack_and_gather(shp, ws, wl.n_chunks)
    plan = olayout.plan_layer(shp, wl.n_chunks)
    t_ref, _ = olayout.pack_layer(plan, [w.raw() for w in ws])
    got = slot[:lay["total_bytes"]].cpu().numpy()
    assert np.array_equal(got, t_ref)
    assert remote == 15 * 16515072
    # the chunks are the slot's pieces, byte for byte
    for i in (0, 7, 15):
        assert torch.equal(chunks[i], slot[i * lay["chunk_bytes"]:(i + 1) * lay["chunk_bytes"]])


def test_pack_rejects_misaligned_source():
    shp = [(4, 4, "bf16")]
    views, lay = swr.plan_layer(shp, 2)
    src = torch.zeros(64, dtype=torch.uint8, device=DEV)
    chunks = [torch.zeros(lay["chunk_bytes"], dtype=torch.uint8, device=DEV) for _ in range(2)]
    with pytest.raises(swr.SwrError) as e:
        swr.pack_layer(lay, views, [src.data_ptr() + 4], chunks)
    assert e.value.code == swr.E_ALIGN


@pytest.mark.parametrize("shapes,n", [CASES[1], CASES[3], CASES[6]])
def test_dma_gather_bit_exact(shapes, n):
    """The DMA-engine gather writes exactly the copy kernel's bytes: T, and
    nothing past |T|."""
    note(f"dma gather shapes={[(o, i, d) for _, o, i, d in shapes][:4]} n={n}")
    ws = [synth.weight(synth.seed_for(11, 1, t), o, i, d) for t, (_, o, i, d) in enumerate(shapes)]
    shp = [(o, i, d) for _, o, i, d in shapes]
    views, lay, chunks, _, _ = _pack_and_gather(shp, ws, n)
    plan = olayout.plan_layer(shp, n)
    t_ref, _ = olayout.pack_layer(plan, [w.raw() for w in ws])
    slot = torch.full((lay["total_bytes"] + 4096,), 0x5A, dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream()
    gate, ready = torch.cuda.Event(), torch.cuda.Event()
    gate.record(torch.cuda.current_stream())
    remote = swr.reassemble_into_slot_dma(chunks, lay["chunk_bytes"], slot, stream=side, gate=gate, ready=ready)
    torch.cuda.current_stream().wait_event(ready)
    got = slot.cpu().numpy()
    assert np.array_equal(got[:lay["total_bytes"]], t_ref)
    assert (got[lay["total_bytes"]:] == 0x5A).all(), "copy wrote past |T|"
    assert remote == olayout.remote_bytes(plan)


def test_dma_gather_full_size_layer():
    """One 264 MB shared-expert layer gathered by the DMA engines equals T."""
    wl = synth.SHARED_EXPERT_DECODE
    note("full-size DMA gather 264 MB N=16")
    ws = wl.layer_weights(1)
    shp = [(o, i, d) for _, o, i, d in wl.weights]
    views, lay, chunks, slot, _ = _pack_and_gather(shp, ws, wl.n_chunks)
    slot2 = torch.zeros_like(slot)
    swr.reassemble_into_slot_dma(chunks, lay["chunk_bytes"], slot2)
    torch.cuda.synchronize()
    assert torch.equal(slot2[:lay["total_bytes"]], slot[:lay["total_bytes"]])
