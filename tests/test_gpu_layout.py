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



def _shard_specs(shapes, ws, n, merged=()):
    """Row shards as the oracle's split rule makes them: weights listed in
    `merged` are [gate; up] (two equal sub-blocks); weights whose rows do not
    split over n stay whole."""
    specs, oracle_ws = [], []
    for j, ((_, o, i, d), w) in enumerate(zip(shapes, ws)):
        sub = [o // 2, o // 2] if j in merged else [o]
        if all(r % n == 0 for r in sub):
            sh = olayout.row_shards(w.raw(), o, i, d, sub, n)
            specs.append(dict(sub_rows=sub, src=[u8(x) for x in sh]))
            oracle_ws.append(dict(out_features=o, in_features=i, dtype=d, sub_rows=sub, shards=sh))
        else:
            specs.append(dict(replicated=True, src=[u8(w.raw())]))
            oracle_ws.append(dict(out_features=o, in_features=i, dtype=d, whole=w.raw()))
    return specs, oracle_ws


@pytest.mark.parametrize("shapes,n,merged", [
    (synth.TINY_PADDED.weights, 4, (0,)),   # [100 x 127] bf16: 254-byte rows; [3 x 5] fp8 stays whole
    (synth.TINY_PADDED.weights, 2, (0,)),
    (synth.TINY_PADDED.weights, 1, ()),
    (synth.TINY.weights, 4, (0,)),
])
def test_redistribute_row_shards_bit_exact(shapes, n, merged):
    """weight_sharding, loading section: flat chunks written from the loader's
    row shards equal the oracle's pack of the whole weights, byte for byte."""
    note(f"redistribute shapes={[(o, i, d) for _, o, i, d in shapes]} n={n}")
    ws = [synth.weight(synth.seed_for(18, 0, t), o, i, d) for t, (_, o, i, d) in enumerate(shapes)]
    shp = [(o, i, d) for _, o, i, d in shapes]
    views, lay = swr.plan_layer(shp, n)
    specs, oracle_ws = _shard_specs(shapes, ws, n, merged)
    chunks = [torch.full((lay["chunk_bytes"],), 0xA5, dtype=torch.uint8, device=DEV) for _ in range(n)]
    swr.redistribute_row_shards(lay, views, specs, chunks)
    torch.cuda.synchronize()
    plan = olayout.plan_layer(shp, n)
    ref = olayout.redistribute(plan, oracle_ws)
    _, packed = olayout.pack_layer(plan, [w.raw() for w in ws])
    for i in range(n):
        got = chunks[i].cpu().numpy()
        assert np.array_equal(got, ref[i]), f"chunk {i}"
        assert np.array_equal(got, packed[i]), f"chunk {i} vs pack"


@pytest.mark.parametrize("wl,merged", [(synth.ATTN_PROJECTIONS, ()), (synth.SHARED_EXPERT_DECODE, (0,))])
def test_redistribute_full_size_layer(wl, merged):
    """A full-size layer at N=16: the projection layer ([1000 x 7168] stays
    whole: 1000 rows do not split over 16 ranks) and the shared expert with
    gate_up split per sub-block.  Both the chunks written from the row shards
    and the chunks swr_pack_layer writes from the whole weights equal the
    oracle's chunks of T, byte for byte."""
    note(f"redistribute full-size {wl.name}")
    n = wl.n_chunks
    ws = wl.layer_weights(0)
    shp = [(o, i, d) for _, o, i, d in wl.weights]
    views, lay = swr.plan_layer(shp, n)
    specs, oracle_ws = _shard_specs(wl.weights, ws, n, merged)
    chunks = [torch.full((lay["chunk_bytes"],), 0xA5, dtype=torch.uint8, device=DEV) for _ in range(n)]
    swr.redistribute_row_shards(lay, views, specs, chunks)
    del specs
    packed = [torch.full((lay["chunk_bytes"],), 0x5A, dtype=torch.uint8, device=DEV) for _ in range(n)]
    swr.pack_layer(lay, views, [u8(w.raw()) for w in ws], packed)
    torch.cuda.synchronize()
    plan = olayout.plan_layer(shp, n)
    ref = olayout.redistribute(plan, oracle_ws)
    del oracle_ws
    for i in range(n):
        assert np.array_equal(chunks[i].cpu().numpy(), ref[i]), f"redistributed chunk {i}"
        assert np.array_equal(packed[i].cpu().numpy(), ref[i]), f"packed chunk {i}"


def test_redistribute_leading_padding_is_zero():
    """Views whose first item starts after byte 0 (a caller-built table): the
    bytes before it are padding and are written as zero, as swr_pack_layer
    writes them; the shards are never read before their start."""
    note("redistribute with a leading gap")
    shapes = [("a", 8, 16, synth.BF16), ("b", 12, 32, synth.FP8)]
    n = 4
    ws = [synth.weight(synth.seed_for(19, 0, t), o, i, d) for t, (_, o, i, d) in enumerate(shapes)]
    shp = [(o, i, d) for _, o, i, d in shapes]
    views, lay = swr.plan_layer(shp, n)
    gap = 64  # move both items 64 bytes up; |T| still covers them
    for v in views:
        v["offset"] += gap
    lay = dict(lay, payload_bytes=lay["payload_bytes"] + gap)
    total = -(-lay["payload_bytes"] // (16 * n)) * 16 * n
    lay = dict(lay, total_bytes=total, chunk_bytes=total // n)
    specs, _ = _shard_specs(shapes, ws, n)
    chunks = [torch.full((lay["chunk_bytes"],), 0xA5, dtype=torch.uint8, device=DEV) for _ in range(n)]
    swr.redistribute_row_shards(lay, views, specs, chunks)
    packed = [torch.full((lay["chunk_bytes"],), 0x5A, dtype=torch.uint8, device=DEV) for _ in range(n)]
    swr.pack_layer(lay, views, [u8(w.raw()) for w in ws], packed)
    torch.cuda.synchronize()
    # the oracle's T for this table: zeros, with each weight's bytes at its offset
    t_ref = np.zeros(total, np.uint8)
    for v, w in zip(views, ws):
        t_ref[v["offset"]:v["offset"] + v["nbytes"]] = w.raw().view(np.uint8).reshape(-1)
    got = np.concatenate([c.cpu().numpy() for c in chunks])
    assert np.array_equal(got, t_ref)
    assert np.array_equal(np.concatenate([c.cpu().numpy() for c in packed]), t_ref)
