"""Pins for the oracle's flat layout, pack, reassembly and views.

Worked numbers follow from the flat-layout rule of the weight-sharding page
(zdszero.github.io, section on one AllGather per layer, steps 1-4): items
start on 16-byte boundaries, |T| is padded to a multiple of 16*N, C = |T|/N.
The arithmetic for each case is written out next to it.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _plan(ws, n):
    return layout.plan_layer(ws, n)


def test_tiny_mlp_n4():
    # gate_up 512*128*2 = 131072 B at 0; down 128*256*2 = 65536 B at 131072;
    # proj 100*128*2 = 25600 B at 196608; end 222208 = 3472 * 64, no padding.
    p = _plan([(512, 128, "bf16"), (128, 256, "bf16"), (100, 128, "bf16")], 4)
    assert p["offsets"] == [0, 131072, 196608]
    assert p["total"] == 222208 and p["chunk"] == 55552
    assert p["payload"] == p["total"]


@pytest.mark.parametrize("n,total,chunk", [(4, 222080, 55520), (3, 222048, 74016), (16, 222208, 13888)])
def test_tiny_padded(n, total, chunk):
    # 131072 B at 0; [100x127] bf16 = 25400 B at 131072 -> ends 156472, next
    # item at 156480 (8 pad bytes); [128x256] bf16 = 65536 B -> ends 222016;
    # fp8 [3x5] = 15 B -> ends 222031.  Rounded up to 64 / 48 / 256.
    p = _plan([(512, 128, "bf16"), (100, 127, "bf16"), (128, 256, "bf16"), (3, 5, "fp8_e4m3fn")], n)
    assert p["offsets"] == [0, 131072, 156480, 222016]
    assert p["sizes"] == [131072, 25400, 65536, 15]
    assert p["payload"] == 222031
    assert p["total"] == total and p["chunk"] == chunk


def test_shared_expert_layer():
    # 28672*6144 = 176,160,768 B; 6144*14336 = 88,080,384 B; sum 264,241,152
    # = 16 * 16,515,072 and a multiple of 256: no padding at N=16.
    p = _plan([(28672, 6144, "fp8_e4m3fn"), (6144, 14336, "fp8_e4m3fn")], 16)
    assert p["offsets"] == [0, 176160768]
    assert p["total"] == 264241152 and p["chunk"] == 16515072


def test_projection_layer():
    shapes = [(24576, 7168), (8192, 7168), (7168, 8192), (4096, 7168), (1000, 7168),
              (7168, 3072), (3072, 7168), (1536, 7168)]
    p = _plan([(o, i, "fp8_e4m3fn") for o, i in shapes], 16)
    assert p["offsets"] == [0, 176160768, 234881024, 293601280, 322961408, 330129408,
                            352149504, 374169600]
    assert p["total"] == 385179648 and p["chunk"] == 24073728


def test_pages_shared_expert_bytes():
    # The PR report prints 176.2 MB + 88.1 MB = 264.2 MB per layer at one byte
    # per element; the plan's item sizes must round to those figures.
    fig = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))["shared_expert_bytes"]
    (go, gi), (do, di) = fig["gate_up_shape"], fig["down_shape"]
    p = _plan([(go, gi, "fp8_e4m3fn"), (do, di, "fp8_e4m3fn")], 16)
    assert round(p["sizes"][0] / 1e6, 1) == fig["gate_up_MB"]
    assert round(p["sizes"][1] / 1e6, 1) == fig["down_MB"]
    assert round(p["total"] / 1e6, 1) == fig["layer_MB"]
    assert round(p["total"] * fig["layers"] / 2 ** 30, 1) == fig["total_GiB"]


def test_chunk_straddles_weights():
    # Chunk boundaries depend only on |T| and N: in the tiny layer at N=4,
    # chunk 2 = [111104, 166656) holds the tail of gate_up and the head of down.
    p = _plan([(512, 128, "bf16"), (128, 256, "bf16"), (100, 128, "bf16")], 4)
    c = p["chunk"]
    lo, hi = 2 * c, 3 * c
    assert (lo, hi) == (111104, 166656)
    assert lo < p["offsets"][1] < hi
    lo3, hi3 = 3 * c, 4 * c
    assert lo3 < p["offsets"][2] < hi3


def _bytewise_pack(ws, raws, n):
    """Build T one byte at a time from the rule, without the oracle's slicing."""
    t = []
    for (o, i, dt), raw in zip(ws, raws):
        while len(t) % 16:
            t.append(0)
        t.extend(int(b) for b in raw)
    while len(t) % (16 * n):
        t.append(0)
    return bytes(t)


shapes = st.lists(st.tuples(st.integers(1, 9), st.integers(1, 11), st.sampled_from(["bf16", "fp8_e4m3fn"])),
                  min_size=1, max_size=5)


@settings(max_examples=60, deadline=None)
@given(ws=shapes, n=st.sampled_from([1, 2, 3, 4, 5, 16]), seed=st.integers(0, 2 ** 16))
def test_plan_pack_bruteforce(ws, n, seed):
    rng = np.random.default_rng(seed)
    raws = [rng.integers(1, 256, size=o * i * layout.ELEM_BYTES[dt], dtype=np.uint8) for o, i, dt in ws]
    p = _plan(ws, n)
    ref = _bytewise_pack(ws, raws, n)
    t, chunks = layout.pack_layer(p, raws)
    assert bytes(t) == ref
    assert p["total"] == len(ref) and p["total"] % (16 * n) == 0
    assert p["total"] - p["payload"] < 16 * n
    for j in range(len(ws)):
        assert p["offsets"][j] % 16 == 0
        if j:
            prev_end = p["offsets"][j - 1] + p["sizes"][j - 1]
            assert prev_end <= p["offsets"][j] < prev_end + 16
    assert len(chunks) == n and all(len(c) == p["chunk"] for c in chunks)
    for i, c in enumerate(chunks):
        assert bytes(c) == ref[i * p["chunk"]:(i + 1) * p["chunk"]]
    slot = layout.reassemble(chunks)
    assert bytes(slot) == ref
    for j, (o, i, dt) in enumerate(ws):
        v = layout.view(slot, p, j)
        assert v.shape == (o, i)
        assert v.tobytes() == raws[j].tobytes()
    assert layout.remote_bytes(p) == (n - 1) * p["chunk"]


def test_padding_is_zero():
    ws = [(100, 127, "bf16"), (3, 5, "fp8_e4m3fn")]
    raws = [np.full(100 * 127 * 2, 0xAB, np.uint8), np.full(15, 0xCD, np.uint8)]
    p = _plan(ws, 4)
    t, _ = layout.pack_layer(p, raws)
    mask = np.zeros(p["total"], bool)
    for off, size in zip(p["offsets"], p["sizes"]):
        mask[off:off + size] = True
    assert (t[~mask] == 0).all() and (~mask).sum() == p["total"] - sum(p["sizes"])


# ---------------------------------------------------------------- row shards

def test_row_shards_follow_the_split_rule():
    """Rank r holds rows [r*R/n, (r+1)*R/n) of every sub-block, in order; a merged
    [gate; up] weight is split per sub-block, not as one block."""
    out_f, in_f, n = 8, 3, 2
    raw = np.arange(out_f * in_f, dtype=np.uint8)
    shards = layout.row_shards(raw, out_f, in_f, "fp8_e4m3fn", [4, 4], n)
    rows = raw.reshape(out_f, in_f)
    assert np.array_equal(shards[0].reshape(-1, in_f), rows[[0, 1, 4, 5]])
    assert np.array_equal(shards[1].reshape(-1, in_f), rows[[2, 3, 6, 7]])
    single = layout.row_shards(raw, out_f, in_f, "fp8_e4m3fn", [8], n)
    assert np.array_equal(single[0].reshape(-1, in_f), rows[:4])
    with pytest.raises(ValueError):
        layout.row_shards(raw, out_f, in_f, "fp8_e4m3fn", [5, 3], n)


@pytest.mark.parametrize("sub_rows,n", [([12], 1), ([12], 4), ([6, 6], 3), ([8, 4, 12], 4)])
def test_unshard_inverts_row_shards(sub_rows, n):
    out_f, in_f = sum(sub_rows), 7
    raw = np.random.default_rng(n).integers(0, 256, out_f * in_f * 2, dtype=np.uint8)
    shards = layout.row_shards(raw, out_f, in_f, "bf16", sub_rows, n)
    assert sum(s.size for s in shards) == raw.size
    assert np.array_equal(layout.unshard_rows(shards, out_f, in_f, "bf16", sub_rows), raw)


def test_redistribute_equals_pack_of_whole_weights():
    shp = [(16, 5, "bf16"), (12, 3, "fp8_e4m3fn"), (7, 9, "bf16")]
    n = 4
    plan = layout.plan_layer(shp, n)
    rng = np.random.default_rng(3)
    raws = [rng.integers(0, 256, o * i * layout.ELEM_BYTES[d], dtype=np.uint8) for o, i, d in shp]
    ws = [dict(out_features=16, in_features=5, dtype="bf16", sub_rows=[8, 8],
               shards=layout.row_shards(raws[0], 16, 5, "bf16", [8, 8], n)),
          dict(out_features=12, in_features=3, dtype="fp8_e4m3fn", sub_rows=[12],
               shards=layout.row_shards(raws[1], 12, 3, "fp8_e4m3fn", [12], n)),
          dict(out_features=7, in_features=9, dtype="bf16", whole=raws[2])]  # 7 rows do not split over 4 ranks
    chunks = layout.redistribute(plan, ws)
    _, ref = layout.pack_layer(plan, raws)
    assert all(np.array_equal(a, b) for a, b in zip(chunks, ref))
