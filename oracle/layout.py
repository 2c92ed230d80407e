"""Flat layout of one layer's weights -- oracle (test infrastructure only).

Follows "weight_sharding" (zdszero.github.io), section on one AllGather per
layer (the flat layout), its four numbered steps:

1. the layer's weights are laid end to end, in order, in one logical byte
   buffer T; every item starts on a 16-byte boundary and the total length is
   padded up to a multiple of 16*N;
2. T is cut into N equal byte chunks, chunk i = T[i*C:(i+1)*C], C = |T|/N;
3. one gather puts the N chunks back together into the full T;
4. weight j is a reinterpretation of T[o_j : o_j + s_j] -- no copy.

Readings where the page is silent: padding bytes are zero; offsets are
relative to the start of T; items keep the caller's order.
"""
from __future__ import annotations

import numpy as np

ELEM_BYTES = {"bf16": 2, "fp8_e4m3fn": 1}
ITEM_ALIGN = 16


def align_up(x: int, a: int) -> int:
    return -(-int(x) // int(a)) * int(a)


def plan_layer(weights: list[tuple[int, int, str]], n_chunks: int) -> dict:
    """Offset table and sizes for one layer (step 1 and 2).

    ``weights`` is a list of (out_features, in_features, dtype).  Returns a
    dict with per-item ``offsets`` and ``sizes`` (bytes), ``payload`` (end
    of the last item), ``total`` (|T|) and ``chunk`` (C).
    """
    if n_chunks < 1:
        raise ValueError("n_chunks must be >= 1")
    offsets, sizes = [], []
    end = 0
    for out_f, in_f, dtype in weights:
        start = align_up(end, ITEM_ALIGN)
        size = int(out_f) * int(in_f) * ELEM_BYTES[dtype]
        offsets.append(start)
        sizes.append(size)
        end = start + size
    total = align_up(end, ITEM_ALIGN * n_chunks)
    return {
        "offsets": offsets,
        "sizes": sizes,
        "payload": end,
        "total": total,
        "chunk": total // n_chunks,
        "n_chunks": int(n_chunks),
        "dtypes": [w[2] for w in weights],
        "shapes": [(int(w[0]), int(w[1])) for w in weights],
    }


def pack_layer(plan: dict, raw_weights: list[np.ndarray]) -> tuple[np.ndarray, list[np.ndarray]]:
    """Build T from the weights' raw bytes and cut it into N chunks (steps 1-2).

    Returns (T, chunks); chunk i is a copy of T[i*C:(i+1)*C]."""
    t = np.zeros(plan["total"], dtype=np.uint8)
    for off, size, raw in zip(plan["offsets"], plan["sizes"], raw_weights):
        b = np.ascontiguousarray(raw).view(np.uint8).reshape(-1)
        if b.size != size:
            raise ValueError(f"weight has {b.size} bytes, plan says {size}")
        t[off:off + size] = b
    c = plan["chunk"]
    chunks = [t[i * c:(i + 1) * c].copy() for i in range(plan["n_chunks"])]
    return t, chunks


def reassemble(chunks: list[np.ndarray]) -> np.ndarray:
    """Step 3 on one device: the gathered buffer is the chunks in rank order."""
    return np.concatenate([np.asarray(c, dtype=np.uint8).reshape(-1) for c in chunks])


def view(slot: np.ndarray, plan: dict, j: int) -> np.ndarray:
    """Step 4: weight j as an array over the slot's bytes (no copy).

    BF16 items come back as uint16 bit patterns, FP8 items as uint8 codes,
    both shaped [out_features, in_features]."""
    off, size = plan["offsets"][j], plan["sizes"][j]
    out_f, in_f = plan["shapes"][j]
    raw = slot[off:off + size]
    if plan["dtypes"][j] == "bf16":
        return raw.view(np.uint16).reshape(out_f, in_f)
    return raw.reshape(out_f, in_f)


def remote_bytes(plan: dict, self_rank: int = 0) -> int:
    """Bytes a rank receives from its peers in one gather: every chunk but its own."""
    del self_rank  # every rank owns exactly one chunk of C bytes
    return (plan["n_chunks"] - 1) * plan["chunk"]


# ---------------------------------------------------------------- row shards
#
# "weight_sharding", loading section: a tensor-parallel loader gives each of
# N ranks a row shard of every weight (for a merged linear such as gate_up,
# a row shard of each sub-block: the gate rows and the up rows are split
# separately); weights whose rows do not divide by N stay whole on every
# rank.  The one-time re-layout turns those row shards into the flat chunks
# of the layout above.  Plainest reading: the re-layout's result is exactly
# pack_layer of the whole weights, so the oracle rebuilds each whole weight
# from its row shards and packs.


def row_shards(raw: np.ndarray, out_features: int, in_features: int, dtype: str, sub_rows: list[int],
               n: int) -> list[np.ndarray]:
    """Rank r's row shard of one weight: for each sub-block b in order, its
    rows [r*R_b/n, (r+1)*R_b/n), as contiguous bytes."""
    if sum(sub_rows) != out_features or any(r % n for r in sub_rows):
        raise ValueError("every sub-block's rows must split evenly over the ranks")
    rows = np.asarray(raw, dtype=np.uint8).reshape(out_features, in_features * ELEM_BYTES[dtype])
    starts = np.cumsum([0] + list(sub_rows))
    out = []
    for r in range(n):
        parts = [rows[starts[b] + r * (sub_rows[b] // n):starts[b] + (r + 1) * (sub_rows[b] // n)]
                 for b in range(len(sub_rows))]
        out.append(np.ascontiguousarray(np.concatenate(parts)).reshape(-1))
    return out


def unshard_rows(shards: list[np.ndarray], out_features: int, in_features: int, dtype: str,
                 sub_rows: list[int]) -> np.ndarray:
    """The whole weight's bytes from its n row shards (inverse of row_shards)."""
    n = len(shards)
    row_bytes = in_features * ELEM_BYTES[dtype]
    per_rank = [np.asarray(s, dtype=np.uint8).reshape(-1, row_bytes) for s in shards]
    blocks = []
    first = 0  # first row of sub-block b inside a rank's shard
    for rb in sub_rows:
        k = rb // n
        blocks.extend(per_rank[r][first:first + k] for r in range(n))
        first += k
    whole = np.concatenate(blocks) if blocks else np.zeros((0, row_bytes), np.uint8)
    assert whole.shape[0] == out_features
    return whole.reshape(-1)


def redistribute(plan: dict, weights: list[dict]) -> list[np.ndarray]:
    """Flat chunks from per-weight row shards.  ``weights[j]`` holds
    ``out_features``, ``in_features``, ``dtype`` and either ``whole`` (bytes of
    a weight that stays whole) or ``shards`` plus ``sub_rows``."""
    raws = []
    for w in weights:
        if "whole" in w:
            raws.append(np.asarray(w["whole"], dtype=np.uint8).reshape(-1))
        else:
            raws.append(unshard_rows(w["shards"], w["out_features"], w["in_features"], w["dtype"], w["sub_rows"]))
    return pack_layer(plan, raws)[1]
