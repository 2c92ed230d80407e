"""Memory and transfer accounting -- oracle (test infrastructure only).

Weight-sharding page (zdszero.github.io), cost section:
* transfer: with a ring gather every rank receives about (N-1)/N * S bytes
  per layer per forward, S being the layer's gathered bytes.  On one device
  the chunks are all local, so the count is exact: every chunk but the
  rank's own, (N-1) * C = (N-1)/N * |T|.
* memory: replicated weights R become R/N resident per rank plus two
  full-layer slots, R/N + 2 * max_l |T_l|.

Readings: S and |T_l| are the padded flat sizes and R = sum_l |T_l|, which
makes both formulas exact rather than approximate.
"""
from __future__ import annotations


def transfer_bytes(total: int, n_chunks: int) -> int:
    if total % n_chunks:
        raise ValueError("|T| must be a multiple of N")
    return (n_chunks - 1) * (total // n_chunks)


def slot_bytes(totals: list[int]) -> int:
    """Both ping-pong slots together: two times the largest layer."""
    return 2 * max(totals) if totals else 0


def resident_per_rank(totals: list[int], n_chunks: int) -> int:
    """One rank's chunks over all layers: sum_l C_l = R / N."""
    return sum(t // n_chunks for t in totals)


def weight_shard_memory(totals: list[int], n_chunks: int) -> int:
    """R/N + 2 * max_l |T_l| per rank."""
    return resident_per_rank(totals, n_chunks) + slot_bytes(totals)


def replicated_memory(totals: list[int]) -> int:
    return sum(totals)
