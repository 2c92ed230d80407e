"""Seeded synthetic inputs for the flat-weight reassembly path.

This module only draws numbers and encodes them into the storage formats the
path consumes (BF16 bit patterns, FP8 E4M3FN codes with a per-output-row fp32
scale).  It holds none of the method's arithmetic: no layout, no packing, no
reassembly, no GEMM.  It is imported by the CPU oracle tests, the GPU parity
tests, the benchmark and the smoke check, so that both sides of every parity
check see byte-identical inputs.

Recipe
------
* Generator: ``numpy.random.Generator(PCG64(SeedSequence([seed, block])))``
  per block of ``BLOCK_ROWS`` rows, standard normal in fp32, times ``sigma``.
  Drawing per row block keeps large tensors cheap to build on many threads
  and keeps a tensor's first rows independent of how many rows it has.
* Seed: ``10000*config + 100*layer + tensor_id``; tensor_id 0 is gate_up,
  1 is down, 2.. are projections in listed order, 50+j is the activation
  matrix for the j-th distinct input width.
* Weights are N(0, 0.02); activations are N(0, 1).
* BF16 encoding: round-to-nearest-even from fp32.
* FP8 encoding (synthetic-weight quantiser, not compared against anything):
  per output row, ``scale = max_k |W[row, k]| / 448`` (1.0 for an all-zero
  row), codes are ``E4M3FN(W / scale)`` rounded to nearest even after
  clamping to the largest finite magnitude 448.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_ROWS = 256
FP8_MAX = 448.0

BF16 = "bf16"
FP8 = "fp8_e4m3fn"
ELEM_BYTES = {BF16: 2, FP8: 1}


def seed_for(config: int, layer: int, tensor_id: int) -> int:
    return 10000 * int(config) + 100 * int(layer) + int(tensor_id)


def _threads() -> int:
    env = os.environ.get("SWR_SYNTH_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(seed: int, rows: int, cols: int, sigma: float = 1.0) -> np.ndarray:
    """fp32 [rows, cols] ~ N(0, sigma^2), drawn per block of BLOCK_ROWS rows."""
    out = np.empty((rows, cols), dtype=np.float32)
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS

    def fill(b: int) -> None:
        r0 = b * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, b])))
        blk = out[r0:r1]
        g.standard_normal(out=blk.reshape(-1), dtype=np.float32)
        if sigma != 1.0:
            blk *= np.float32(sigma)

    if nblk <= 2 or rows * cols < (1 << 22):
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> BF16 bit patterns (uint16), round to nearest, ties to even.

    The inputs here are finite normal draws, so no NaN handling is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def fp8_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """fp32 [rows, cols] -> (E4M3FN codes uint8 [rows, cols], fp32 scale [rows])."""
    import torch  # the reference float8 encoder lives in torch

    amax = np.abs(x).max(axis=1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = (t / torch.from_numpy(scale)[:, None]).clamp_(-FP8_MAX, FP8_MAX)
    codes = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


@dataclass
class Weight:
    """One synthetic weight: raw bytes [out, in*elem] plus the fp32 row scale."""

    out_features: int
    in_features: int
    dtype: str
    data: np.ndarray  # uint16 [out, in] for bf16, uint8 [out, in] for fp8
    scale: np.ndarray | None  # fp32 [out] for fp8, None for bf16

    @property
    def nbytes(self) -> int:
        return self.out_features * self.in_features * ELEM_BYTES[self.dtype]

    def raw(self) -> np.ndarray:
        """The weight's bytes as a flat uint8 array (row-major, out x in)."""
        return np.ascontiguousarray(self.data).view(np.uint8).reshape(-1)


def weight(seed: int, out_features: int, in_features: int, dtype: str, sigma: float = 0.02) -> Weight:
    w = normal_f32(seed, out_features, in_features, sigma)
    if dtype == BF16:
        return Weight(out_features, in_features, dtype, bf16_bits(w), None)
    if dtype == FP8:
        codes, scale = fp8_rows(w)
        return Weight(out_features, in_features, dtype, codes, scale)
    raise ValueError(f"unknown dtype {dtype!r}")


def activations(seed: int, m: int, k: int) -> np.ndarray:
    """BF16 bit patterns [m, k] of N(0, 1) tokens."""
    return bf16_bits(normal_f32(seed, m, k, 1.0))


# --------------------------------------------------------------------------
# Workload shapes.  Weight lists are (name, out_features, in_features, dtype)
# in the order the layer packs them.
# --------------------------------------------------------------------------


@dataclass
class Workload:
    config: int
    name: str
    weights: list[tuple[str, int, int, str]]
    n_chunks: int
    layers: int
    tokens: list[int]
    hidden: int = 0
    intermediate: int = 0
    extra: dict = field(default_factory=dict)

    def layer_weights(self, layer: int, sigma: float = 0.02) -> list[Weight]:
        return [
            weight(seed_for(self.config, layer, tid), o, i, dt, sigma)
            for tid, (_, o, i, dt) in enumerate(self.weights)
        ]


TINY = Workload(
    config=1,
    name="tiny-mlp-h128-i256-n4",
    weights=[("gate_up", 512, 128, BF16), ("down", 128, 256, BF16), ("proj", 100, 128, BF16)],
    n_chunks=4,
    layers=1,
    tokens=[4],
    hidden=128,
    intermediate=256,
)

# Same as TINY but with items whose byte sizes are not multiples of 16, so
# item and total padding both occur; the FP8 item has no MLP role.
TINY_PADDED = Workload(
    config=11,
    name="tiny-padded-n4",
    weights=[("gate_up", 512, 128, BF16), ("odd", 100, 127, BF16), ("down", 128, 256, BF16),
             ("fp8_small", 3, 5, FP8)],
    n_chunks=4,
    layers=1,
    tokens=[4],
    hidden=128,
    intermediate=256,
)

SHARED_EXPERT_DECODE = Workload(
    config=2,
    name="shared-expert-mlp-decode-h6144-i14336-fp8",
    weights=[("gate_up", 28672, 6144, FP8), ("down", 6144, 14336, FP8)],
    n_chunks=16,
    layers=8,
    tokens=[1, 8, 32, 64],
    hidden=6144,
    intermediate=14336,
)

ATTN_PROJECTIONS = Workload(
    config=3,
    name="replicated-attn-projections-fp8",
    weights=[("p0", 24576, 7168, FP8), ("p1", 8192, 7168, FP8), ("p2", 7168, 8192, FP8),
             ("p3", 4096, 7168, FP8), ("p4", 1000, 7168, FP8), ("p5", 7168, 3072, FP8),
             ("p6", 3072, 7168, FP8), ("p7", 1536, 7168, FP8)],
    n_chunks=16,
    layers=16,
    tokens=[16],
)

SHARED_EXPERT_PREFILL = Workload(
    config=4,
    name="shared-expert-mlp-prefill-h6144-i14336-fp8",
    weights=SHARED_EXPERT_DECODE.weights,
    n_chunks=16,
    layers=4,
    tokens=[4096, 16384],
    hidden=6144,
    intermediate=14336,
)

# X[B, D] @ W[D, F]; W is drawn as [D, F] and stored transposed (out x in).
SHARDED_MATMUL = Workload(
    config=5,
    name="sharded-matmul-b2048-d8192-f28672-bf16",
    weights=[("w_t", 28672, 8192, BF16)],
    n_chunks=8,
    layers=1,
    tokens=[2048],
    extra={"B": 2048, "D": 8192, "F": 28672, "shards": 8},
)


def sharded_matmul_inputs(b: int, d: int, f: int, config: int = 5) -> tuple[np.ndarray, np.ndarray]:
    """(X bf16 bits [b, d], W^T bf16 bits [f, d]) with W drawn as [d, f]."""
    x = activations(seed_for(config, 0, 50), b, d)
    w = normal_f32(seed_for(config, 0, 0), d, f, 0.02)
    w_t = np.ascontiguousarray(bf16_bits(w).T)
    return x, w_t


WORKLOADS = {w.config: w for w in (TINY, TINY_PADDED, SHARED_EXPERT_DECODE, ATTN_PROJECTIONS,
                                     SHARED_EXPERT_PREFILL, SHARDED_MATMUL)}
