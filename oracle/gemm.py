"""Projection, MLP and sharded-matmul references -- oracle (test infrastructure only).

Conventions (weight-sharding page, core abstraction: W is out x in):
  Y[m, o] = s[o] * sum_k X[m, k] * W[o, k]
with X in BF16, W in BF16 (s = 1) or FP8 E4M3FN with a per-output-row fp32
scale s, everything evaluated in float64 and rounded once to BF16 at the end.

MLP (vLLM PR #50656 report, test code: the fused gate_up weight is the gate
rows followed by the up rows, and the activation is SiLU of the first half
times the second half; the mini-sglang tensor-parallel chapter, Megatron
split, names the same gate_up -> SiLU x up -> down chain):
  G = X @ dec(W_gate_up)^T * s_gu          (kept in float64, not rounded)
  h = bf16( silu(G[:, :I]) * G[:, I:] )
  Y = bf16( (h @ dec(W_down)^T) * s_d )

FP8-activation MLP (an option beyond the pages; numerics.quantize_rows_e4m3):
  X is quantised per token, G = (dec(q_X) @ dec(W_gate_up)^T) * s_X[:, None] * s_gu,
  h = bf16( silu(G[:, :I]) * G[:, I:] ) is quantised per token in turn, and
  Y = bf16( (dec(q_h) @ dec(W_down)^T) * s_h[:, None] * s_d ).

Sharded matmul (copecc.github.io sharded-matrices notes, "local matmul"
cases): X[B, D] @ W[D, F].  Splitting F (the output columns) leaves the
contraction whole, so every shard is a finished slice of Y (case 1);
splitting D on both operands gives partial sums that add up to Y (case 3).
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f64, decode_weight, f64_to_bf16_bits, fp8_to_f64, quantize_rows_e4m3, silu


def proj_f64(x_bits: np.ndarray, w_raw: np.ndarray, dtype: str, out_f: int, in_f: int,
             scale: np.ndarray | None = None) -> np.ndarray:
    """Unrounded Y = (X @ dec(W)^T) * s[None, :] in float64."""
    x = bf16_to_f64(x_bits).reshape(-1, in_f)
    w = decode_weight(w_raw, dtype, out_f, in_f)
    y = x @ w.T
    if scale is not None:
        y = y * np.asarray(scale, dtype=np.float32).astype(np.float64)[None, :]
    return y


def proj(x_bits, w_raw, dtype, out_f, in_f, scale=None) -> np.ndarray:
    """BF16 bit patterns of the projection output [M, out]."""
    return f64_to_bf16_bits(proj_f64(x_bits, w_raw, dtype, out_f, in_f, scale))


def proj_rows_bruteforce(x_bits, w_raw, dtype, out_f, in_f, scale, rows, cols) -> np.ndarray:
    """Unrounded outputs Y[rows, cols] by explicit loops (no BLAS), one dot at a time."""
    x = bf16_to_f64(x_bits).reshape(-1, in_f)
    w = decode_weight(w_raw, dtype, out_f, in_f)
    res = np.empty((len(rows), len(cols)), dtype=np.float64)
    for a, m in enumerate(rows):
        for b, o in enumerate(cols):
            acc = 0.0
            xm, wo = x[m], w[o]
            for k in range(in_f):
                acc += float(xm[k]) * float(wo[k])
            s = 1.0 if scale is None else float(np.float32(scale[o]))
            res[a, b] = acc * s
    return res


def mlp_f64(x_bits, w_gu_raw, s_gu, w_d_raw, s_d, dtype, hidden, inter):
    """Returns (G float64 [M, 2I], h bf16 bits [M, I], Y float64 unrounded [M, H])."""
    g = proj_f64(x_bits, w_gu_raw, dtype, 2 * inter, hidden, s_gu)
    with np.errstate(over="ignore"):
        h_bits = f64_to_bf16_bits(silu(g[:, :inter]) * g[:, inter:])
    y = proj_f64(h_bits, w_d_raw, dtype, hidden, inter, s_d)
    return g, h_bits, y


def mlp(x_bits, w_gu_raw, s_gu, w_d_raw, s_d, dtype, hidden, inter) -> np.ndarray:
    """BF16 bit patterns of the MLP output [M, H]."""
    return f64_to_bf16_bits(mlp_f64(x_bits, w_gu_raw, s_gu, w_d_raw, s_d, dtype, hidden, inter)[2])


def mlp_intermediate_slice_f64(x_bits, w_gu_raw, s_gu, w_d_raw, s_d, dtype, hidden, inter, lo, hi):
    """Unrounded MLP contribution of intermediate indices [lo, hi): the gate rows
    lo..hi, the matching up rows I+lo..I+hi and the down columns lo..hi (the
    per-rank partial of the PR report's tensor-parallel shared expert)."""
    w_gu = np.asarray(w_gu_raw).reshape(2 * inter, -1)
    rows = np.r_[lo:hi, inter + lo:inter + hi]
    sub_gu = np.ascontiguousarray(w_gu[rows])
    sub_s_gu = None if s_gu is None else np.asarray(s_gu)[rows]
    w_d = np.asarray(w_d_raw).reshape(hidden, -1)
    elem = w_d.shape[1] // inter
    sub_d = np.ascontiguousarray(w_d[:, lo * elem:hi * elem])
    _, _, y = mlp_f64(x_bits, sub_gu, sub_s_gu, sub_d, s_d, dtype, hidden, hi - lo)
    return y


def proj_fp8act_f64(x: np.ndarray, w_raw, out_f: int, in_f: int, scale) -> tuple:
    """FP8 weights, FP8 activations: X (float values of bf16 tokens) is
    quantised per token; returns (q_x, s_x, unrounded Y float64 [M, out])."""
    q_x, s_x = quantize_rows_e4m3(np.asarray(x, dtype=np.float64).reshape(-1, in_f))
    w = decode_weight(w_raw, "fp8_e4m3fn", out_f, in_f)
    y = (fp8_to_f64(q_x) @ w.T) * s_x.astype(np.float64)[:, None]
    if scale is not None:
        y = y * np.asarray(scale, dtype=np.float32).astype(np.float64)[None, :]
    return q_x, s_x, y


def mlp_fp8act_f64(x_bits, w_gu_raw, s_gu, w_d_raw, s_d, hidden, inter):
    """FP8 weights and FP8 activations.  Returns (q_x, s_x, G float64 [M, 2I],
    h bf16 bits [M, I], q_h, s_h, Y float64 unrounded [M, H])."""
    q_x, s_x, g = proj_fp8act_f64(bf16_to_f64(x_bits), w_gu_raw, 2 * inter, hidden, s_gu)
    with np.errstate(over="ignore"):
        h_bits = f64_to_bf16_bits(silu(g[:, :inter]) * g[:, inter:])
    q_h, s_h, y = proj_fp8act_f64(bf16_to_f64(h_bits), w_d_raw, hidden, inter, s_d)
    return q_x, s_x, g, h_bits, q_h, s_h, y


# ---------------------------------------------------------------- sharded matmul

def matmul_f64(x_bits: np.ndarray, w_t_bits: np.ndarray) -> np.ndarray:
    """Y = X @ W with W stored transposed (W^T is [F, D], BF16 bits)."""
    return bf16_to_f64(x_bits) @ bf16_to_f64(w_t_bits).T


def column_shards(w_t_bits: np.ndarray, n: int) -> list[np.ndarray]:
    """Split F into n equal blocks: row blocks of W^T (a dim-0 split of out x in)."""
    f = w_t_bits.shape[0]
    if f % n:
        raise ValueError("F must divide evenly")
    step = f // n
    return [w_t_bits[i * step:(i + 1) * step] for i in range(n)]


def contraction_shards(x_bits: np.ndarray, w_t_bits: np.ndarray, n: int):
    """Split D into n equal blocks on both operands: (X[:, blk], W^T[:, blk]) pairs."""
    d = x_bits.shape[1]
    if d % n:
        raise ValueError("D must divide evenly")
    step = d // n
    return [(x_bits[:, i * step:(i + 1) * step], w_t_bits[:, i * step:(i + 1) * step]) for i in range(n)]


def concat_columns(parts: list[np.ndarray]) -> np.ndarray:
    return np.concatenate(parts, axis=1)


def sum_partials(parts: list[np.ndarray]) -> np.ndarray:
    """Partial results added in shard order 0..n-1."""
    acc = np.zeros_like(np.asarray(parts[0], dtype=np.float64))
    for p in parts:
        acc = acc + np.asarray(p, dtype=np.float64)
    return acc


def row_tolerance(y_ref: np.ndarray, rel: float = 1e-2) -> np.ndarray:
    """Per-row bound rel * max(1, max |y_ref| over the row), shaped [M, 1]."""
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y_ref.ndim == 1:
        y_ref = y_ref[None, :]
    return rel * np.maximum(1.0, np.abs(y_ref).max(axis=1, keepdims=True))
