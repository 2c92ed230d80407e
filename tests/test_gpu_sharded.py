"""GPU: sharded-matmul layout equivalence on one device (copecc.github.io,
sharded-matrices notes, local matmul cases 1 and 3).

X[B, D] @ W[D, F] computed three ways:
* full:    one proj_forward over W^T [F, D];
* columns: F split into 8 row blocks of W^T, each written into its column
           slice of Y -- the contraction is untouched, so this must be bitwise
           equal to the full product from the same kernel;
* K split: D split into 8 blocks on both operands, each giving an fp32
           partial, added in shard order by swr_sum_partials.
All three agree with the oracle's float64 product within the row bar.
"""
import numpy as np
import pytest
import torch

import sharded_weight_reassembly_amd as swr
import synth
from oracle import gemm

from gpu_util import DEV, assert_close_rows, bf16, note, values

pytestmark = pytest.mark.gpu


def _three_ways(x_bits, w_t_bits, shards):
    b, d = x_bits.shape
    f = w_t_bits.shape[0]
    xd = bf16(x_bits)
    wd = bf16(w_t_bits)
    y_full = torch.empty((b, f), dtype=torch.bfloat16, device=DEV)
    swr.proj_forward(wd, "bf16", None, f, d, xd, y_full)
    fs = f // shards
    y_cols = torch.empty((b, f), dtype=torch.bfloat16, device=DEV)
    for j in range(shards):
        swr.proj_forward(wd[j * fs:(j + 1) * fs], "bf16", None, fs, d, xd, y_cols[:, j * fs:(j + 1) * fs], ldy=f)
    ds = d // shards
    parts = []
    for j in range(shards):
        w_k = wd[:, j * ds:(j + 1) * ds].contiguous()  # what rank j would hold
        p = torch.empty((b, f), dtype=torch.float32, device=DEV)
        swr.proj_forward(w_k, "bf16", None, f, ds, xd[:, j * ds:(j + 1) * ds], p, ldx=d)
        parts.append(p)
    y_sum = torch.empty((b, f), dtype=torch.bfloat16, device=DEV)
    swr.sum_partials(parts, y_sum)
    torch.cuda.synchronize()
    return y_full, y_cols, y_sum, parts


def test_small_sharded_matmul():
    note("sharded matmul small")
    b, d, f = 96, 1024, 1536
    x, w_t = synth.sharded_matmul_inputs(b, d, f, config=15)
    y_full, y_cols, y_sum, parts = _three_ways(x, w_t, 8)
    assert torch.equal(y_full.view(torch.int16), y_cols.view(torch.int16))
    ref = gemm.matmul_f64(x, w_t)
    assert_close_rows(values(y_full), ref, what="full")
    assert_close_rows(values(y_sum), ref, what="K-split sum")
    # every partial against the oracle's partial
    ds = d // 8
    for j, p in enumerate(parts):
        ref_j = gemm.matmul_f64(np.ascontiguousarray(x[:, j * ds:(j + 1) * ds]),
                                np.ascontiguousarray(w_t[:, j * ds:(j + 1) * ds]))
        assert_close_rows(values(p), ref_j, what=f"partial {j}")


def test_sum_partials_order_and_tail():
    note("sum_partials")
    rng = np.random.default_rng(3)
    for n, count in [(1, 5), (3, 1001), (8, 4096), (64, 37)]:
        parts_np = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
        parts = [torch.from_numpy(p).to(DEV) for p in parts_np]
        out = torch.empty(count, dtype=torch.float32, device=DEV)
        swr.sum_partials(parts, out)
        torch.cuda.synchronize()
        acc = parts_np[0].copy()
        for p in parts_np[1:]:
            acc = (acc + p).astype(np.float32)  # fp32 adds in shard order
        assert np.array_equal(out.cpu().numpy(), acc)


def test_full_size_sharded_matmul_sampled():
    """B=2048, D=8192, F=28672, 8 shards; the oracle computes 48 sampled rows x 512 sampled columns."""
    wl = synth.SHARDED_MATMUL
    b, d, f = wl.extra["B"], wl.extra["D"], wl.extra["F"]
    note("sharded matmul full size")
    x, w_t = synth.sharded_matmul_inputs(b, d, f)
    y_full, y_cols, y_sum, parts = _three_ways(x, w_t, wl.extra["shards"])
    del parts
    assert torch.equal(y_full.view(torch.int16), y_cols.view(torch.int16))
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(b, 48, replace=False))
    cols = np.sort(rng.choice(f, 512, replace=False))
    ref = gemm.matmul_f64(np.ascontiguousarray(x[rows]), np.ascontiguousarray(w_t[cols]))
    assert_close_rows(values(y_full)[np.ix_(rows, cols)], ref, what="full")
    assert_close_rows(values(y_sum)[np.ix_(rows, cols)], ref, what="K-split sum")
