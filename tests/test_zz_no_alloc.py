"""GPU checks of swr_mlp_forward_noalloc, the MLP entry point that takes no
workspace (its scratch is a fixed per-GPU array of the library): for callers
that cannot allocate device memory.

Each case calls it twice in a row, the second time with fewer tokens, and
compares both outputs with swr_mlp_forward's on the same inputs (same kernels,
so bit for bit) and with the oracle (the tolerance bar).  Between the two
calls the scratch keeps the first call's contents, so a kernel that read
stale scratch instead of what the call wrote would show up in the second one.
"""
import numpy as np
import pytest
import torch

import sharded_weight_reassembly_amd as swr
import synth
from oracle import gemm, numerics

from gpu_util import DEV, assert_close_rows, bf16, bits, f32, note, u8, values

pytestmark = pytest.mark.gpu


def _run_both(gu, d, hidden, inter, x_bits):
    m = x_bits.shape[0]
    xd = bf16(x_bits)
    wgu, wd = u8(gu.raw()), u8(d.raw())
    sgu = f32(gu.scale) if gu.scale is not None else None
    sd = f32(d.scale) if d.scale is not None else None
    y_ws = torch.full((m, hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(swr.mlp_workspace_bytes(m, hidden, inter, gu.dtype), dtype=torch.uint8, device=DEV)
    swr.mlp_forward(wgu, sgu, wd, sd, gu.dtype, hidden, inter, xd, y_ws, ws)
    y_na = torch.full((m, hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    swr.mlp_forward_noalloc(wgu, sgu, wd, sd, gu.dtype, hidden, inter, xd, y_na)
    torch.cuda.synchronize()
    return bits(y_ws), bits(y_na)


@pytest.mark.parametrize("dt", [synth.FP8, synth.BF16])
def test_noalloc_matches_workspace_entry_point(dt):
    """hidden 1024, intermediate 2048: 64 tokens (split-K down GEMM, scratch
    holds h and partials), then 8 tokens."""
    hidden, inter = 1024, 2048
    gu = synth.weight(synth.seed_for(31, 0, 0), 2 * inter, hidden, dt)
    d = synth.weight(synth.seed_for(31, 0, 1), hidden, inter, dt)
    x = synth.activations(synth.seed_for(31, 0, 50), 64, hidden)
    for m in (64, 8):
        note(f"noalloc mlp {dt} h={hidden} i={inter} m={m}")
        y_ws, y_na = _run_both(gu, d, hidden, inter, x[:m])
        assert np.array_equal(y_na, y_ws), f"m={m}: differs from swr_mlp_forward"
        _, _, ref = gemm.mlp_f64(x[:m], gu.raw(), gu.scale, d.raw(), d.scale, dt, hidden, inter)
        assert_close_rows(numerics.bf16_to_f64(y_na), ref, what=f"noalloc m={m}")


def test_noalloc_full_size_shared_expert():
    """Hidden 6144, intermediate 14336, FP8: 64 tokens (about 8 MB of scratch)
    then 1 token; sampled output columns against the oracle."""
    wl = synth.SHARED_EXPERT_DECODE
    gu, d = wl.layer_weights(0)
    x = synth.activations(synth.seed_for(2, 0, 50), 64, wl.hidden)
    g = gemm.proj_f64(x, gu.raw(), gu.dtype, 2 * wl.intermediate, wl.hidden, gu.scale)
    with np.errstate(over="ignore"):
        h = numerics.f64_to_bf16_bits(numerics.silu(g[:, :wl.intermediate]) * g[:, wl.intermediate:])
    cols = np.sort(np.random.default_rng(3).choice(wl.hidden, size=256, replace=False))
    for m in (64, 1):
        note(f"noalloc full-size shared expert m={m}")
        y_ws, y_na = _run_both(gu, d, wl.hidden, wl.intermediate, x[:m])
        assert np.array_equal(y_na, y_ws), f"m={m}: differs from swr_mlp_forward"
        ref = gemm.proj_f64(h[:m], np.ascontiguousarray(d.data[cols]), d.dtype, len(cols), wl.intermediate,
                            d.scale[cols])
        assert_close_rows(numerics.bf16_to_f64(y_na)[:, cols], ref, what=f"noalloc full m={m}")


def test_noalloc_refuses_sizes_beyond_its_scratch():
    """4096 tokens of the shared expert need about 117 MB of scratch: refused
    with SWR_E_CAPACITY before anything is enqueued."""
    wl = synth.SHARED_EXPERT_DECODE
    need = swr.mlp_workspace_bytes(4096, wl.hidden, wl.intermediate, synth.FP8)
    assert need > swr.NOALLOC_SCRATCH_BYTES
    buf = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    p = buf.data_ptr()
    with pytest.raises(swr.SwrError) as e:
        swr.mlp_forward_noalloc(p, p, p, p, synth.FP8, wl.hidden, wl.intermediate, p, p, m=4096)
    assert e.value.code == swr.E_CAPACITY
