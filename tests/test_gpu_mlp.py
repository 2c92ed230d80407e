"""GPU parity: swr_mlp_forward (gate_up -> SiLU*up -> down) against the oracle.

vLLM PR #50656 report, test code: gate rows then up rows; SiLU of the gate
half times the up half; then the down projection.  Bar: max|y - y_ref| <=
1e-2 * max(1, max|y_ref| of the row).
"""
import numpy as np
import pytest
import torch

import sharded_weight_reassembly_amd as swr
import synth
from oracle import gemm, numerics

from gpu_util import DEV, assert_close_rows, bf16, f32, note, u8, values

pytestmark = pytest.mark.gpu


def _mlp(gu, d, hidden, inter, x_bits, m=None):
    m = x_bits.shape[0] if m is None else m
    dt = gu.dtype
    y = torch.full((max(m, 1), hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    nb = swr.mlp_workspace_bytes(m, hidden, inter, dt)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    swr.mlp_forward(u8(gu.raw()), f32(gu.scale) if gu.scale is not None else None, u8(d.raw()),
                    f32(d.scale) if d.scale is not None else None, dt, hidden, inter, bf16(x_bits), y, ws, m=m)
    torch.cuda.synchronize()
    return y[:m]


@pytest.mark.parametrize("dt", [synth.BF16, synth.FP8])
@pytest.mark.parametrize("hidden,inter", [(128, 256), (256, 96), (512, 1024), (192, 320)])
@pytest.mark.parametrize("m", [1, 4, 16, 33, 64, 100])
def test_mlp_parity(dt, hidden, inter, m):
    note(f"mlp h={hidden} i={inter} {dt} m={m}")
    gu = synth.weight(synth.seed_for(13, 0, 0), 2 * inter, hidden, dt)
    d = synth.weight(synth.seed_for(13, 0, 1), hidden, inter, dt)
    x = synth.activations(synth.seed_for(13, 0, 50), m, hidden)
    y = _mlp(gu, d, hidden, inter, x)
    _, _, ref = gemm.mlp_f64(x, gu.raw(), gu.scale, d.raw(), d.scale, dt, hidden, inter)
    assert_close_rows(values(y), ref, what=f"mlp {hidden}/{inter} {dt} m={m}")


@pytest.mark.parametrize("hidden,inter,m", [(2048, 4128, 1), (2048, 4128, 40), (2048, 2144, 17), (2048, 2144, 64)])
def test_short_row_blocks_silu(hidden, inter, m):
    """gate_up shapes where the planner shortens row blocks (gate rows and the
    matching up rows) to fill whole waves of CUs and the last block is
    partial: 20 gate rows per block, the last of 8 (I = 4128) or 4 (I = 2144)."""
    note(f"short silu row blocks h={hidden} i={inter} m={m}")
    gu = synth.weight(synth.seed_for(13, 2, 0), 2 * inter, hidden, synth.FP8)
    d = synth.weight(synth.seed_for(13, 2, 1), hidden, inter, synth.FP8)
    x = synth.activations(synth.seed_for(13, 2, 50), m, hidden)
    y = _mlp(gu, d, hidden, inter, x)
    _, _, ref = gemm.mlp_f64(x, gu.raw(), gu.scale, d.raw(), d.scale, synth.FP8, hidden, inter)
    assert_close_rows(values(y), ref, what=f"mlp {hidden}/{inter} m={m}")


@pytest.mark.parametrize("m", [1, 9, 13, 16])
def test_gate_up_one_token_block_on_eight_waves(m):
    """I = 10240 gives 160 blocks of 64 gate + 64 up rows, so at 1-16 tokens
    gate_up runs the eight-wave kernel with activations through LDS (the
    down GEMM, 512 rows, stays on four waves with a K split)."""
    hidden, inter = 512, 10240
    note(f"gate_up one token block, eight waves h={hidden} i={inter} m={m}")
    gu = synth.weight(synth.seed_for(13, 3, 0), 2 * inter, hidden, synth.FP8)
    d = synth.weight(synth.seed_for(13, 3, 1), hidden, inter, synth.FP8)
    x = synth.activations(synth.seed_for(13, 3, 50), m, hidden)
    y = _mlp(gu, d, hidden, inter, x)
    _, _, ref = gemm.mlp_f64(x, gu.raw(), gu.scale, d.raw(), d.scale, synth.FP8, hidden, inter)
    assert_close_rows(values(y), ref, what=f"mlp {hidden}/{inter} m={m}")


@pytest.mark.parametrize("hidden,inter,m", [(512, 4096, 64), (448, 4096, 40), (512, 2048, 17)])
def test_down_split_k_matches_projection(hidden, inter, m):
    """17-64 tokens: the MLP's down GEMM splits K over workgroups (512 x 4096
    at 64 tokens: 4 row blocks x 4 splits) and a finalize kernel adds the
    splits.  Its output must be the bits of swr_proj_forward on the MLP's own
    h (which sits at the start of the workspace) and within the bar of the
    oracle; a second, smaller call on the same workspace must be right too."""
    note(f"down split-K h={hidden} i={inter} m={m}")
    gu = synth.weight(synth.seed_for(13, 3, 0), 2 * inter, hidden, synth.FP8)
    d = synth.weight(synth.seed_for(13, 3, 1), hidden, inter, synth.FP8)
    x = synth.activations(synth.seed_for(13, 3, 50), m, hidden)
    nb = swr.mlp_workspace_bytes(m, hidden, inter, synth.FP8)
    assert nb > (m * inter * 2 + 255) // 256 * 256  # the down GEMM splits K
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    wgu, sgu, wd, sd = u8(gu.raw()), f32(gu.scale), u8(d.raw()), f32(d.scale)
    for mm in (m, m - 7):
        y = torch.full((mm, hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
        swr.mlp_forward(wgu, sgu, wd, sd, synth.FP8, hidden, inter, bf16(x[:mm]), y, ws, m=mm)
        torch.cuda.synchronize()
        h = ws[: mm * inter * 2].view(torch.bfloat16).view(mm, inter).clone()
        y2 = torch.full((mm, hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
        pb = swr.proj_workspace_bytes(mm, hidden, inter, synth.FP8)  # 0: this token count does not split K
        pw = torch.empty(pb, dtype=torch.uint8, device=DEV) if pb > 0 else None
        swr.proj_forward(wd, synth.FP8, sd, hidden, inter, h, y2, workspace=pw)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "MLP down differs from the projection"
        _, _, ref = gemm.mlp_f64(x[:mm], gu.raw(), gu.scale, d.raw(), d.scale, synth.FP8, hidden, inter)
        assert_close_rows(values(y), ref, what=f"mlp {hidden}/{inter} m={mm}")


def test_tiny_config_mlp_and_projection():
    """The tiny workload: hidden 128, intermediate 256, BF16, 4 tokens, N=4 chunks,
    run through views of the reassembled slot."""
    wl = synth.TINY
    note("tiny workload through slot views")
    ws = wl.layer_weights(0)
    shp = [(o, i, d) for _, o, i, d in wl.weights]
    views, lay = swr.plan_layer(shp, wl.n_chunks)
    chunks = [torch.empty(lay["chunk_bytes"], dtype=torch.uint8, device=DEV) for _ in range(wl.n_chunks)]
    swr.pack_layer(lay, views, [u8(w.raw()) for w in ws], chunks)
    slot = torch.empty(lay["total_bytes"], dtype=torch.uint8, device=DEV)
    swr.reassemble_into_slot(chunks, lay["chunk_bytes"], slot)
    x = synth.activations(synth.seed_for(1, 0, 50), 4, 128)
    xd = bf16(x)
    y = torch.empty((4, 128), dtype=torch.bfloat16, device=DEV)
    wsp = torch.empty(swr.mlp_workspace_bytes(4, 128, 256, "bf16"), dtype=torch.uint8, device=DEV)
    base = slot.data_ptr()
    swr.mlp_forward(base + views[0]["offset"], None, base + views[1]["offset"], None, "bf16", 128, 256, xd, y, wsp)
    yp = torch.empty((4, 100), dtype=torch.bfloat16, device=DEV)
    swr.proj_forward(base + views[2]["offset"], "bf16", None, 100, 128, xd, yp)
    torch.cuda.synchronize()
    _, _, ref = gemm.mlp_f64(x, ws[0].raw(), None, ws[1].raw(), None, "bf16", 128, 256)
    assert_close_rows(values(y), ref, what="tiny mlp")
    refp = gemm.proj_f64(x, ws[2].raw(), "bf16", 100, 128)
    assert_close_rows(values(yp), refp, what="tiny proj")


def test_intermediate_slices_add_up_on_gpu():
    """The PR report's equivalence: the MLP over intermediate slices [r*s, (r+1)*s)
    (gate rows, matching up rows, down columns) summed over r equals the full
    MLP.  Here each slice runs through mlp_forward, whose output is rounded to
    bf16: each slice is held to the bar against the oracle's slice, and the sum
    of the four bf16 slices against the sum of the oracle's bf16-rounded slices
    (the same composition).  The unrounded fp32 form of the same equivalence is
    test_tensor_parallel_partials."""
    note("intermediate-slice partials")
    hidden, inter, ranks = 256, 512, 4
    dt = synth.FP8
    gu = synth.weight(21, 2 * inter, hidden, dt)
    d = synth.weight(22, hidden, inter, dt)
    x = synth.activations(23, 12, hidden)
    sh = inter // ranks
    total = np.zeros((12, hidden))
    total_ref = np.zeros((12, hidden))
    for r in range(ranks):
        rows = np.r_[r * sh:(r + 1) * sh, inter + r * sh:inter + (r + 1) * sh]
        gu_r = synth.Weight(2 * sh, hidden, dt, np.ascontiguousarray(gu.data[rows]), gu.scale[rows])
        d_r = synth.Weight(hidden, sh, dt, np.ascontiguousarray(d.data[:, r * sh:(r + 1) * sh]), d.scale)
        y_r = values(_mlp(gu_r, d_r, hidden, sh, x))
        ref_r = gemm.mlp_intermediate_slice_f64(x, gu.raw(), gu.scale, d.raw(), d.scale, dt, hidden, inter,
                                                r * sh, (r + 1) * sh)
        assert_close_rows(y_r, ref_r, what=f"slice {r}")
        total += y_r
        total_ref += numerics.bf16_round(ref_r)
    assert_close_rows(total, total_ref, what="sum of bf16 slices")
    _, _, ref = gemm.mlp_f64(x, gu.raw(), gu.scale, d.raw(), d.scale, dt, hidden, inter)
    # and the oracle's own rounded slices add up to its full MLP within the bar
    assert_close_rows(total_ref, ref, what="oracle: sum of bf16 slices vs full MLP")


@pytest.fixture(scope="module")
def shared_expert_layer():
    wl = synth.SHARED_EXPERT_DECODE
    gu, d = wl.layer_weights(0)
    x = synth.activations(synth.seed_for(2, 0, 50), 64, wl.hidden)
    return wl, gu, d, x


@pytest.mark.parametrize("m", [1, 8, 13, 16, 32, 64])
def test_full_size_shared_expert_mlp(shared_expert_layer, m):
    """Hidden 6144, intermediate 14336, FP8 E4M3FN with row scales; sampled output columns."""
    wl, gu, d, x = shared_expert_layer
    note(f"full-size shared-expert MLP m={m}")
    y = values(_mlp(gu, d, wl.hidden, wl.intermediate, x[:m]))
    _check_full(wl, gu, d, x, m, y)


_FULL_REF = {}


def _check_full(wl, gu, d, x, m, y):
    # The oracle's G needs every gate/up row; computed once at M=64 (rows of
    # X are independent, so smaller M are row prefixes).
    if "h" not in _FULL_REF:
        g = gemm.proj_f64(x, gu.raw(), gu.dtype, 2 * wl.intermediate, wl.hidden, gu.scale)
        with np.errstate(over="ignore"):
            _FULL_REF["h"] = numerics.f64_to_bf16_bits(numerics.silu(g[:, :wl.intermediate]) * g[:, wl.intermediate:])
    h = _FULL_REF["h"][:m]
    cols = np.sort(np.random.default_rng(1).choice(wl.hidden, size=512, replace=False))
    ref = gemm.proj_f64(h, np.ascontiguousarray(d.data[cols]), d.dtype, len(cols), wl.intermediate, d.scale[cols])
    assert_close_rows(y[:, cols], ref, what=f"shared expert m={m}")


@pytest.mark.parametrize("m", [4096, 16384])
def test_prefill_shared_expert_sampled_tokens(shared_expert_layer, m):
    """Prefill-shaped MLP (M = 4096 / 16384 tokens, hidden 6144, intermediate 14336,
    FP8 weights): the oracle recomputes 24 sampled tokens completely."""
    wl, gu, d, _ = shared_expert_layer
    note(f"prefill shared-expert MLP m={m}")
    x = synth.activations(synth.seed_for(4, 0, 50), m, wl.hidden)
    y = values(_mlp(gu, d, wl.hidden, wl.intermediate, x))
    toks = np.sort(np.random.default_rng(m).choice(m, 24, replace=False))
    _, _, ref = gemm.mlp_f64(np.ascontiguousarray(x[toks]), gu.raw(), gu.scale, d.raw(), d.scale, gu.dtype,
                             wl.hidden, wl.intermediate)
    assert_close_rows(y[toks], ref, what=f"prefill m={m}")
    assert np.isfinite(y).all()


def _rank_shards(gu, d, inter, ranks, r):
    """Rank r's contiguous weights of the tensor-parallel shared expert: its gate
    rows then its up rows, and its columns of down."""
    sh = inter // ranks
    rows = np.r_[r * sh:(r + 1) * sh, inter + r * sh:inter + (r + 1) * sh]
    gu_r = synth.Weight(2 * sh, gu.in_features, gu.dtype, np.ascontiguousarray(gu.data[rows]),
                        None if gu.scale is None else gu.scale[rows])
    d_r = synth.Weight(d.out_features, sh, d.dtype, np.ascontiguousarray(d.data[:, r * sh:(r + 1) * sh]), d.scale)
    return gu_r, d_r


def _tp_mlp(gu, d, hidden, inter, ranks, x_bits):
    """Every rank's fp32 partial (swr_mlp_forward_partial) and their sum in rank
    order rounded once (swr_sum_partials)."""
    m = x_bits.shape[0]
    parts = [torch.full((m, hidden), float("nan"), dtype=torch.float32, device=DEV) for _ in range(ranks)]
    ws = torch.empty(swr.mlp_workspace_bytes(m, hidden, inter // ranks, gu.dtype), dtype=torch.uint8, device=DEV)
    xd = bf16(x_bits)
    for r in range(ranks):
        gu_r, d_r = _rank_shards(gu, d, inter, ranks, r)
        swr.mlp_forward_partial(u8(gu_r.raw()), f32(gu_r.scale) if gu_r.scale is not None else None, u8(d_r.raw()),
                                f32(d_r.scale) if d_r.scale is not None else None, gu.dtype, hidden, inter // ranks,
                                xd, parts[r], ws)
        torch.cuda.synchronize()  # the rank's shard tensors go out of scope
    y = torch.empty((m, hidden), dtype=torch.bfloat16, device=DEV)
    swr.sum_partials(parts, y)
    torch.cuda.synchronize()
    return parts, y


@pytest.mark.parametrize("dt", [synth.BF16, synth.FP8])
@pytest.mark.parametrize("hidden,inter,ranks,m", [(256, 512, 4, 12), (512, 1024, 8, 33), (128, 256, 2, 1)])
def test_tensor_parallel_partials(dt, hidden, inter, ranks, m):
    """PR report, TP-sharded shared expert: each rank's fp32 partial equals the
    oracle's contribution of its intermediate slice, and the rank-ordered sum
    equals the full MLP."""
    note(f"tp partials h={hidden} i={inter} ranks={ranks} {dt} m={m}")
    gu = synth.weight(synth.seed_for(17, 0, 0), 2 * inter, hidden, dt)
    d = synth.weight(synth.seed_for(17, 0, 1), hidden, inter, dt)
    x = synth.activations(synth.seed_for(17, 0, 50), m, hidden)
    parts, y = _tp_mlp(gu, d, hidden, inter, ranks, x)
    sh = inter // ranks
    for r in range(ranks):
        ref = gemm.mlp_intermediate_slice_f64(x, gu.raw(), gu.scale, d.raw(), d.scale, dt, hidden, inter,
                                              r * sh, (r + 1) * sh)
        assert_close_rows(values(parts[r]), ref, what=f"rank {r} partial")
    _, _, ref = gemm.mlp_f64(x, gu.raw(), gu.scale, d.raw(), d.scale, dt, hidden, inter)
    assert_close_rows(values(y), ref, what="sum of rank partials")


@pytest.mark.parametrize("m", [1, 64])
def test_tensor_parallel_full_size(shared_expert_layer, m):
    """The shared expert (hidden 6144, intermediate 14336, FP8) split over 16
    ranks: the summed partials equal the oracle's MLP on sampled columns."""
    wl, gu, d, x = shared_expert_layer
    note(f"tp shared expert 16 ranks m={m}")
    _, y = _tp_mlp(gu, d, wl.hidden, wl.intermediate, 16, x[:m])
    _check_full(wl, gu, d, x, m, values(y))
