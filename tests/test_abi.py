"""Host-side checks of the C ABI (no GPU needed).

* the library loads and exports every function include/swr.h declares;
* swr_plan_layer (host only) agrees with the oracle's flat layout;
* argument errors come back as status codes before anything is enqueued.
"""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import sharded_weight_reassembly_amd as swr
from oracle import layout as olayout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swr.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swr_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 20
    L = swr.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(swr.EXPORTS)


def test_version_string():
    assert "gfx950" in swr.version()


@pytest.mark.parametrize("ws,n", [
    ([(512, 128, "bf16"), (128, 256, "bf16"), (100, 128, "bf16")], 4),
    ([(512, 128, "bf16"), (100, 127, "bf16"), (128, 256, "bf16"), (3, 5, "fp8_e4m3fn")], 3),
    ([(28672, 6144, "fp8_e4m3fn"), (6144, 14336, "fp8_e4m3fn")], 16),
])
def test_plan_matches_oracle(ws, n):
    views, lay = swr.plan_layer(ws, n)
    ref = olayout.plan_layer(ws, n)
    assert [v["offset"] for v in views] == ref["offsets"]
    assert [v["nbytes"] for v in views] == ref["sizes"]
    assert lay["total_bytes"] == ref["total"] and lay["chunk_bytes"] == ref["chunk"]
    assert lay["payload_bytes"] == ref["payload"] and lay["n_chunks"] == n and lay["n_weights"] == len(ws)


@settings(max_examples=200, deadline=None)
@given(ws=st.lists(st.tuples(st.integers(1, 3000), st.integers(1, 3000), st.sampled_from(["bf16", "fp8_e4m3fn"])),
                   min_size=1, max_size=64),
       n=st.integers(1, 64))
def test_plan_matches_oracle_random(ws, n):
    views, lay = swr.plan_layer(ws, n)
    ref = olayout.plan_layer(ws, n)
    assert [v["offset"] for v in views] == ref["offsets"]
    assert (lay["total_bytes"], lay["chunk_bytes"], lay["payload_bytes"]) == (ref["total"], ref["chunk"], ref["payload"])


@pytest.mark.parametrize("ws,n,code", [
    ([], 4, swr.E_INVALID),
    ([(4, 4, "bf16")], 0, swr.E_INVALID),
    ([(4, 4, "bf16")], 65, swr.E_INVALID),
    ([(0, 4, "bf16")], 4, swr.E_SHAPE),
    ([(4, -1, "bf16")], 4, swr.E_SHAPE),
    ([(4, 4, 7)], 4, swr.E_INVALID),
    ([(1 << 40, 1 << 20, "bf16")], 4, swr.E_SHAPE),
    ([(4, 4, "bf16")] * 65, 4, swr.E_INVALID),
])
def test_plan_errors(ws, n, code):
    with pytest.raises(swr.SwrError) as e:
        swr.plan_layer(ws, n)
    assert e.value.code == code
    assert swr.lib().swr_last_error().decode()


def _vp_array(vals):
    arr = (ctypes.c_void_p * max(len(vals), 1))()
    for i, v in enumerate(vals):
        arr[i] = v
    return arr


def test_reassemble_argument_errors_before_enqueue():
    L = swr.lib()
    good = 1 << 20
    chunks = _vp_array([good, good + 4096])
    # null slot
    assert L.swr_reassemble_into_slot(chunks, 2, 4096, None, 8192, 0, None, None, None, None) == swr.E_INVALID
    # chunk size not a multiple of 16
    assert L.swr_reassemble_into_slot(chunks, 2, 4008, good, 8192, 0, None, None, None, None) == swr.E_ALIGN
    # slot too small
    assert L.swr_reassemble_into_slot(chunks, 2, 4096, good, 8191, 0, None, None, None, None) == swr.E_CAPACITY
    # misaligned slot
    assert L.swr_reassemble_into_slot(chunks, 2, 4096, good + 8, 8192, 0, None, None, None, None) == swr.E_ALIGN
    # misaligned chunk
    bad = _vp_array([good, good + 4])
    assert L.swr_reassemble_into_slot(bad, 2, 4096, good, 8192, 0, None, None, None, None) == swr.E_ALIGN
    # self rank out of range, too many chunks
    assert L.swr_reassemble_into_slot(chunks, 2, 4096, good, 8192, 2, None, None, None, None) == swr.E_INVALID
    assert L.swr_reassemble_into_slot(_vp_array([good] * 65), 65, 16, good, 1 << 20, 0, None, None, None,
                                      None) == swr.E_INVALID


def test_redistribute_errors_before_enqueue():
    L = swr.lib()
    a = 1 << 20
    shp = [(512, 128, "bf16"), (100, 128, "bf16")]
    views, lay = swr.plan_layer(shp, 4)
    lay_s, views_s = swr._layout_struct(lay), swr._views_struct(views)
    chunks = _vp_array([a + i * lay["chunk_bytes"] for i in range(4)])

    def call(shards):
        return L.swr_redistribute_row_shards(ctypes.byref(lay_s), views_s, swr.row_shards_struct(shards), chunks,
                                             None)

    good = [dict(sub_rows=[256, 256], src=[a] * 4), dict(sub_rows=[100], src=[a] * 4)]
    assert L.swr_redistribute_row_shards(None, views_s, swr.row_shards_struct(good), chunks, None) == swr.E_INVALID
    # 100 rows over 4 ranks is fine; 102 rows would not be
    assert call([good[0], dict(sub_rows=[98, 2], src=[a] * 4)]) == swr.E_SHAPE
    assert call([dict(sub_rows=[256, 252], src=[a] * 4), good[1]]) == swr.E_SHAPE   # rows do not add up
    assert call([dict(sub_rows=[], src=[a] * 4), good[1]]) == swr.E_INVALID         # no sub-blocks
    assert call([good[0], dict(sub_rows=[100], src=[a, a, a + 8, a])]) == swr.E_ALIGN
    assert call([good[0], dict(sub_rows=[100], src=[a, a, None, a])]) == swr.E_INVALID
    assert call([good[0], dict(replicated=True, src=[None])]) == swr.E_INVALID


def test_size_checks_do_not_overflow():
    """Sizes whose products or sums would wrap in int64 are refused before
    anything is enqueued (a wrapped size would pass a capacity check)."""
    L = swr.lib()
    a = 1 << 20
    huge = 1 << 62  # 4 * huge wraps to 0
    chunks4 = _vp_array([a] * 4)
    for fn in (L.swr_reassemble_into_slot, L.swr_reassemble_into_slot_dma):
        assert fn(chunks4, 4, huge, a, 8192, 0, None, None, None, None) == swr.E_CAPACITY
    shp = [(512, 128, "bf16"), (100, 128, "bf16")]
    views, lay = swr.plan_layer(shp, 4)
    chunks = _vp_array([a + i * lay["chunk_bytes"] for i in range(4)])
    srcs = _vp_array([a, a])
    # N * (C + 2^62) wraps to N * C = |T|
    wrapped = dict(lay, chunk_bytes=lay["chunk_bytes"] + huge)
    assert L.swr_pack_layer(ctypes.byref(swr._layout_struct(wrapped)), swr._views_struct(views), srcs, chunks,
                            None) == swr.E_INVALID
    # a view whose offset + nbytes wraps below the payload end
    long_view = [views[0], dict(views[1], nbytes=(1 << 63) - views[1]["offset"])]
    assert L.swr_pack_layer(ctypes.byref(swr._layout_struct(lay)), swr._views_struct(long_view), srcs, chunks,
                            None) == swr.E_INVALID
    # negative shapes whose product matches the view's bytes
    neg = [views[0], dict(views[1], out_features=-100, in_features=-128)]
    rs = swr.row_shards_struct([dict(sub_rows=[256, 256], src=[a] * 4), dict(replicated=True, src=[a])])
    assert L.swr_redistribute_row_shards(ctypes.byref(swr._layout_struct(lay)), swr._views_struct(neg), rs, chunks,
                                         None) == swr.E_INVALID
    assert L.swr_redistribute_row_shards(ctypes.byref(swr._layout_struct(wrapped)), swr._views_struct(views), rs,
                                         chunks, None) == swr.E_INVALID


def test_dma_reassemble_checks_like_the_kernel_path():
    L = swr.lib()
    good = 1 << 20
    chunks = _vp_array([good, good + 4096])
    for fn in (L.swr_reassemble_into_slot, L.swr_reassemble_into_slot_dma):
        assert fn(None, 2, 4096, good, 8192, 0, None, None, None, None) == swr.E_INVALID
        assert fn(chunks, 2, 4008, good, 8192, 0, None, None, None, None) == swr.E_ALIGN
        assert fn(chunks, 2, 4096, good, 8191, 0, None, None, None, None) == swr.E_CAPACITY
        assert fn(chunks, 2, 4096, good + 8, 8192, 0, None, None, None, None) == swr.E_ALIGN
        assert fn(chunks, 2, 4096, good, 8192, 2, None, None, None, None) == swr.E_INVALID


def test_gemm_argument_errors_before_enqueue():
    L = swr.lib()
    a = 1 << 20
    # FP8 without scales
    assert L.swr_proj_forward(a, swr.FP8_E4M3FN, None, 64, 64, a, 64, 4, a, 0, 64, None, 0, None) == swr.E_INVALID
    # misaligned X
    assert L.swr_proj_forward(a, swr.BF16, None, 64, 64, a + 2, 64, 4, a, 0, 64, None, 0, None) == swr.E_ALIGN
    # ldx too small
    assert L.swr_proj_forward(a, swr.BF16, None, 64, 64, a, 32, 4, a, 0, 64, None, 0, None) == swr.E_SHAPE
    # unknown dtype
    assert L.swr_proj_forward(a, 3, None, 64, 64, a, 64, 4, a, 0, 64, None, 0, None) == swr.E_INVALID
    # workspace too small for the MLP
    need = swr.mlp_workspace_bytes(4, 128, 256, "bf16")
    assert need >= 4 * 256 * 2
    assert L.swr_mlp_forward(a, None, a, None, swr.BF16, 128, 256, a, 4, a, a, need - 1, None) == swr.E_CAPACITY
    assert L.swr_mlp_forward(a, None, a, None, swr.BF16, 128, 256, a, 4, a, a + 16, need, None) == swr.E_ALIGN
    assert L.swr_mlp_workspace_bytes(4, 0, 256, swr.BF16) == swr.E_SHAPE


def _descs(specs):
    arr = (swr.ProjDesc * len(specs))()
    for i, (w, s, x, y, o, k, ldx, ldy, dt) in enumerate(specs):
        arr[i].W, arr[i].row_scale, arr[i].X, arr[i].Y = w, s, x, y
        arr[i].out_features, arr[i].in_features, arr[i].ldx, arr[i].ldy = o, k, ldx, ldy
        arr[i].dtype, arr[i].y_fp32 = dt, 0
    return arr


def test_grouped_projection_errors_before_enqueue():
    L = swr.lib()
    a = 1 << 20
    ok = (a, a, a, a, 64, 256, 256, 64, swr.FP8_E4M3FN)
    assert L.swr_proj_forward_grouped(None, 1, 4, None, 0, None) == swr.E_INVALID
    assert L.swr_proj_forward_grouped(_descs([ok]), 0, 4, None, 0, None) == swr.E_INVALID
    assert L.swr_proj_forward_grouped(_descs([ok] * 17), 17, 4, None, 0, None) == swr.E_INVALID
    # the bad descriptor is the second one: nothing may be enqueued for the first
    no_scale = (a, None, a, a, 64, 256, 256, 64, swr.FP8_E4M3FN)
    assert L.swr_proj_forward_grouped(_descs([ok, no_scale]), 2, 4, None, 0, None) == swr.E_INVALID
    misaligned = (a, a, a, a + 8, 64, 256, 256, 64, swr.FP8_E4M3FN)
    assert L.swr_proj_forward_grouped(_descs([ok, misaligned]), 2, 4, None, 0, None) == swr.E_ALIGN
    short_ldx = (a, a, a, a, 64, 256, 128, 64, swr.FP8_E4M3FN)
    assert L.swr_proj_forward_grouped(_descs([ok, short_ldx]), 2, 4, None, 0, None) == swr.E_SHAPE
    bad_dtype = (a, a, a, a, 64, 256, 256, 64, 7)
    assert L.swr_proj_forward_grouped(_descs([bad_dtype]), 1, 4, None, 0, None) == swr.E_INVALID
    assert L.swr_proj_forward_grouped(_descs([ok]), 1, 4, a + 16, 256, None) == swr.E_ALIGN


def test_grouped_workspace_bytes():
    L = swr.lib()
    a = 1 << 20
    stageable = [(a, a, a, a, 1000, 512, 512, 1000, swr.FP8_E4M3FN), (a, a, a, a, 300, 768, 768, 300, swr.FP8_E4M3FN)]
    # one launch without any K split: no scratch
    assert L.swr_proj_grouped_workspace_bytes(_descs(stageable), 2, 16) == 0
    # K = 320 cannot be staged: separate launches, scratch of the largest single projection
    mixed = stageable + [(a, a, a, a, 640, 320, 320, 640, swr.FP8_E4M3FN)]
    need = L.swr_proj_grouped_workspace_bytes(_descs(mixed), 3, 16)
    singles = [swr.proj_workspace_bytes(16, o, k, "fp8_e4m3fn") for (_, _, _, _, o, k, _, _, _) in mixed]
    assert need == max(singles)
    # tokens past the decode range: one launch of the tiled kernel, no scratch
    assert L.swr_proj_grouped_workspace_bytes(_descs(stageable), 2, 65) == 0
    assert L.swr_proj_grouped_workspace_bytes(_descs(mixed), 3, 300) == 0  # K = 320 is a multiple of 64
    # K = 100 fits no tiled kernel: separate launches, scratch of the largest single projection
    odd = stageable + [(a, a, a, a, 640, 100, 104, 640, swr.FP8_E4M3FN)]
    assert L.swr_proj_grouped_workspace_bytes(_descs(odd), 3, 300) == max(
        swr.proj_workspace_bytes(300, o, k, "fp8_e4m3fn") for (_, _, _, _, o, k, _, _, _) in odd)


def test_planner_handles_every_token_count():
    """The GEMM planner runs on the host before any launch: no token count or
    shape of the workloads may trip it (zero tokens included)."""
    L = swr.lib()
    a = 1 << 20
    shapes = [(6144, 14336), (28672, 6144), (24576, 7168), (1000, 7168), (100, 128), (320, 512), (96, 256)]
    for m in (0, 1, 2, 8, 16, 17, 31, 32, 33, 63, 64, 65):
        for out_f, in_f in shapes:
            for dt in ("bf16", "fp8_e4m3fn"):
                assert swr.proj_workspace_bytes(m, out_f, in_f, dt) >= 0
        assert swr.mlp_workspace_bytes(m, 6144, 14336, "fp8_e4m3fn") >= 0
    # zero tokens through the grouped entry: separate-launch planning, nothing enqueued
    descs = _descs([(a, a, a, a, 320, 512, 512, 320, swr.FP8_E4M3FN)])
    assert L.swr_proj_grouped_workspace_bytes(descs, 1, 0) >= 0


def test_mlp_workspace_covers_h():
    for m in (1, 8, 32, 64, 100):
        for dt in ("bf16", "fp8_e4m3fn"):
            need = swr.mlp_workspace_bytes(m, 6144, 14336, dt)
            assert need >= m * 14336 * 2 and need % 256 == 0


def test_planner_errors_without_gpu_work():
    L = swr.lib()
    h = ctypes.c_void_p()
    a = 1 << 20
    assert L.swr_planner_create(3, 3, 1, 2, a, a, 4096, ctypes.byref(h)) == swr.E_INVALID
    assert L.swr_planner_create(0, 4, 1, 2, a, a, 0, ctypes.byref(h)) == swr.E_INVALID
    assert L.swr_planner_set_gate(None, swr.GATE_AFTER) == swr.E_INVALID
    assert L.swr_planner_create(0, 4, 1, 2, a + 8, a, 4096, ctypes.byref(h)) == swr.E_ALIGN
    assert L.swr_planner_create(0, 4, 1, 2, None, a, 4096, ctypes.byref(h)) == swr.E_INVALID
    assert L.swr_planner_reset(None) == swr.E_INVALID
    assert L.swr_planner_set_copy_engine(None, 0) == swr.E_INVALID
    assert L.swr_planner_set_gather_lds(None, 0) == swr.E_INVALID
    assert L.swr_planner_pause_timing(None, 1) == swr.E_INVALID


def test_fp8act_entry_points_validate_without_gpu_work():
    L = swr.lib()
    a = 1 << 20
    # null pointers and shapes are refused before anything is enqueued
    assert L.swr_quantize_rows_e4m3(None, 16, 4, 16, a, 16, a, None) == swr.E_INVALID
    assert L.swr_quantize_rows_e4m3(a, 16, -1, 16, a, 16, a, None) == swr.E_SHAPE
    assert L.swr_quantize_rows_e4m3(a, 8, 4, 16, a, 16, a, None) == swr.E_SHAPE
    assert L.swr_mlp_forward_fp8act(a, None, a, a, 256, 320, a, 4, a, a, 1 << 20, None) == swr.E_INVALID
    assert L.swr_mlp_forward_fp8act(a, a, a, a, 250, 320, a, 4, a, a, 1 << 20, None) == swr.E_SHAPE
    # workspace: codes and scales of X and h, and h, in 256-byte sections
    m, h, i = 300, 256, 320
    def up(n):
        return (n + 255) // 256 * 256
    assert swr.mlp_fp8act_workspace_bytes(m, h, i) == up(m * h) + up(4 * m) + up(2 * m * i) + up(m * i) + up(4 * m)
    assert swr.mlp_fp8act_workspace_bytes(0, h, i) == 0


def test_memory_and_transfer_account_from_library_layouts():
    """weight_sharding, cost section: per rank R/N + 2 max_l |T_l| bytes of
    weights (its chunks plus two slots) and (N-1)/N * S bytes received per
    layer.  The library's own layouts for the two decode workloads against
    numbers worked out by hand:
      shared expert, 8 layers, N = 16: |T| = 28672*6144 + 6144*14336 =
        264,241,152 (no padding: both items are multiples of 16 and the sum
        of 256); C = 16,515,072; R/N = 8 C = 132,120,576; two slots
        528,482,304; total 660,602,880; received per layer 15 C = 247,726,080;
      attention projections, 16 layers, N = 16: |T| = 385,179,648,
        C = 24,073,728; R/N = 16 C = 385,179,648; two slots 770,359,296;
        total 1,155,538,944; received per layer 15 C = 361,105,920."""
    se = [(28672, 6144, "fp8_e4m3fn"), (6144, 14336, "fp8_e4m3fn")]
    attn = [(24576, 7168), (8192, 7168), (7168, 8192), (4096, 7168), (1000, 7168), (7168, 3072), (3072, 7168),
            (1536, 7168)]
    attn = [(o, i, "fp8_e4m3fn") for o, i in attn]
    for ws, layers, want in ((se, 8, (264_241_152, 16_515_072, 660_602_880, 247_726_080)),
                             (attn, 16, (385_179_648, 24_073_728, 1_155_538_944, 361_105_920))):
        lays = [swr.plan_layer(ws, 16)[1] for _ in range(layers)]
        totals = [lay["total_bytes"] for lay in lays]
        resident = sum(lay["chunk_bytes"] for lay in lays)  # one rank's chunks: R / N
        memory = resident + 2 * max(totals)
        received = (16 - 1) * lays[0]["chunk_bytes"]
        assert (totals[0], lays[0]["chunk_bytes"], memory, received) == want


def test_noalloc_mlp_refuses_before_any_hip_call():
    """swr_mlp_forward_noalloc checks pointers and its scratch limit on the host
    first: 4096 shared-expert tokens need about 117 MB of scratch, more than
    its fixed 16 MiB, and come back as SWR_E_CAPACITY (no GPU is touched)."""
    L = swr.lib()
    p = 1 << 20
    assert L.swr_mlp_forward_noalloc(p, p, p, p, 1, 6144, 14336, p, 4096, p, None) == swr.E_CAPACITY
    assert "scratch" in L.swr_last_error().decode()
    assert L.swr_mlp_forward_noalloc(None, p, p, p, 1, 6144, 14336, p, 64, p, None) == swr.E_INVALID
    assert swr.mlp_workspace_bytes(64, 6144, 14336, "fp8_e4m3fn") <= swr.NOALLOC_SCRATCH_BYTES
