"""GPU parity: swr_proj_forward against the oracle.

The bar (fp32 accumulation): max|y - y_ref| <= 1e-2 * max(1, max|y_ref| of
the row).  Exact checks where the arithmetic fixes the answer: one-hot rows
select a decoded weight column exactly, the bf16 output is the round-to-
nearest-even of the fp32 output of the same call.
"""
import numpy as np
import pytest
import torch

import sharded_weight_reassembly_amd as swr
import synth
from oracle import gemm, numerics

from gpu_util import DEV, assert_close_rows, bf16, bits, f32, note, u8, values

pytestmark = pytest.mark.gpu


def _run_proj(w, x_bits, m=None, y_fp32=False, workspace=True, ldy=None, x_pad=0):
    o, k, dt = w.out_features, w.in_features, w.dtype
    m = x_bits.shape[0] if m is None else m
    wd = u8(w.raw())
    sd = f32(w.scale) if w.scale is not None else None
    xb = np.zeros((x_bits.shape[0], k + x_pad), np.uint16)
    xb[:, :k] = x_bits
    xd = bf16(xb)
    ldy = o if ldy is None else ldy
    y = torch.full((max(m, 1), ldy), float("nan"), dtype=torch.float32 if y_fp32 else torch.bfloat16, device=DEV)
    ws = None
    if workspace:
        nb = swr.proj_workspace_bytes(m, o, k, dt)
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
    swr.proj_forward(wd, dt, sd, o, k, xd, y, m=m, ldx=k + x_pad, ldy=ldy, y_fp32=y_fp32, workspace=ws)
    torch.cuda.synchronize()
    return y[:m, :o]


SHAPES = [
    # (out, in, dtype) -- several row tiles, ragged row tails, K tails, odd shapes
    (512, 128, synth.BF16),
    (100, 128, synth.BF16),
    (128, 256, synth.BF16),
    (100, 127, synth.BF16),      # odd projection: plain kernel
    (3, 5, synth.FP8),            # tiny FP8 item: plain kernel
    (1000, 512, synth.FP8),       # ragged rows (1000 = 15*64 + 40)
    (300, 1536, synth.FP8),
    (64, 64, synth.FP8),
    (777, 320, synth.BF16),       # K = 5*64: not a multiple of 256
    (2048, 1024, synth.FP8),
    (64, 8192, synth.FP8),        # few row blocks: 512-K stages with a 4-way K split at <= 16 tokens
    (96, 16384, synth.FP8),       # 512-K stages, 8-way K split
]


@pytest.mark.parametrize("o,k,dt", SHAPES)
@pytest.mark.parametrize("m", [1, 4, 16, 17, 33, 64, 65, 130])
def test_proj_parity(o, k, dt, m):
    note(f"proj o={o} k={k} {dt} m={m}")
    w = synth.weight(synth.seed_for(12, 0, o % 97), o, k, dt)
    x = synth.activations(synth.seed_for(12, 0, 50), m, k)
    y = _run_proj(w, x)
    ref = gemm.proj_f64(x, w.raw(), dt, o, k, w.scale)
    assert_close_rows(values(y), ref, what=f"proj {o}x{k} {dt} m={m}")


@pytest.mark.parametrize("o,k,m", [(4128, 512, 1), (4128, 512, 8), (7712, 2048, 17), (7712, 2048, 40),
                                   (7712, 2048, 64)])
def test_short_row_blocks(o, k, m):
    """Shapes where the planner shortens row blocks to fill whole waves of CUs
    and the last block is partial (4128 rows at <= 16 tokens: 20-row blocks,
    the last of 8 rows; 7712 rows at 17-64 tokens: 64-row blocks of 128-row
    tiles, the last of 32): every row is computed once and only once."""
    note(f"short row blocks o={o} k={k} m={m}")
    w = synth.weight(synth.seed_for(12, 1, o % 97), o, k, synth.FP8)
    x = synth.activations(synth.seed_for(12, 1, 50), m, k)
    y = _run_proj(w, x)
    ref = gemm.proj_f64(x, w.raw(), synth.FP8, o, k, w.scale)
    assert_close_rows(values(y), ref, what=f"short row blocks {o}x{k} m={m}")


@pytest.mark.parametrize("dt", [synth.BF16, synth.FP8])
def test_bf16_output_is_rne_of_fp32_output(dt):
    note(f"rne check {dt}")
    w = synth.weight(5, 640, 1024, dt)
    x = synth.activations(6, 24, 1024)
    y32 = _run_proj(w, x, y_fp32=True)
    y16 = _run_proj(w, x, y_fp32=False)
    want = numerics.f64_to_bf16_bits(values(y32))
    assert np.array_equal(bits(y16), want)


@pytest.mark.parametrize("dt", [synth.BF16, synth.FP8])
def test_one_hot_rows_select_columns_exactly(dt):
    """X = e_k rows: Y[:, o] = bf16(s[o] * dec(W[o, k])) exactly, for 64 k in one step."""
    note(f"one-hot {dt}")
    o, k = 192, 256
    w = synth.weight(7, o, k, dt)
    ks = list(range(0, 64)) + [100, 200, 255]
    x = np.zeros((len(ks), k), np.uint16)
    for r, kk in enumerate(ks):
        x[r, kk] = 0x3F80
    y = bits(_run_proj(w, x))
    wd = numerics.decode_weight(w.raw(), dt, o, k)
    s = np.ones(o) if w.scale is None else w.scale.astype(np.float64)
    for r, kk in enumerate(ks):
        assert np.array_equal(y[r], numerics.f64_to_bf16_bits(wd[:, kk] * s)), f"k={kk}"


def test_every_fp8_code_decodes_like_the_table():
    """Row c of W holds code c at k=0 (NaN codes replaced by 0); X = e_0."""
    note("fp8 code table")
    codes = np.zeros((256, 64), np.uint8)
    codes[:, 0] = np.arange(256)
    codes[0x7F, 0] = 0
    codes[0xFF, 0] = 0
    w = synth.Weight(256, 64, synth.FP8, codes, np.ones(256, np.float32))
    x = np.zeros((1, 64), np.uint16)
    x[0, 0] = 0x3F80
    y = values(_run_proj(w, x, y_fp32=True))[0]
    want = numerics.fp8_to_f64(codes[:, 0])
    assert np.array_equal(y, want)


def test_strided_x_and_y_and_no_workspace():
    note("strided x/y, no workspace")
    w = synth.weight(8, 320, 512, synth.FP8)
    x = synth.activations(9, 20, 512)
    ref = gemm.proj_f64(x, w.raw(), synth.FP8, 320, 512, w.scale)
    y = _run_proj(w, x, ldy=400, x_pad=64, workspace=False)
    assert_close_rows(values(y), ref, what="strided")
    y2 = _run_proj(w, x, ldy=400, x_pad=64, workspace=True)
    assert_close_rows(values(y2), ref, what="strided+ws")


def test_zero_tokens_is_a_no_op():
    w = synth.weight(8, 64, 64, synth.BF16)
    wd = u8(w.raw())
    x = torch.zeros((1, 64), dtype=torch.bfloat16, device=DEV)
    y = torch.full((1, 64), 3.0, dtype=torch.bfloat16, device=DEV)
    swr.proj_forward(wd, synth.BF16, None, 64, 64, x, y, m=0)
    torch.cuda.synchronize()
    assert (y == 3.0).all()


def test_workspace_too_small_is_an_error():
    w = synth.weight(8, 64, 4096, synth.BF16)
    need = swr.proj_workspace_bytes(4, 64, 4096, synth.BF16)
    assert need > 0
    wd = u8(w.raw())
    x = torch.zeros((4, 4096), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(swr.SwrError) as e:
        swr.proj_forward(wd, synth.BF16, None, 64, 4096, x, y, workspace=ws)
    assert e.value.code == swr.E_CAPACITY


def test_full_size_projection_layer_sampled_rows():
    """The 8 FP8 projections of one replicated attention layer at M=16, through
    views of one reassembled slot; the oracle recomputes a sample of output
    columns of every projection."""
    wl = synth.ATTN_PROJECTIONS
    note("full-size projection layer M=16")
    ws = wl.layer_weights(0)
    shp = [(o, i, d) for _, o, i, d in wl.weights]
    views, lay = swr.plan_layer(shp, wl.n_chunks)
    src = [u8(w.raw()) for w in ws]
    chunks = [torch.empty(lay["chunk_bytes"], dtype=torch.uint8, device=DEV) for _ in range(wl.n_chunks)]
    swr.pack_layer(lay, views, src, chunks)
    del src
    slot = torch.empty(lay["total_bytes"], dtype=torch.uint8, device=DEV)
    swr.reassemble_into_slot(chunks, lay["chunk_bytes"], slot)
    m = 16
    xs = {}
    rng = np.random.default_rng(0)
    for j, (w, v) in enumerate(zip(ws, views)):
        k, o = w.in_features, w.out_features
        if k not in xs:
            xs[k] = synth.activations(synth.seed_for(3, 0, 50 + len(xs)), m, k)
        x = xs[k]
        y = torch.empty((m, o), dtype=torch.bfloat16, device=DEV)
        nb = swr.proj_workspace_bytes(m, o, k, w.dtype)
        wsp = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
        swr.proj_forward(slot.data_ptr() + v["offset"], w.dtype, f32(w.scale), o, k, bf16(x), y, workspace=wsp)
        torch.cuda.synchronize()
        cols = np.sort(rng.choice(o, size=min(o, 96), replace=False))
        sub = np.ascontiguousarray(w.data[cols])
        ref = gemm.proj_f64(x, sub, w.dtype, len(cols), k, w.scale[cols])
        assert_close_rows(values(y)[:, cols], ref, what=f"projection {j} [{o}x{k}]")


@pytest.mark.parametrize("o,k,m", [(16452, 512, 5), (20000, 256, 16), (16400, 768, 1)])
def test_many_row_blocks_at_few_tokens(o, k, m):
    """FP8 weights with more than two waves of 32-row blocks at <= 16 tokens:
    the planner takes 64-row blocks at two workgroups per CU; ragged rows."""
    note(f"many row blocks {o}x{k} m={m}")
    w = synth.weight(synth.seed_for(18, o % 97, 0), o, k, synth.FP8)
    x = synth.activations(synth.seed_for(18, o % 97, 50), m, k)
    y = torch.full((m, o), float("nan"), dtype=torch.bfloat16, device=DEV)
    nb = swr.proj_workspace_bytes(m, o, k, synth.FP8)
    wsp = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
    swr.proj_forward(u8(w.raw()), synth.FP8, f32(w.scale), o, k, bf16(x), y, workspace=wsp)
    torch.cuda.synchronize()
    ref = gemm.proj_f64(x, w.raw(), synth.FP8, o, k, w.scale)
    assert_close_rows(values(y), ref, what=f"{o}x{k} m={m}")


@pytest.mark.parametrize("workspace", [True, False])
@pytest.mark.parametrize("o,k,m", [(10304, 512, 1), (10304, 512, 8), (10304, 512, 13), (10304, 512, 16),
                                   (8192, 7168, 16), (6144, 14336, 9), (6144, 14336, 13)])
def test_one_token_block_on_eight_waves(o, k, m, workspace):
    """FP8 weights at one token block, where the planner takes the eight-wave
    kernel with activations through LDS: 64-row blocks shortened to fill the
    CUs (10304 rows: 44-row blocks, the last of 8), tokens past M inside the
    16-token block, K split into partial sums with a workspace from 9 tokens
    (8192 x 7168, 6144 x 14336) and the four-wave plan without one or below
    9 tokens.  Sampled output columns where the oracle would be slow."""
    note(f"one token block, eight waves {o}x{k} m={m} workspace={workspace}")
    w = synth.weight(synth.seed_for(19, o % 97, k % 89), o, k, synth.FP8)
    x = synth.activations(synth.seed_for(19, o % 97, 50), m, k)
    y = values(_run_proj(w, x, workspace=workspace))
    cols = np.arange(o) if o * k <= (1 << 23) else np.sort(np.random.default_rng(3).choice(o, 512, replace=False))
    ref = gemm.proj_f64(x, np.ascontiguousarray(w.data[cols]), synth.FP8, len(cols), k, w.scale[cols])
    assert_close_rows(y[:, cols], ref, what=f"{o}x{k} m={m} workspace={workspace}")


@pytest.mark.parametrize("y_fp32", [False, True])
@pytest.mark.parametrize("m", [8, 16])
def test_one_token_block_on_eight_waves_strided(m, y_fp32):
    """The eight-wave plan at one token block with row strides on both sides
    (ldx = K + 64, ldy = out + 64) and fp32 output: only the first out
    columns of each Y row are written."""
    o, k = 10304, 512
    note(f"one token block, eight waves, strided {o}x{k} m={m} y_fp32={y_fp32}")
    w = synth.weight(synth.seed_for(19, 1, 0), o, k, synth.FP8)
    x = synth.activations(synth.seed_for(19, 1, 50), m, k)
    ldy = o + 64
    wd, sd = u8(w.raw()), f32(w.scale)
    xb = np.zeros((m, k + 64), np.uint16)
    xb[:, :k] = x
    y = torch.full((m, ldy), float("nan"), dtype=torch.float32 if y_fp32 else torch.bfloat16, device=DEV)
    nb = swr.proj_workspace_bytes(m, o, k, synth.FP8)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
    swr.proj_forward(wd, synth.FP8, sd, o, k, bf16(xb), y, m=m, ldx=k + 64, ldy=ldy, y_fp32=y_fp32, workspace=ws)
    torch.cuda.synchronize()
    yv = values(y)
    assert np.isnan(yv[:, o:]).all(), "columns past out_f were written"
    ref = gemm.proj_f64(x, w.raw(), synth.FP8, o, k, w.scale)
    assert_close_rows(yv[:, :o], ref, what=f"strided {o}x{k} m={m} y_fp32={y_fp32}")


@pytest.mark.parametrize("o,k,dt,m", [
    (1000, 512, synth.FP8, 300),     # row tail and token tail in the tiled kernel
    (2048, 1024, synth.BF16, 513),
    (384, 192, synth.FP8, 257),      # 3 K tiles, 128-row weight tiles
    (4096, 256, synth.BF16, 1024),   # 256-row weight tiles
    (300, 64, synth.BF16, 260),      # a single K tile: two BF16 steps, no full ring cycle
    (640, 192, synth.BF16, 300),     # six BF16 steps: one ring cycle and a tail of two
    (200, 64, synth.FP8, 270),       # a single FP8 step
    (320, 128, synth.FP8, 270),      # two FP8 steps: no full ring cycle
    (4096, 256, synth.FP8, 600),     # four FP8 steps with 256-row tiles: one ring cycle and a tail of one
    (2000, 320, synth.FP8, 513),     # five FP8 steps: one ring cycle and a tail of two
    (6144, 512, synth.FP8, 4096),    # FP8 weights in 128-token x 256-row tiles (the 4096-token down GEMM's shape class)
    (6144, 320, synth.FP8, 4000),    # the same tiles with a token tail and five steps
    (8192, 192, synth.BF16, 4096),   # BF16, 256-row tiles: three double steps (one cycle of two and a tail)
    (8192, 128, synth.BF16, 4096),   # BF16, 256-row tiles: two double steps
])
def test_tiled_prefill_parity(o, k, dt, m):
    note(f"tiled proj o={o} k={k} {dt} m={m}")
    w = synth.weight(synth.seed_for(14, 0, o % 89), o, k, dt)
    x = synth.activations(synth.seed_for(14, 0, 50), m, k)
    y = values(_run_proj(w, x))
    ref = gemm.proj_f64(x, w.raw(), dt, o, k, w.scale)
    assert_close_rows(y, ref, what=f"tiled {o}x{k} {dt} m={m}")


@pytest.mark.parametrize("dt", [synth.BF16, synth.FP8])
@pytest.mark.parametrize("o,pad,y_fp32", [(1000, 64, False), (1004, 64, False), (1000, 4, False),
                                          (1000, 64, True), (1002, 62, True), (1000, 2, True)])
def test_tiled_strided_output(o, pad, y_fp32, dt):
    """Tiled kernels writing into Y rows of ldy = out + pad: with every row
    16-byte aligned (ldy a multiple of 8 for BF16, of 4 for fp32) the outputs
    leave through LDS in 16-byte stores (out = 1004 in BF16 and 1002 in fp32
    end in a partial piece), otherwise one element per store.  Nothing past
    column out of a row is written."""
    k, m = 192, 300
    note(f"tiled strided output o={o} pad={pad} y_fp32={y_fp32} {dt} m={m}")
    w = synth.weight(synth.seed_for(14, 3, o % 89), o, k, dt)
    x = synth.activations(synth.seed_for(14, 3, 50), m, k)
    y = torch.full((m, o + pad), float("nan"), dtype=torch.float32 if y_fp32 else torch.bfloat16, device=DEV)
    swr.proj_forward(u8(w.raw()), dt, f32(w.scale) if w.scale is not None else None, o, k, bf16(x), y, m=m,
                     ldx=k, ldy=o + pad, y_fp32=y_fp32)
    torch.cuda.synchronize()
    yv = values(y)
    assert np.isnan(yv[:, o:]).all(), "columns past out_f were written"
    ref = gemm.proj_f64(x, w.raw(), dt, o, k, w.scale)
    assert_close_rows(yv[:, :o], ref, what=f"tiled strided {o}x{k} {dt} m={m} ldy={o + pad}")


@pytest.mark.parametrize("dt", [synth.BF16, synth.FP8])
def test_tiled_fp32_output_large(dt):
    """fp32 outputs at 4096 tokens x 6144 rows: for FP8 weights the first 4096
    rows run as a whole wave of 256 x 256 tiles and the last 2048 as
    128-token tiles, both through the fp32 LDS epilogue; for BF16 weights
    256 x 128 tiles.  Every output is checked."""
    o, k, m = 6144, 512, 4096
    note(f"tiled fp32 output o={o} k={k} {dt} m={m}")
    w = synth.weight(synth.seed_for(14, 4, 0), o, k, dt)
    x = synth.activations(synth.seed_for(14, 4, 50), m, k)
    y = values(_run_proj(w, x, y_fp32=True))
    ref = gemm.proj_f64(x, w.raw(), dt, o, k, w.scale)
    assert_close_rows(y, ref, what=f"tiled fp32 {o}x{k} {dt} m={m}")


@pytest.mark.parametrize("dt", [synth.BF16, synth.FP8])
def test_tiled_last_wave_in_half_tiles(dt):
    """2048 tokens x 16484 rows: 8 x 65 = 520 tiles of 256 x 256, a last wave
    of 8 on 256 CUs, so the first 16384 rows run as 512 full tiles and the
    last 100 as 128-row tiles in a second launch.  Every column of the tail
    and a sample of the rest are checked."""
    o, k, m = 16484, 128, 2048
    note(f"tiled last wave in half tiles o={o} k={k} {dt} m={m}")
    w = synth.weight(synth.seed_for(14, 2, 0), o, k, dt)
    x = synth.activations(synth.seed_for(14, 2, 50), m, k)
    y = values(_run_proj(w, x))
    rng = np.random.default_rng(5)
    cols = np.sort(np.concatenate([rng.choice(16384, 412, replace=False), np.arange(16384, o)]))
    raw = w.raw().reshape(o, -1)
    ref = gemm.proj_f64(x, np.ascontiguousarray(raw[cols]), dt, len(cols), k,
                        None if w.scale is None else w.scale[cols])
    assert_close_rows(y[:, cols], ref, what=f"tiled {o}x{k} {dt} m={m} sampled columns")


@pytest.mark.parametrize("dt", [synth.BF16, synth.FP8])
def test_tiled_prefill_x_beyond_4gib(dt):
    """X of 131372 tokens x 16384 (4.01 GiB of bf16) runs in three launches,
    each spanning less than 2 GiB (the tiled kernels address X with 32-bit
    buffer offsets); tokens on both sides of each split and at the ends are
    checked."""
    o, k, m, base_rows = 384, 16384, 131372, 512
    assert m * k * 2 >= 1 << 32
    note(f"tiled proj beyond 4 GiB of X: o={o} k={k} {dt} m={m}")
    w = synth.weight(synth.seed_for(14, 1, 0), o, k, dt)
    xb = synth.activations(synth.seed_for(14, 1, 50), base_rows, k)  # token t is row t % 512
    x = bf16(xb).repeat((m + base_rows - 1) // base_rows, 1)[:m].contiguous()
    y = torch.full((m, o), float("nan"), dtype=torch.bfloat16, device=DEV)
    swr.proj_forward(u8(w.raw()), dt, f32(w.scale) if w.scale is not None else None, o, k, x, y)
    torch.cuda.synchronize()
    del x
    part = ((1 << 31) - 1) // (k * 2) // 256 * 256
    toks = sorted({0, 1, 255, 256, part - 1, part, part + 1, part + 256, 2 * part - 1, 2 * part, 2 * part + 1,
                   m - 2, m - 1, 40000, 100000})
    got = values(y[toks])
    ref = gemm.proj_f64(xb[[t % base_rows for t in toks]], w.raw(), dt, o, k, w.scale)
    assert_close_rows(got, ref, what=f"tokens {toks}")


@pytest.mark.parametrize("dt", [synth.BF16, synth.FP8])
@pytest.mark.parametrize("hidden,inter,m", [(256, 320, 300), (512, 1024, 600), (128, 256, 4096),
                                            (256, 2048, 4096)])  # FP8 gate_up in 128-token x 256-row tiles
def test_tiled_prefill_mlp(dt, hidden, inter, m):
    note(f"tiled mlp h={hidden} i={inter} {dt} m={m}")
    gu = synth.weight(synth.seed_for(15, 0, 0), 2 * inter, hidden, dt)
    d = synth.weight(synth.seed_for(15, 0, 1), hidden, inter, dt)
    x = synth.activations(synth.seed_for(15, 0, 50), m, hidden)
    y = torch.empty((m, hidden), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(swr.mlp_workspace_bytes(m, hidden, inter, dt), dtype=torch.uint8, device=DEV)
    swr.mlp_forward(u8(gu.raw()), f32(gu.scale) if gu.scale is not None else None, u8(d.raw()),
                    f32(d.scale) if d.scale is not None else None, dt, hidden, inter, bf16(x), y, ws)
    torch.cuda.synchronize()
    _, _, ref = gemm.mlp_f64(x, gu.raw(), gu.scale, d.raw(), d.scale, dt, hidden, inter)
    assert_close_rows(values(y), ref, what=f"tiled mlp {hidden}/{inter} {dt} m={m}")


def _grouped(ws, xs, m, y_fp32=False):
    ys = [torch.full((max(m, 1), w.out_features), float("nan"), device=DEV,
                     dtype=torch.float32 if y_fp32 else torch.bfloat16) for w in ws]
    projs = [dict(w=u8(w.raw()), dtype=w.dtype, row_scale=f32(w.scale) if w.scale is not None else None,
                  out_f=w.out_features, in_f=w.in_features, x=bf16(xs[w.in_features]), y=y)
             for w, y in zip(ws, ys)]
    nb = swr.proj_grouped_workspace_bytes(projs, m)
    wsp = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV) if nb > 0 else None
    swr.proj_forward_grouped(projs, m, workspace=wsp)
    torch.cuda.synchronize()
    return nb, [y[:m] for y in ys]


GROUPS = [
    # (shapes, dtype): K mixes and ragged row counts; all stageable -> one launch
    ([(1000, 512), (300, 768), (64, 256), (2048, 1024)], synth.FP8),
    ([(512, 256), (100, 512), (777, 768)], synth.BF16),
    # K = 320 is not a multiple of 256: separate launches
    ([(640, 320), (300, 768), (100, 127)], synth.FP8),
]


@pytest.mark.parametrize("gi", range(len(GROUPS)))
@pytest.mark.parametrize("m", [1, 4, 13, 16, 17, 33, 64, 65])
def test_grouped_projection_parity(gi, m):
    shapes, dt = GROUPS[gi]
    note(f"grouped projections group={gi} m={m}")
    ws = [synth.weight(synth.seed_for(16, gi, j), o, k, dt) for j, (o, k) in enumerate(shapes)]
    xs = {k: synth.activations(synth.seed_for(16, gi, 50 + k % 97), m, k) for _, k in shapes}
    nb, ys = _grouped(ws, xs, m)
    if all(k % 256 == 0 for _, k in shapes) and m <= 64:
        assert nb == 0  # one launch, no K split
    for w, y in zip(ws, ys):
        ref = gemm.proj_f64(xs[w.in_features], w.raw(), w.dtype, w.out_features, w.in_features, w.scale)
        assert_close_rows(values(y), ref, what=f"grouped {w.out_features}x{w.in_features} {w.dtype} m={m}")


@pytest.mark.parametrize("m", [1, 8])
def test_grouped_eight_waves_below_13_tokens(m):
    """An FP8 group with 167 blocks of 128 rows takes the eight-wave group
    kernel below 13 tokens too (ragged rows, K of 512, 256 and 768)."""
    shapes = [(12800, 512), (8192, 256), (300, 768)]
    note(f"grouped eight waves below 13 tokens m={m}")
    ws = [synth.weight(synth.seed_for(16, 11, j), o, k, synth.FP8) for j, (o, k) in enumerate(shapes)]
    xs = {k: synth.activations(synth.seed_for(16, 11, 50 + k % 97), m, k) for _, k in shapes}
    nb, ys = _grouped(ws, xs, m)
    assert nb == 0  # one launch, no K split
    for w, y in zip(ws, ys):
        ref = gemm.proj_f64(xs[w.in_features], w.raw(), w.dtype, w.out_features, w.in_features, w.scale)
        assert_close_rows(values(y), ref, what=f"grouped {w.out_features}x{w.in_features} m={m}")


@pytest.mark.parametrize("dt", [synth.BF16, synth.FP8])
def test_grouped_last_wave_in_half_tiles(dt):
    """2048 tokens over projections of 8192, 6000 and 2300 rows (K = 128):
    8 x 65 = 520 tiles of 256 x 256, a last wave of 8, so one tile column
    of the last projection (its rows past 2048) runs as 128-row tiles in a
    second grouped launch.  Every column of that tail and a sample of the
    rest of each projection are checked."""
    m, k = 2048, 128
    shapes = [(8192, k), (6000, k), (2300, k)]
    note(f"grouped last wave in half tiles {dt} m={m}")
    ws = [synth.weight(synth.seed_for(16, 9, j), o, kk, dt) for j, (o, kk) in enumerate(shapes)]
    xs = {k: synth.activations(synth.seed_for(16, 9, 50), m, k)}
    nb, ys = _grouped(ws, xs, m)
    rng = np.random.default_rng(7)
    for w, y in zip(ws, ys):
        o = w.out_features
        cols = np.sort(np.unique(np.concatenate([rng.choice(o, 256, replace=False), np.arange(max(0, o - 300), o)])))
        raw = w.raw().reshape(o, -1)
        ref = gemm.proj_f64(xs[k], np.ascontiguousarray(raw[cols]), dt, len(cols), k,
                            None if w.scale is None else w.scale[cols])
        assert_close_rows(values(y)[:, cols], ref, what=f"grouped {o}x{k} {dt} m={m} sampled columns")


@pytest.mark.parametrize("y_fp32", [False, True])
@pytest.mark.parametrize("m", [16, 33])
def test_grouped_projection_strided(m, y_fp32):
    """FP8 group 0 with every X and Y a strided view (ldx = K + 64, ldy =
    out + 32): the eight-wave group reads only the first K columns of each
    token row and writes only the first out columns of each Y row."""
    shapes, dt = GROUPS[0]
    note(f"grouped projections strided m={m} y_fp32={y_fp32}")
    ws = [synth.weight(synth.seed_for(16, 7, j), o, k, dt) for j, (o, k) in enumerate(shapes)]
    xs = {k: synth.activations(synth.seed_for(16, 7, 50 + k % 97), m, k) for _, k in shapes}
    xd = {}
    for k, x in xs.items():
        xb = np.zeros((m, k + 64), np.uint16)
        xb[:, :k] = x
        xd[k] = bf16(xb)
    ys = [torch.full((m, w.out_features + 32), float("nan"), device=DEV,
                     dtype=torch.float32 if y_fp32 else torch.bfloat16) for w in ws]
    projs = [dict(w=u8(w.raw()), dtype=w.dtype, row_scale=f32(w.scale), out_f=w.out_features,
                  in_f=w.in_features, x=xd[w.in_features], y=y) for w, y in zip(ws, ys)]
    assert swr.proj_grouped_workspace_bytes(projs, m) == 0
    swr.proj_forward_grouped(projs, m)
    torch.cuda.synchronize()
    for w, y in zip(ws, ys):
        yv = values(y)
        assert np.isnan(yv[:, w.out_features:]).all(), "columns past out_f were written"
        ref = gemm.proj_f64(xs[w.in_features], w.raw(), w.dtype, w.out_features, w.in_features, w.scale)
        assert_close_rows(yv[:, :w.out_features], ref, what=f"grouped strided {w.out_features}x{w.in_features} m={m}")


@pytest.mark.parametrize("gi,y_fp32", [(0, False), (1, False), (0, True)])
@pytest.mark.parametrize("m", [65, 300, 600])
def test_grouped_prefill_one_launch_equals_separate(gi, y_fp32, m):
    """Prefill-sized groups (M > 64, K a multiple of 64) run as one launch of
    the tiled kernels over all the group's tiles.  Each projection must give
    the bits of its own swr_proj_forward call (the same K order per output,
    whichever tile width either launch picks) and meet the bar against the
    oracle on sampled token rows."""
    shapes, dt = GROUPS[gi]
    note(f"grouped prefill group={gi} fp32={y_fp32} m={m}")
    ws = [synth.weight(synth.seed_for(17, gi, j), o, k, dt) for j, (o, k) in enumerate(shapes)]
    xs = {k: synth.activations(synth.seed_for(17, gi, 50 + k % 97), m, k) for _, k in shapes}
    nb, ys = _grouped(ws, xs, m, y_fp32=y_fp32)
    assert nb == 0  # one launch, no scratch
    rows = np.random.default_rng(m).choice(m, size=min(m, 24), replace=False)
    for w, y in zip(ws, ys):
        y1 = torch.full_like(y, float("nan"))
        swr.proj_forward(u8(w.raw()), w.dtype, f32(w.scale) if w.scale is not None else None, w.out_features,
                         w.in_features, bf16(xs[w.in_features]), y1)
        torch.cuda.synchronize()
        bits = torch.int32 if y_fp32 else torch.int16
        assert torch.equal(y.view(bits), y1.view(bits)), f"{w.out_features}x{w.in_features} differs from one launch"
        ref = gemm.proj_f64(xs[w.in_features][rows], w.raw(), w.dtype, w.out_features, w.in_features, w.scale)
        assert_close_rows(values(y[rows]), ref, what=f"grouped prefill {w.out_features}x{w.in_features} m={m}")


def test_grouped_fp32_output_and_zero_tokens():
    note("grouped fp32 output, M=0")
    ws = [synth.weight(31, 320, 512, synth.FP8), synth.weight(32, 96, 256, synth.FP8)]
    xs = {512: synth.activations(33, 9, 512), 256: synth.activations(34, 9, 256)}
    _, ys = _grouped(ws, xs, 9, y_fp32=True)
    for w, y in zip(ws, ys):
        ref = gemm.proj_f64(xs[w.in_features], w.raw(), w.dtype, w.out_features, w.in_features, w.scale)
        assert_close_rows(values(y), ref, what="grouped fp32")
    y = torch.full((1, 320), 3.0, dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((1, 512), dtype=torch.bfloat16, device=DEV)
    swr.proj_forward_grouped([dict(w=u8(ws[0].raw()), dtype=synth.FP8, row_scale=f32(ws[0].scale), out_f=320,
                                   in_f=512, x=x, y=y)], 0)
    torch.cuda.synchronize()
    assert (y == 3.0).all()


@pytest.mark.parametrize("m", [4, 16])
def test_full_size_projection_layer_grouped(m):
    """The 8 FP8 projections of one replicated attention layer at M=4 and 16
    in ONE grouped call through views of one reassembled slot; the oracle
    recomputes a sample of output columns of every projection."""
    wl = synth.ATTN_PROJECTIONS
    note(f"full-size projection layer M={m}, grouped")
    ws = wl.layer_weights(1)
    shp = [(o, i, d) for _, o, i, d in wl.weights]
    views, lay = swr.plan_layer(shp, wl.n_chunks)
    src = [u8(w.raw()) for w in ws]
    chunks = [torch.empty(lay["chunk_bytes"], dtype=torch.uint8, device=DEV) for _ in range(wl.n_chunks)]
    swr.pack_layer(lay, views, src, chunks)
    del src
    slot = torch.empty(lay["total_bytes"], dtype=torch.uint8, device=DEV)
    swr.reassemble_into_slot(chunks, lay["chunk_bytes"], slot)
    xs, projs, ys = {}, [], []
    for j, (w, v) in enumerate(zip(ws, views)):
        k, o = w.in_features, w.out_features
        if k not in xs:
            xs[k] = synth.activations(synth.seed_for(3, 1, 50 + len(xs)), m, k)
        y = torch.empty((m, o), dtype=torch.bfloat16, device=DEV)
        ys.append(y)
        projs.append(dict(w=slot.data_ptr() + v["offset"], dtype=w.dtype, row_scale=f32(w.scale), out_f=o, in_f=k,
                          x=bf16(xs[k]), y=y))
    assert swr.proj_grouped_workspace_bytes(projs, m) == 0  # one launch
    swr.proj_forward_grouped(projs, m)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    for j, (w, y) in enumerate(zip(ws, ys)):
        o, k = w.out_features, w.in_features
        cols = np.sort(rng.choice(o, size=min(o, 96), replace=False))
        ref = gemm.proj_f64(xs[k], np.ascontiguousarray(w.data[cols]), w.dtype, len(cols), k, w.scale[cols])
        assert_close_rows(values(y)[:, cols], ref, what=f"grouped projection {j} [{o}x{k}]")
