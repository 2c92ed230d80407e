"""Pins for the oracle's projection, MLP and sharded-matmul references.

Each pin is something other than the oracle's own formula: explicit loops
without BLAS, closed forms (one-hot rows, identity weights, hand-built
gate/up rows), torch's float64 ops, and the algebraic identities the pages
state (the PR report's intermediate-slice partial sums; the sharded-matrices
notes' column split and contraction split).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gemm, numerics


def _w(seed, o, i, dt):
    return synth.weight(seed, o, i, dt)


@pytest.mark.parametrize("dt", ["bf16", "fp8_e4m3fn"])
def test_proj_matches_loops(dt):
    w = _w(1, 37, 23, dt)
    x = synth.activations(2, 5, 23)
    y = gemm.proj_f64(x, w.raw(), dt, 37, 23, w.scale)
    rows, cols = [0, 2, 4], [0, 5, 17, 36]
    ref = gemm.proj_rows_bruteforce(x, w.raw(), dt, 37, 23, w.scale, rows, cols)
    np.testing.assert_allclose(y[np.ix_(rows, cols)], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("dt", ["bf16", "fp8_e4m3fn"])
def test_one_hot_row_selects_a_column(dt):
    # X row = e_k gives Y row = bf16(s * dec(W[:, k])) exactly.
    o, i, k = 40, 24, 7
    w = _w(3, o, i, dt)
    x = np.zeros((1, i), np.uint16)
    x[0, k] = 0x3F80  # 1.0
    y = gemm.proj(x, w.raw(), dt, o, i, w.scale)
    col = numerics.decode_weight(w.raw(), dt, o, i)[:, k]
    if w.scale is not None:
        col = col * w.scale.astype(np.float64)
    assert np.array_equal(y[0], numerics.f64_to_bf16_bits(col))


def test_identity_weight_returns_input():
    n = 128
    eye = np.where(np.eye(n, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    x = synth.activations(4, 6, n)
    assert np.array_equal(gemm.proj(x, eye, "bf16", n, n), x)


def test_scale_is_per_output_row():
    # Two rows with the same codes and different scales: outputs differ by the scale ratio.
    codes = np.tile(np.array([[0x38, 0x40, 0xB8]], np.uint8), (2, 1))  # 1, 2, -1
    x = np.array([[0x3F80, 0x3F80, 0x4040]], np.uint16)  # 1, 1, 3
    y = gemm.proj_f64(x, codes, "fp8_e4m3fn", 2, 3, np.array([1.0, 0.25], np.float32))
    assert y.tolist() == [[0.0, 0.0]]  # 1 + 2 - 3
    x2 = np.array([[0x4000, 0x3F80, 0x3F80]], np.uint16)  # 2, 1, 1
    y2 = gemm.proj_f64(x2, codes, "fp8_e4m3fn", 2, 3, np.array([1.0, 0.25], np.float32))
    assert y2.tolist() == [[3.0, 0.75]]


def test_m1_is_gemv():
    w = _w(5, 64, 48, "fp8_e4m3fn")
    x = synth.activations(6, 1, 48)
    y = gemm.proj_f64(x, w.raw(), "fp8_e4m3fn", 64, 48, w.scale)[0]
    wd = numerics.decode_weight(w.raw(), "fp8_e4m3fn", 64, 48)
    xv = numerics.bf16_to_f64(x)[0]
    ref = np.array([sum(float(a) * float(b) for a, b in zip(wd[r], xv)) for r in range(64)])
    np.testing.assert_allclose(y, ref * w.scale.astype(np.float64), rtol=1e-13, atol=1e-15)


def test_mlp_gate_comes_first():
    # gate row j reads x_a, up row j reads x_b: h_j = silu(x_a) * x_b (not silu(x_b) * x_a).
    hidden, inter = 4, 2
    one = 0x3F80
    wgu = np.zeros((2 * inter, hidden), np.uint16)
    wgu[0, 0] = one       # gate 0 <- x0
    wgu[1, 1] = one       # gate 1 <- x1
    wgu[2, 2] = one       # up 0   <- x2
    wgu[3, 3] = one       # up 1   <- x3
    wd = np.zeros((hidden, inter), np.uint16)
    wd[0, 0] = one
    wd[1, 1] = one
    xv = np.array([[0.5, -2.0, 3.0, 0.75]])
    x = numerics.f64_to_bf16_bits(xv)
    g, h, y = gemm.mlp_f64(x, wgu, None, wd, None, "bf16", hidden, inter)
    silu = lambda z: z / (1 + np.exp(-z))
    want_h = np.array([silu(0.5) * 3.0, silu(-2.0) * 0.75])
    assert np.array_equal(numerics.bf16_to_f64(h)[0], numerics.bf16_round(want_h))
    assert np.array_equal(y[0], np.r_[numerics.bf16_round(want_h), 0.0, 0.0])


@pytest.mark.parametrize("dt", ["bf16", "fp8_e4m3fn"])
def test_mlp_matches_torch_f64(dt):
    hidden, inter, m = 32, 48, 5
    gu = _w(7, 2 * inter, hidden, dt)
    d = _w(8, hidden, inter, dt)
    x = synth.activations(9, m, hidden)
    _, h, y = gemm.mlp_f64(x, gu.raw(), gu.scale, d.raw(), d.scale, dt, hidden, inter)
    xt = torch.from_numpy(numerics.bf16_to_f64(x))
    wgu = torch.from_numpy(numerics.decode_weight(gu.raw(), dt, 2 * inter, hidden))
    wd = torch.from_numpy(numerics.decode_weight(d.raw(), dt, hidden, inter))
    if gu.scale is not None:
        wgu = wgu * torch.from_numpy(gu.scale.astype(np.float64))[:, None]
        wd = wd * torch.from_numpy(d.scale.astype(np.float64))[:, None]
    gt = xt @ wgu.T
    ht = (torch.nn.functional.silu(gt[:, :inter]) * gt[:, inter:]).to(torch.bfloat16).double()
    yt = ht @ wd.T
    assert np.array_equal(numerics.bf16_to_f64(h), ht.numpy())
    np.testing.assert_allclose(y, yt.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dt", ["bf16", "fp8_e4m3fn"])
def test_mlp_intermediate_slices_add_up(dt):
    # The PR report's equivalence test: slicing the intermediate dimension
    # across 4 ranks and summing the partial MLPs gives the replicated MLP.
    hidden, inter, ranks = 16, 12, 4
    gu = _w(10, 2 * inter, hidden, dt)
    d = _w(11, hidden, inter, dt)
    x = synth.activations(12, 12, hidden)
    _, _, full = gemm.mlp_f64(x, gu.raw(), gu.scale, d.raw(), d.scale, dt, hidden, inter)
    sh = inter // ranks
    d_arr = d.data  # [hidden, inter] elements
    parts = [gemm.mlp_intermediate_slice_f64(x, gu.data, gu.scale, d_arr, d.scale, dt, hidden, inter,
                                             r * sh, (r + 1) * sh) for r in range(ranks)]
    np.testing.assert_allclose(gemm.sum_partials(parts), full, rtol=1e-12, atol=1e-12)


def test_sharded_matmul_layouts_agree():
    b, dd, f, n = 16, 64, 96, 8
    x, w_t = synth.sharded_matmul_inputs(b, dd, f, config=99)
    full = gemm.matmul_f64(x, w_t)
    cols = gemm.concat_columns([gemm.matmul_f64(x, s) for s in gemm.column_shards(w_t, n)])
    np.testing.assert_allclose(cols, full, rtol=1e-13, atol=1e-13)
    parts = [gemm.matmul_f64(xs, ws) for xs, ws in gemm.contraction_shards(x, w_t, n)]
    np.testing.assert_allclose(gemm.sum_partials(parts), full, rtol=1e-12, atol=1e-12)
    # explicit loops on a few outputs
    xf, wf = numerics.bf16_to_f64(x), numerics.bf16_to_f64(w_t)
    for (r, c) in [(0, 0), (3, 95), (15, 40)]:
        assert abs(full[r, c] - sum(xf[r, k] * wf[c, k] for k in range(dd))) < 1e-12


def test_row_tolerance():
    y = np.array([[0.5, -0.2], [30.0, -100.0]])
    assert gemm.row_tolerance(y).ravel().tolist() == [1e-2, 1.0]


def test_mlp_fp8act_hand_case():
    """The FP8-activation MLP composition (quantise X -> gate_up -> SiLU*up ->
    bf16 h -> quantise h -> down) on two hand-built tokens whose every
    rounding is worked out below, so that quantising G instead of h, skipping
    h's or X's quantisation, putting s_x on the down GEMM, dropping s_h or
    swapping gate and up each changes an output.

    Weights (E4M3FN codes: 0x38 = 1, 0x30 = 0.5, 0x28 = 0.25, 0 = 0):
      gate rows 0, 1 = [0.25, 0, 0, 0]      scale 1   -> g = x0 / 4
      up row 0       = [0, 1, 0, 0]         scale 8   -> u0 = 8 x1
      up row 1       = [0, 0, 1, 0.5]       scale 0.5 -> u1 = (x2 + x3/2) / 2
      down rows      = [1, 0], [0, 0.5], [0.25, 0.25], [0, 0]; scales 1, 1, 2, 1
    g is 112 or 56, where z / (1 + exp(-z)) == z exactly in float64.

    Token 0: x = [448, 1, -28, 8]; amax 448 -> s_x = 1, every x is an E4M3
      value.  g = 112, u = [8, -12], h = [896, -1344] (both exact in bf16).
      s_h = 1344 / 448 = 3; h / s_h = [298.67, -448] -> codes 288, -448
      (E4M3 spacing is 32 in [256, 448]), so dequantised h = [864, -1344].
      y = [864, -672, 2 * (216 - 336), 0] = [864, -672, -240, 0].
    Token 1: x = [224, 0.30078125, 3, -1]; s_x = 0.5; x / s_x =
      [448, 0.6015625, 6, -2] -> 0.6015625 lies between 0.5625 and 0.625
      (spacing 1/16) and is nearer 0.625, so dequantised x1 = 0.3125.
      g = 56, u = [2.5, 1.25], h = [140, 70]; s_h = 140 / 448 = 0.3125,
      h / s_h = [448, 224] exact.  y = [140, 35, 2 * (35 + 17.5), 0].
    The BF16-activation MLP of the same inputs gives token 0 y0 = 896 and
    token 1 y0 = bf16(56 * 8 * 0.30078125 = 134.75) = 135: both differ."""
    hidden, inter = 4, 2
    wgu = np.array([[0x28, 0, 0, 0], [0x28, 0, 0, 0], [0, 0x38, 0, 0], [0, 0, 0x38, 0x30]], np.uint8)
    s_gu = np.array([1.0, 1.0, 8.0, 0.5], np.float32)
    wd = np.array([[0x38, 0], [0, 0x30], [0x28, 0x28], [0, 0]], np.uint8)
    s_d = np.array([1.0, 1.0, 2.0, 1.0], np.float32)
    x = numerics.f64_to_bf16_bits(np.array([[448.0, 1.0, -28.0, 8.0], [224.0, 0.30078125, 3.0, -1.0]]))
    assert numerics.bf16_to_f64(x)[1, 1] == 0.30078125  # representable in bf16
    q_x, s_x, g, h, q_h, s_h, y = gemm.mlp_fp8act_f64(x, wgu, s_gu, wd, s_d, hidden, inter)
    assert s_x.tolist() == [1.0, 0.5]
    assert (numerics.fp8_to_f64(q_x) * s_x[:, None]).tolist() == [[448, 1, -28, 8], [224, 0.3125, 3, -1]]
    assert g.tolist() == [[112, 112, 8, -12], [56, 56, 2.5, 1.25]]
    assert numerics.bf16_to_f64(h).tolist() == [[896, -1344], [140, 70]]
    assert s_h.tolist() == [3.0, 0.3125]
    assert (numerics.fp8_to_f64(q_h) * s_h[:, None]).tolist() == [[864, -1344], [140, 70]]
    assert y.tolist() == [[864, -672, -240, 0], [140, 35, 105, 0]]
    # the BF16-activation MLP of the same inputs differs where the pages' path
    # keeps activations unquantised
    _, _, y16 = gemm.mlp_f64(x, wgu, s_gu, wd, s_d, "fp8_e4m3fn", hidden, inter)
    assert y16[0, 0] == 896 and numerics.bf16_round(y16[1, 0]) == 135


def test_mlp_fp8act_equals_w8a16_on_representable_activations():
    """When both quantisations are exact, the FP8-activation MLP equals the
    pages' W8A16 MLP bit for bit.  Token row: x0 = 256 * 2**e, x1 = +-448 *
    2**e (the row maximum, so s_x = 2**e) and E4M3 values times 2**e
    elsewhere.  gate rows: 0.25 * x0 = 64 * 2**e (>= 64, where silu(z) == z
    in float64); up row j: x_{j+1}.  So h_j = 64 * 2**e * x_{j+1}, its row
    maximum is |h_0| = 448 * 64 * 4**e, s_h = 64 * 4**e and h / s_h are the
    E4M3 codes of x_{j+1} / 2**e: exact.  Power-of-two scales commute with
    float64 rounding, so the two compositions give identical bits; a wrong
    scale (s_x on the down GEMM, a missing s_x or s_h) would not."""
    rng = np.random.default_rng(5)
    hidden, inter, m = 8, 5, 12
    e = rng.integers(0, 3, size=(m, 1)).astype(np.float64)
    mags = numerics.fp8_to_f64(rng.integers(0x08, 0x7F, size=(m, hidden)).astype(np.uint8))
    signs = np.where(rng.integers(0, 2, size=(m, hidden)) == 1, -1.0, 1.0)
    xv = mags * signs
    xv[:, 0] = 256.0
    xv[:, 1] = 448.0 * signs[:, 1]
    xv = xv * 2.0 ** e
    x = numerics.f64_to_bf16_bits(xv)
    assert np.array_equal(numerics.bf16_to_f64(x), xv)
    wgu = np.zeros((2 * inter, hidden), np.uint8)
    wgu[:inter, 0] = 0x28  # 0.25
    for j in range(inter):
        wgu[inter + j, j + 1] = 0x38  # 1.0
    s_gu = np.ones(2 * inter, np.float32)
    wd = rng.integers(0, 0x7F, size=(hidden, inter)).astype(np.uint8)
    s_d = (2.0 ** rng.integers(-3, 3, size=hidden)).astype(np.float32)
    q_x, s_x, g, h, q_h, s_h, y = gemm.mlp_fp8act_f64(x, wgu, s_gu, wd, s_d, hidden, inter)
    _, h16, y16 = gemm.mlp_f64(x, wgu, s_gu, wd, s_d, "fp8_e4m3fn", hidden, inter)
    assert s_x.tolist() == (2.0 ** e[:, 0]).tolist()
    assert s_h.tolist() == (64.0 * 4.0 ** e[:, 0]).tolist()
    assert np.array_equal(numerics.fp8_to_f64(q_h) * s_h[:, None].astype(np.float64), numerics.bf16_to_f64(h))
    assert np.array_equal(h, h16)
    assert np.array_equal(y, y16)
