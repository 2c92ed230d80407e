"""Pins for the oracle's number formats: E4M3FN table, BF16 rounding, SiLU.

The E4M3FN table is checked against values fixed by the OCP FP8 definition
and against torch's float8_e4m3fn decoder (an independent library routine).
BF16 rounding is checked on hand-made ties and against torch's fp32 -> bf16
conversion, which rounds to nearest even.
"""
import math

import numpy as np
import pytest
import torch

from oracle import gemm, numerics


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
    (0x40, 2.0), (0x3C, 1.5), (0x7E, 448.0), (0x77, 240.0), (0xB8, -1.0), (0xFE, -448.0),
])
def test_fp8_known_codes(code, value):
    assert numerics.FP8_E4M3FN_TABLE[code] == value


def test_fp8_nan_and_signed_zero():
    t = numerics.FP8_E4M3FN_TABLE
    assert math.isnan(t[0x7F]) and math.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2
    assert t[0x80] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0


def test_fp8_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = numerics.FP8_E4M3FN_TABLE
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(ref[~both_nan], ours[~both_nan])
    assert np.array_equal(np.isnan(ref), np.isnan(ours))


def test_fp8_positive_codes_increase():
    t = numerics.FP8_E4M3FN_TABLE[:0x7F]
    assert (np.diff(t) > 0).all()


def test_bf16_ties_to_even():
    one = 1.0
    ulp = 2.0 ** -7
    cases = {
        one + ulp / 2: one,                 # tie, 1.0 has an even mantissa
        one + 3 * ulp / 2: one + 2 * ulp,   # tie, rounds up to the even neighbour
        one + ulp / 2 + 2.0 ** -20: one + ulp,
        -(one + ulp / 2): -one,
        3.0: 3.0,
        2.0 ** -133: 2.0 ** -133,           # smallest subnormal
        2.0 ** -134: 0.0,                   # tie with zero -> even (zero)
        1.5 * 2.0 ** -133: 2.0 * 2.0 ** -133,
        3.4e38: np.inf,
    }
    for x, want in cases.items():
        got = float(numerics.bf16_round(np.array([x]))[0])
        assert got == want, (x, got, want)


def test_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000),
                        rng.standard_normal(1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = numerics.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(ref, ours)
    back = numerics.bf16_to_f64(ours)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 2.5])
    s = numerics.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    assert abs(s[2] - (-1.0 / (1.0 + math.exp(1.0)))) < 1e-15
    assert abs(s[3] - 40.0) < 1e-12 and abs(s[4]) < 1e-15
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-15, atol=1e-300)


# ---------------------------------------------------------------- FP8 activations (E4M3FN encoding)

def _finite_codes():
    return [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_e4m3_encode_round_trips_every_finite_code():
    codes = np.array(_finite_codes(), dtype=np.uint8)
    vals = numerics.fp8_to_f64(codes).astype(np.float32)
    assert np.array_equal(numerics.e4m3_encode(vals), codes)


def test_e4m3_encode_midpoints_tie_to_the_even_code():
    """Between consecutive finite values the midpoint (exact in binary32: one
    more mantissa bit) goes to the even code, and the binary32 neighbours of
    the midpoint to the nearer value."""
    pos = numerics.FP8_E4M3FN_TABLE[:0x7F]
    for c in range(0x7E):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)
        assert float(mid) == (pos[c] + pos[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert numerics.e4m3_encode(np.array([mid]))[0] == even, hex(c)
        assert numerics.e4m3_encode(np.array([-mid]))[0] == even | 0x80
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert numerics.e4m3_encode(np.array([below]))[0] == c
        assert numerics.e4m3_encode(np.array([above]))[0] == c + 1


def test_e4m3_encode_saturates_and_keeps_the_sign():
    v = np.array([448.0, 463.9, 464.0, 1e30, np.float32(3.4e38), -448.0, -1e30, 0.0, -0.0], dtype=np.float32)
    assert numerics.e4m3_encode(v).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80]


def test_e4m3_encode_matches_brute_force_nearest():
    """Random binary32 values against a plain loop over the 126 positive finite
    values: nearest, ties to the even code."""
    rng = np.random.default_rng(11)
    vals = np.concatenate([rng.standard_normal(300) * 100, rng.standard_normal(300) * 0.01,
                           rng.uniform(-2 ** -6, 2 ** -6, 200)]).astype(np.float32)
    pos = numerics.FP8_E4M3FN_TABLE[:0x7F]
    got = numerics.e4m3_encode(vals)
    for v, g in zip(vals.tolist(), got.tolist()):
        a = min(abs(v), 448.0)
        best = None
        for c in range(0x7F):
            d = abs(a - pos[c])
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        want = best[1] | (0x80 if np.signbit(np.float32(v)) else 0)
        assert g == want, (v, hex(g), hex(want))


def test_quantize_rows_lossless_for_representable_rows_and_zero_rows():
    """A row of E4M3FN values times 2**k whose largest magnitude is 448 * 2**k
    has scale 2**k exactly and quantises without loss; an all-zero row gets
    scale 1 and zero codes."""
    rng = np.random.default_rng(12)
    codes = rng.choice(np.array(_finite_codes(), dtype=np.uint8), size=(4, 96))
    codes[:, 5] = 0x7E  # the row maximum is 448
    rows = numerics.fp8_to_f64(codes) * (2.0 ** np.array([-3, 0, 2, 7]))[:, None]
    x = np.vstack([rows, np.zeros((1, 96))])
    q, s = numerics.quantize_rows_e4m3(x)
    assert s.tolist() == [2.0 ** -3, 1.0, 4.0, 128.0, 1.0]
    np.testing.assert_array_equal(numerics.fp8_to_f64(q[:4]) * s[:4, None], rows)
    assert not q[4].any()


def test_fp8act_projection_equals_the_bf16_oracle_on_representable_tokens():
    """With tokens that quantise without loss, the FP8-activation projection is
    the W8A16 projection of the same tokens (both float64)."""
    rng = np.random.default_rng(13)
    o, k = 48, 80
    codes = rng.choice(np.array(_finite_codes(), dtype=np.uint8), size=(3, k))
    codes[:, 0] = 0x7E
    x = numerics.fp8_to_f64(codes) * 0.25  # bf16-representable too (3 mantissa bits)
    w = rng.integers(0, 0x7E, size=(o, k)).astype(np.uint8)
    s = rng.uniform(0.001, 0.01, o).astype(np.float32)
    _, _, y = gemm.proj_fp8act_f64(x, w.reshape(-1), o, k, s)
    ref = gemm.proj_f64(numerics.f64_to_bf16_bits(x), w.reshape(-1), "fp8_e4m3fn", o, k, s)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-300)


def test_e4m3_encode_matches_torch_cast_in_range():
    """torch's float32 -> float8_e4m3fn cast (round to nearest even) agrees on
    values within the finite range, including every midpoint."""
    rng = np.random.default_rng(14)
    pos = numerics.FP8_E4M3FN_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = np.concatenate([rng.uniform(-448, 448, 2000), rng.standard_normal(2000) * 0.05, mids, -mids])
    vals = vals.astype(np.float32)
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(numerics.e4m3_encode(vals), want)
