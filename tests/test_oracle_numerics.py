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

from oracle import numerics


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
