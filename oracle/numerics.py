"""Number formats used by the path -- oracle (test infrastructure only).

* BF16: 1 sign, 8 exponent, 7 mantissa bits (the upper half of an IEEE
  binary32).  Results are rounded to BF16 with round-to-nearest, ties to
  even, straight from float64.
* FP8 E4M3FN (OCP 8-bit floating point, E4M3 "FN" variant): 1 sign,
  4 exponent (bias 7), 3 mantissa bits; exponent field 0 is subnormal
  (2**-6 * m/8); there is no infinity; S.1111.111 is NaN; the largest finite
  magnitude is 448.  The weight-sharding page (section on loading, quantised
  variants) keeps FP8 weight bytes in the flat buffer and the per-row scales
  outside it; the weight value is decode(code) * scale[row].
* SiLU(z) = z / (1 + exp(-z)) (the gate activation of the shared-expert MLP,
  vLLM PR #50656 report, test code section).
* FP8 activations (an option beyond the pages, which keep activations in
  BF16): a token row x is quantised to E4M3FN codes with one fp32 scale,
  s = amax(|x|) / 448 in binary32 (s = 1 for an all-zero row); each code is
  the E4M3FN value nearest to the binary32 quotient x / s, ties to the even
  code, magnitudes above 448 saturating to 448 -- the definition written out
  as an argmin over the format's value table, not as bit arithmetic.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest BF16 value (ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)  # x = m * 2**e with 0.5 <= |m| < 1
    # 8 significant bits for normal numbers; below 2**-126 the step is 2**-133
    q = np.maximum(e - 8, -133)
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    return np.where(np.abs(y) > BF16_MAX, np.copysign(np.inf, x), y)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    y = bf16_round(x).astype(np.float32)  # exact: every BF16 value is a binary32 value
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def fp8_e4m3fn_value(code: int) -> float:
    """Value of one E4M3FN code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * 2.0 ** (1 - 7) * (man / 8.0)
    return sign * 2.0 ** (exp - 7) * (1.0 + man / 8.0)


FP8_E4M3FN_TABLE = np.array([fp8_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def fp8_to_f64(codes: np.ndarray) -> np.ndarray:
    return FP8_E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_weight(raw: np.ndarray, dtype: str, out_f: int, in_f: int) -> np.ndarray:
    """Raw weight storage (bf16 bit patterns or fp8 codes) -> float64 [out, in]."""
    if dtype == "bf16":
        return bf16_to_f64(np.asarray(raw).view(np.uint16).reshape(out_f, in_f))
    if dtype == "fp8_e4m3fn":
        return fp8_to_f64(np.asarray(raw).view(np.uint8).reshape(out_f, in_f))
    raise ValueError(f"unknown dtype {dtype!r}")


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


# the non-negative finite E4M3FN values, increasing with the code 0x00..0x7E
_E4M3_POS = FP8_E4M3FN_TABLE[:0x7F]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """E4M3FN codes of binary32 values: nearest finite value, ties to the even
    code, magnitudes above 448 saturate; the sign bit is the input's."""
    y = np.asarray(y, dtype=np.float32)
    a = np.minimum(np.abs(y).astype(np.float64), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << np.uint8(7))


def quantize_rows_e4m3(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row E4M3FN quantisation of float values (bf16 values as float64 or
    float32): returns (codes uint8 [rows, cols], scales float32 [rows])."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (x32 / s[:, None]).astype(np.float32)
    return e4m3_encode(q), s
