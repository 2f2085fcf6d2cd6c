"""Storage codecs of the oracle, written from the number formats' definitions.

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use this package.  Nothing in the HIP library reads it.

Every stored value decodes exactly into float64 (binary32, bfloat16 and
fp8 e4m3 all embed in binary64), so the oracle sees the inputs with no
rounding at all.
"""
from __future__ import annotations

import numpy as np

__all__ = ["bf16_to_f64", "fp8_e4m3fn_to_f64", "decode_codes"]


def bf16_to_f64(codes: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32: sign, 8-bit exponent,
    7-bit fraction.  Widening the 16-bit pattern into the top of a 32-bit
    word gives the identical number."""
    c = np.asarray(codes, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return c.view(np.float32).astype(np.float64)


def fp8_e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP fp8 E4M3 ("fn": finite, no infinities).

    Fields: sign s (1 bit), exponent e (4 bits, bias 7), mantissa m (3 bits).
    e = 0: subnormal (-1)^s * (m / 8) * 2^(1 - 7);
    e > 0: normal    (-1)^s * (1 + m / 8) * 2^(e - 7);
    e = 15 and m = 7 is NaN (the only non-finite pattern), so the largest
    finite magnitude is (1 + 6/8) * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0,
                   (m / 8.0) * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def decode_codes(codes: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage codes ('f32', 'bf16', 'fp8') to float64."""
    if dtype == "f32":
        return np.asarray(codes, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(codes)
    if dtype == "fp8":
        return fp8_e4m3fn_to_f64(codes)
    raise ValueError(f"unknown storage type {dtype!r}")
