"""Storage codecs of the oracle, written from the number formats' definitions.

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use this package.  Nothing in the HIP library reads it.

Every stored value decodes exactly into float64 (binary32, bfloat16 and
fp8 e4m3 all embed in binary64), so the oracle sees the inputs with no
rounding at all.
"""
from __future__ import annotations

import numpy as np

__all__ = ["bf16_to_f64", "fp8_e4m3fn_to_f64", "int4_to_f64", "decode_codes",
           "round_to_grid", "f64_to_bf16_codes", "f64_to_fp8_e4m3fn_codes", "f64_to_int4_codes", "encode_codes"]


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


def int4_to_f64(codes: np.ndarray) -> np.ndarray:
    """Packed signed 4-bit integers: byte i of a row holds elements 2i (low
    nibble) and 2i + 1 (high nibble), each a two's-complement value in
    [-8, 7].  A [..., n] byte array decodes to [..., 2n] float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    lo = c & 0xF
    hi = (c >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def decode_codes(codes: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage codes ('f32', 'bf16', 'fp8', 'int4') to float64 (int4:
    the last axis doubles)."""
    if dtype == "f32":
        return np.asarray(codes, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(codes)
    if dtype == "fp8":
        return fp8_e4m3fn_to_f64(codes)
    if dtype == "int4":
        return int4_to_f64(codes)
    raise ValueError(f"unknown storage type {dtype!r}")


# ----------------------------------------------------------------------------
# encoders (round to nearest, ties to even), from the same definitions
# ----------------------------------------------------------------------------

def round_to_grid(x: np.ndarray, frac_bits: int, emin: int) -> np.ndarray:
    """Round float64 values to the nearest number with ``frac_bits`` fraction
    bits and smallest normal exponent ``emin`` (subnormals below it keep the
    quantum 2^(emin - frac_bits)); ties go to the even neighbour.  No range
    limit: the callers saturate or overflow as their format says.

    With x = f * 2^e, 1 <= |f| < 2 (e from frexp, exact), the representable
    neighbours of x are the multiples of 2^(max(e, emin) - frac_bits), so the
    rounding is one scaled round-half-even on an exact quotient.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    _, e2 = np.frexp(x[fin])                    # x = m * 2^e2, 0.5 <= |m| < 1
    e = np.maximum(e2.astype(np.int64) - 1, emin)
    quantum = np.ldexp(1.0, (e - frac_bits).astype(np.int64))
    out[fin] = np.round(x[fin] / quantum) * quantum   # np.round: half to even; x / quantum exact
    return out


def f64_to_bf16_codes(x: np.ndarray) -> np.ndarray:
    """bfloat16 (8 fraction bits incl. none hidden: 7 stored, exponent range of
    binary32) nearest-even codes; overflow gives infinity, NaN stays NaN."""
    r = round_to_grid(x, 7, -126)
    r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, r), r)  # (2 - 2^-7) * 2^127
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _fp8_table():
    codes = np.arange(256, dtype=np.uint8)
    vals = fp8_e4m3fn_to_f64(codes)
    return {float(v): int(c) for v, c in zip(vals, codes) if np.isfinite(v) and not (v == 0 and c == 0x80)}


_FP8_CODE_OF = None


def f64_to_fp8_e4m3fn_codes(x: np.ndarray) -> np.ndarray:
    """OCP fp8 E4M3 nearest-even codes with saturation: magnitudes that round
    above 448 (the largest finite value) become +-448; NaN gives the NaN
    code 0x7F.  Zero keeps its sign (0x80 for -0.0)."""
    global _FP8_CODE_OF
    if _FP8_CODE_OF is None:
        _FP8_CODE_OF = _fp8_table()
    x = np.asarray(x, dtype=np.float64)
    r = np.clip(round_to_grid(x, 3, -6), -448.0, 448.0)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_r, flat_x, flat_o = r.reshape(-1), x.reshape(-1), out.reshape(-1)
    for i in range(flat_r.size):
        v = flat_r[i]
        if np.isnan(v):
            flat_o[i] = 0x7F
        elif v == 0:
            flat_o[i] = 0x80 if np.signbit(flat_x[i]) else 0x00
        else:
            flat_o[i] = _FP8_CODE_OF[float(v)]
    return out


def f64_to_int4_codes(x: np.ndarray) -> np.ndarray:
    """Packed signed 4-bit codes of x [..., 2n] (values already divided by
    their scale): each element becomes the nearest integer, ties to the even
    one, saturated to [-8, 7] (NaN gives 0); element 2i goes to the low
    nibble of byte i, element 2i + 1 to the high one, as two's complement.
    Returns [..., n] uint8."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-1] % 2:
        raise ValueError("INT4 rows hold an even number of elements")
    k = np.clip(np.rint(np.nan_to_num(x, nan=0.0)), -8, 7).astype(np.int64)  # np.rint: half to even
    nib = k & 0xF
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def encode_codes(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 to storage codes ('f32', 'bf16', 'fp8', 'int4'), nearest-even
    (int4: the last axis halves)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return f64_to_bf16_codes(x)
    if dtype == "fp8":
        return f64_to_fp8_e4m3fn_codes(x)
    if dtype == "int4":
        return f64_to_int4_codes(x)
    raise ValueError(f"unknown storage type {dtype!r}")
