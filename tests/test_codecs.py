"""Exhaustive checks of the oracle's storage codecs and of the input quantiser.

The codecs are written from the format definitions; here they are compared
code by code with torch's own conversions (a library routine) and with
properties fixed by the definitions (largest finite e4m3 value 448, smallest
subnormal 2^-9, NaN only at S.1111.111, monotone magnitudes).
"""
import numpy as np
import torch

from oracle import bf16_to_f64, decode_codes, fp8_e4m3fn_to_f64
from workloads import _to_bf16_codes, _to_fp8_codes


def test_bf16_all_codes_match_torch():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = bf16_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_fp8_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8_e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_fp8_definition_properties():
    v = fp8_e4m3fn_to_f64(np.arange(256, dtype=np.uint8))
    assert np.flatnonzero(np.isnan(v)).tolist() == [0x7F, 0xFF]
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.nanmax(np.abs(v)) == 448.0
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x38] == 1.0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)
    np.testing.assert_array_equal(v[0x80:0xFF], -pos)


def test_f32_passthrough():
    x = np.array([0.0, -1.5, 3.25e-30, np.float32(1e38)], np.float32)
    np.testing.assert_array_equal(decode_codes(x, "f32"), x.astype(np.float64))


def test_bf16_quantiser_is_round_to_nearest_even():
    # exact halfway cases between two bf16 neighbours: ties go to the even code
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)
    x = np.array([one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4, one + 3 * ulp / 4], np.float32)
    got = bf16_to_f64(_to_bf16_codes(x))
    np.testing.assert_array_equal(got, [1.0, 1.0 + 2 * 2.0 ** -7, 1.0, 1.0 + 2.0 ** -7])


def test_fp8_quantiser_saturates_and_rounds():
    x = np.array([500.0, -1e6, 448.0, 1.0 + 1 / 16, 1.0 + 3 / 16, 2.0 ** -10, 3 * 2.0 ** -11], np.float32)
    got = fp8_e4m3fn_to_f64(_to_fp8_codes(x))
    np.testing.assert_array_equal(got, [448.0, -448.0, 448.0, 1.0, 1.25, 0.0, 2.0 ** -9])
