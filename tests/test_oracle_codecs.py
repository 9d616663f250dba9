"""Pins for the oracle's format decoders and the generator's storage rounding.

The decoders are written from the format definitions; here they are checked against torch's own
float8_e4m3fn / bfloat16 casts (independent library routines) and against closed-form values of
the E4M3FN definition.
"""
import numpy as np
import pytest
import torch

from oracle.codecs import bf16_bits_to_f64, e4m3_codes_to_f64, e4m3_table
from workloads import f32_to_bf16_bits, f32_to_e4m3_codes


def test_e4m3_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    tab = e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(tab))
    assert nan.sum() == 2                      # 0x7F and 0xFF only
    assert np.array_equal(ref[~nan], tab[~nan])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x38, 1.0),
    (0x3C, 1.5), (0x7E, 448.0), (0xFE, -448.0), (0xB8, -1.0), (0x40, 2.0), (0x48, 4.0),
    (0x50, 8.0), (0x58, 16.0)])
def test_e4m3_closed_form_values(code, value):
    assert e4m3_codes_to_f64(np.array([code], np.uint8))[0] == value


def test_e4m3_small_integers_exact():
    # every integer in [-16, 16] has an exact code (3 mantissa bits): used by the exact fp8 variant
    ints = np.arange(-16, 17, dtype=np.float32)
    assert np.array_equal(e4m3_codes_to_f64(f32_to_e4m3_codes(ints)), ints.astype(np.float64))


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=200000).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).double().numpy()
    got = bf16_bits_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_generator_bf16_rounding_is_rne():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(1_000_000) * 10.0 ** rng.integers(-8, 8, 1_000_000)).astype(np.float32)
    # exact halfway cases (low 16 bits == 0x8000), finite: exponent field kept below 0xFF
    hi = rng.integers(0, 1 << 13, 4096).astype(np.uint32) << np.uint32(17)
    half = (hi | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, half, -half])
    assert np.isfinite(x).all()
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_generator_e4m3_rounding_is_rne():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * 100).astype(np.float32)
    codes = f32_to_e4m3_codes(x)
    dec = e4m3_codes_to_f64(codes)
    # nearest: no other finite code is strictly closer
    tab = e4m3_table()
    fin = tab[np.isfinite(tab)]
    xc = np.clip(x.astype(np.float64), -448, 448)
    best = np.abs(fin[None, :] - xc[:2000, None]).min(axis=1)
    assert np.allclose(np.abs(dec[:2000] - xc[:2000]), best, rtol=0, atol=0)
