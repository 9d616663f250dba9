"""Mutation checks for the pins of the FP8 latent cache and the fp8 quantisers ("Inference
Optimization for Kimi K3.1 Pro", §3-§4).

Each pin is written once as a check that takes an implementation.  The oracle passes every pin;
each planted mistake (a copy of the oracle's function with one plausible error, built here on the
CPU) must fail at least one of them, so the pins would catch that mistake in the oracle itself.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import dequant_kv_fp8
from oracle.codecs import bf16_bits_to_f64, e4m3_codes_to_f64
from oracle.quant import _e4m3_rne, fp8_quantize_heads, latent_fp8_quantize_rows
from oracle.sfa import f32_to_bf16_rne

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


# ---------------------------------------------------------------- dequantisation of the FP8 cache
def _torch_dequant(codes, scales):
    c = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float32)
    tile = torch.clamp(torch.arange(codes.shape[-1]) // 128, max=4)
    s = torch.from_numpy(np.ascontiguousarray(scales, np.float32))[..., tile]
    return (c * s).to(torch.bfloat16).view(torch.uint16).numpy()


def dequant_pins(fn):
    rng = np.random.default_rng(51)
    codes = rng.choice(FINITE, size=(24, 576)).astype(np.uint8)
    scales = np.abs(rng.standard_normal((24, 8)) * 10.0 ** rng.integers(-4, 3, (24, 8))).astype(np.float32) + 1e-20
    ok_torch = np.array_equal(fn(codes, scales), _torch_dequant(codes, scales))
    ones = np.full((1, 576), 0x38, np.uint8)
    sc = np.array([[2.0 ** -3, 2.0, 2.0 ** 5, 2.0 ** -7, 2.0 ** 9, 7, 7, 7]], np.float32)
    expect = np.concatenate([np.full(128, 2.0 ** -3), np.full(128, 2.0), np.full(128, 2.0 ** 5),
                             np.full(128, 2.0 ** -7), np.full(64, 2.0 ** 9)])
    ok_tiles = np.array_equal(bf16_bits_to_f64(fn(ones, sc))[0], expect)
    unit = np.resize(FINITE, (2, 576)).astype(np.uint8)
    ok_unit = np.array_equal(bf16_bits_to_f64(fn(unit, np.ones((2, 8), np.float32))), e4m3_codes_to_f64(unit))
    return ok_torch and ok_tiles and ok_unit


def _dequant_with(tile_of, to_bf16=f32_to_bf16_rne):
    def fn(codes, scales):
        vals = e4m3_codes_to_f64(codes).astype(np.float32)
        return to_bf16(vals * np.asarray(scales, np.float32)[..., tile_of(codes.shape[-1])])
    return fn


def _truncate_bf16(x):
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


DEQUANT_MUTANTS = {
    "five equal tiles": _dequant_with(lambda d: np.minimum(np.arange(d) // 116, 4)),
    "tile index off by one": _dequant_with(lambda d: np.minimum(np.arange(d) // 128 + 1, 5)),
    "rope under the last value tile": _dequant_with(lambda d: np.minimum(np.arange(d) // 128, 3)),
    "bf16 by truncation": _dequant_with(lambda d: np.minimum(np.arange(d) // 128, 4), _truncate_bf16),
}


def test_dequant_pins_pass_on_the_oracle():
    assert dequant_pins(dequant_kv_fp8)


@pytest.mark.parametrize("name", list(DEQUANT_MUTANTS))
def test_dequant_pins_catch(name):
    assert not dequant_pins(DEQUANT_MUTANTS[name]), name


# ---------------------------------------------------------------- latent-row quantiser
def _bits_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def latent_pins(fn):
    rng = np.random.default_rng(52)
    bits = W.f32_to_bf16_bits((rng.standard_normal((60, 576)) * 10.0 ** rng.integers(-4, 3, (60, 1))).astype(np.float32))
    c1, s1 = fn(_bits_to_f32(bits))
    c2, s2 = W.bf16_rows_to_fp8_tiles(bits)
    ok_gen = np.array_equal(c1, c2) and np.array_equal(s1, s2)
    x = np.zeros((2, 576), np.float32)
    x[0, :128] = np.linspace(-448, 448, 128, dtype=np.float32).round()
    x[1, 512] = 3.0
    codes, sc = fn(x)
    ok_closed = (sc[0].tolist() == [1.0] * 8 and sc[1, 4] == np.float32(3.0) / np.float32(448.0)
                 and e4m3_codes_to_f64(codes[1, 512:513])[0] == 448.0)
    return ok_gen and ok_closed


def _latent_with(bounds, amax_div=448.0, rne=_e4m3_rne):
    def fn(x):
        x = np.asarray(x, np.float32)
        codes = np.empty(x.shape, np.uint8)
        scales = np.ones(x.shape[:-1] + (8,), np.float32)
        for i, (a, b) in enumerate(bounds):
            t = x[..., a:b]
            amax = np.abs(t).max(axis=-1)
            s = np.where(amax > 0, amax / np.float32(amax_div), np.float32(1.0)).astype(np.float32)
            scales[..., i] = s
            codes[..., a:b] = rne((t / s[..., None]).astype(np.float32).astype(np.float64))
        return codes, scales
    return fn


def _truncating_e4m3(y):
    a = np.abs(y)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.ldexp(1.0, (np.maximum(e, -6) - 3).astype(np.int64))
    return _e4m3_rne(np.sign(y) * np.floor(a / step) * step)


TILES = [(0, 128), (128, 256), (256, 384), (384, 512), (512, 576)]
LATENT_MUTANTS = {
    "448 off by one": _latent_with(TILES, amax_div=447.0),
    "tiles of 64": _latent_with([(64 * i, 64 * i + 64) for i in range(8)][:8] + [(512, 576)]),
    "rope merged into the last value tile": _latent_with(TILES[:3] + [(384, 576)]),
    "codes truncated": _latent_with(TILES, rne=_truncating_e4m3),
}


def test_latent_pins_pass_on_the_oracle():
    assert latent_pins(latent_fp8_quantize_rows)


@pytest.mark.parametrize("name", list(LATENT_MUTANTS))
def test_latent_pins_catch(name):
    try:
        caught = not latent_pins(LATENT_MUTANTS[name])
    except (IndexError, ValueError):
        caught = True                  # a shape error is caught as well
    assert caught, name


# ---------------------------------------------------------------- per-head query quantiser
def heads_pins(fn):
    rng = np.random.default_rng(53)
    x = _bits_to_f32(W.f32_to_bf16_bits((rng.standard_normal((80, 128)) * 10.0 ** rng.integers(-3, 3, (80, 1))).astype(np.float32)))
    codes, sq = fn(x)
    t = torch.from_numpy(x)
    amax = t.abs().amax(-1)
    s_t = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    c_t = (t / s_t[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.array_equal(sq, s_t.numpy()) and np.array_equal(codes, c_t)


HEADS_MUTANTS = {
    "one scale for the whole tensor": lambda x: (lambda s: (_e4m3_rne((x / s).astype(np.float64)), np.full(x.shape[:-1], s, np.float32)))(
        np.float32(np.abs(x).max() / np.float32(448.0))),
    "scale amax / 240": lambda x: (lambda sq: (_e4m3_rne((x / sq[:, None]).astype(np.float32).astype(np.float64)), sq))(
        (np.abs(x).max(-1) / np.float32(240.0)).astype(np.float32)),
}


def test_heads_pins_pass_on_the_oracle():
    assert heads_pins(fp8_quantize_heads)


@pytest.mark.parametrize("name", list(HEADS_MUTANTS))
def test_heads_pins_catch(name):
    assert not heads_pins(HEADS_MUTANTS[name]), name
