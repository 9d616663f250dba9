"""Pins for the oracle's MXFP8 quantisation and paged cache append ("Inference Optimization for Kimi
K3.1 Pro", §3-§4: the indexer prolog writes the new keys into the cache, the indexer's Q and K are
MXFP8; "Day0 Inference Adaptation for Next-Gen LLMs", §3.3).

Each pin checks the oracle against something other than itself:
  * element rounding against torch's float8_e4m3fn cast (an independent library routine), on
    random values, on every exact halfway point between neighbouring E4M3 values and on signed
    zeros;
  * shared exponents against closed forms of the OCP definition (floor(log2 amax) - 8);
  * quantise-then-decode error within half an E4M3 step, clamping at 448;
  * agreement with the workload generator's quantiser, which goes through torch's cast;
  * the cache append against a direct reading of the paged layout (token t of sequence b lands at
    logical position seq_len - T + t; nothing else changes).
"""
import numpy as np
import torch

import workloads as W
from oracle import e4m3_codes_to_f64, e8m0_to_f64
from oracle.quant import _e4m3_rne, cache_append_ref, mxfp8_quantize_rows


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_rounding_matches_torch_random():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(300000) * 10.0 ** rng.integers(-5, 3, 300000)).astype(np.float32)
    x = np.clip(x, -448, 448)
    np.testing.assert_array_equal(_e4m3_rne(x.astype(np.float64)), _torch_e4m3(x))


def test_rounding_halfway_points_and_zero_signs():
    vals = np.unique(np.abs(e4m3_codes_to_f64(np.arange(0x7F, dtype=np.uint8))))
    mids = (vals[:-1] + vals[1:]) / 2                       # exact ties: must go to the even code
    x = np.concatenate([mids, -mids, [0.0, -0.0, 2.0 ** -11, -(2.0 ** -11)]])
    np.testing.assert_array_equal(_e4m3_rne(x), _torch_e4m3(x))
    assert _e4m3_rne(np.array([-0.0]))[0] == 0x80 and _e4m3_rne(np.array([-(2.0 ** -11)]))[0] == 0x80


def test_clamp_at_448():
    assert e4m3_codes_to_f64(_e4m3_rne(np.array([449.0, 470.0, 511.9, -500.0]))).tolist() == [448, 448, 448, -448]


def test_shared_exponent_closed_forms():
    rows = np.zeros((4, 64))
    rows[0, :32] = 1.0                  # amax 1 -> s = -8
    rows[1, 5] = 448.0                  # amax 448 -> floor(log2) = 8 -> s = 0
    rows[2, 40] = 2.0 ** -20            # second group amax 2^-20 -> s = -28
    rows[3, :] = 0.0                    # zeros -> s = -127, codes 0
    codes, sc = mxfp8_quantize_rows(rows)
    assert sc.tolist() == [[119, 0], [127, 0], [0, 99], [0, 0]]
    assert (codes[3] == 0).all()
    assert e4m3_codes_to_f64(codes[0, :32]).tolist() == [256.0] * 32


def test_round_trip_error_bound():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((50, 128)) * 10.0 ** rng.integers(-6, 4, (50, 1))).astype(np.float32)
    codes, sc = mxfp8_quantize_rows(v)
    scale = np.repeat(e8m0_to_f64(sc), 32, -1)
    back = e4m3_codes_to_f64(codes) * scale
    el = np.abs(v / scale)
    step = np.where(el >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(el, 1e-300))) - 3), 2.0 ** -9) * scale
    assert (np.abs(back - v) <= step / 2 + (el > 448) * np.abs(v)).all()
    # the largest element of every group lands in [256, 448]
    gmax = np.abs(e4m3_codes_to_f64(codes)).reshape(50, 4, 32).max(-1)
    assert ((gmax >= 256) & (gmax <= 448)).all()


def test_agrees_with_generator_quantiser():
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((64, 128)) * 10.0 ** rng.integers(-3, 3, (64, 1))).astype(np.float32)
    c1, s1 = mxfp8_quantize_rows(v)
    c2, s2 = W.f32_to_mxfp8(v)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)


def test_cache_append_positions():
    P, D, T = 9, 64, 3
    rng = np.random.default_rng(6)
    kc = rng.integers(0, 256, (P, 64, D)).astype(np.uint8)
    ks = rng.integers(0, 256, (P, 64, D // 32)).astype(np.uint8)
    bt = np.array([[4, 7, 1], [2, 0, 8]], np.int32)
    sl = np.array([130, 64], np.int32)          # sequence 0 ends in its third page, 1 fills its first
    new = rng.standard_normal((2, T, D))
    kc2, ks2 = cache_append_ref(new, kc, ks, bt, sl, T)
    codes, sc = mxfp8_quantize_rows(new)
    touched = np.zeros((P, 64), bool)
    for b, positions in ((0, (127, 128, 129)), (1, (61, 62, 63))):
        for t, pos in enumerate(positions):
            p, s = bt[b, pos // 64], pos % 64
            np.testing.assert_array_equal(kc2[p, s], codes[b, t])
            np.testing.assert_array_equal(ks2[p, s], sc[b, t])
            touched[p, s] = True
    np.testing.assert_array_equal(kc2[~touched], kc[~touched])
    np.testing.assert_array_equal(ks2[~touched], ks[~touched])


# ---------------------------------------------------------------- FP8 latent rows ([P1] §4)
from oracle.quant import latent_cache_append_fp8_ref, latent_fp8_quantize_rows  # noqa: E402


def _bf16_rows(rng, shape, scale):
    return W.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _bits_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def test_latent_fp8_agrees_with_generator():
    rng = np.random.default_rng(21)
    bits = _bf16_rows(rng, (300, 576), 10.0 ** rng.integers(-4, 3, (300, 1)))
    c1, s1 = latent_fp8_quantize_rows(_bits_to_f32(bits))
    c2, s2 = W.bf16_rows_to_fp8_tiles(bits)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)


def test_latent_fp8_closed_forms():
    x = np.zeros((3, 576), np.float32)
    x[0, :128] = np.linspace(-448, 448, 128, dtype=np.float32).round()   # amax 448: scale 1
    x[1, 512] = 3.0                                                       # rope tile only
    codes, sc = latent_fp8_quantize_rows(x)
    assert sc[0].tolist() == [1.0] * 8
    np.testing.assert_array_equal(codes[0, :128], _e4m3_rne(x[0, :128].astype(np.float64)))
    assert sc[1, 4] == np.float32(3.0) / np.float32(448.0) and sc[1, :4].tolist() == [1.0] * 4
    assert e4m3_codes_to_f64(codes[1, 512:513])[0] == 448.0 and (codes[2] == 0).all()


def test_latent_fp8_tile_max_is_448_and_error_bound():
    rng = np.random.default_rng(22)
    x = _bits_to_f32(_bf16_rows(rng, (80, 576), 10.0 ** rng.integers(-5, 2, (80, 1))))
    codes, sc = latent_fp8_quantize_rows(x)
    v = e4m3_codes_to_f64(codes)
    tile = np.minimum(np.arange(576) // 128, 4)
    for i in range(5):
        assert (np.abs(v[:, tile == i]).max(axis=1) == 448.0).all()
    s = sc[:, tile].astype(np.float64)
    el = np.abs(x / s)
    step = np.where(el >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(el, 1e-300))) - 3), 2.0 ** -9)
    assert (np.abs(v * s - x) <= (step / 2) * s * (1 + 1e-6) + 1e-30).all()


def test_latent_fp8_append_positions():
    P = 7
    rng = np.random.default_rng(23)
    kc = rng.integers(0, 256, (P, 64, 576)).astype(np.uint8)
    ks = rng.standard_normal((P, 64, 8)).astype(np.float32)
    bt = np.array([[3, 5], [6, 0]], np.int32)
    sl = np.array([66, 2], np.int32)
    new = _bits_to_f32(_bf16_rows(rng, (2, 2, 576), 0.1))
    kc2, ks2 = latent_cache_append_fp8_ref(new, kc, ks, bt, sl, 2)
    codes, sc = latent_fp8_quantize_rows(new)
    touched = np.zeros((P, 64), bool)
    for b, positions in ((0, (64, 65)), (1, (0, 1))):
        for t, pos in enumerate(positions):
            p, s = bt[b, pos // 64], pos % 64
            np.testing.assert_array_equal(kc2[p, s], codes[b, t])
            np.testing.assert_array_equal(ks2[p, s], sc[b, t])
            touched[p, s] = True
    np.testing.assert_array_equal(kc2[~touched], kc[~touched])
    np.testing.assert_array_equal(ks2[~touched], ks[~touched])


# ---------------------------------------------------------------- per-head fp8 queries ([P1] §3)
from oracle.quant import fp8_quantize_heads  # noqa: E402


def test_fp8_heads_match_torch_cast():
    rng = np.random.default_rng(31)
    x = _bits_to_f32(_bf16_rows(rng, (500, 128), 10.0 ** rng.integers(-4, 3, (500, 1))))
    x[0] = 0.0
    codes, sq = fp8_quantize_heads(x)
    t = torch.from_numpy(x)
    amax = t.abs().amax(-1)
    s_t = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    c_t = (t / s_t[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(sq, s_t.numpy())
    np.testing.assert_array_equal(codes, c_t)


def test_fp8_heads_closed_forms():
    x = np.zeros((3, 64), np.float32)
    x[0, 7] = -448.0                               # scale 1, code of -448
    x[1, :] = 2.0 ** -10                           # uniform row: every code is 448
    codes, sq = fp8_quantize_heads(x)
    assert sq.tolist() == [1.0, np.float32(2.0 ** -10) / np.float32(448.0), 1.0]
    assert e4m3_codes_to_f64(codes[0, 7:8])[0] == -448.0 and (codes[0, :7] == 0).all()
    assert (e4m3_codes_to_f64(codes[1]) == 448.0).all() and (codes[2] == 0).all()
