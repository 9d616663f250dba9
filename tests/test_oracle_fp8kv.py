"""Pins for the oracle's FP8 latent cache ("Inference Optimization for Kimi K3.1 Pro", §4: the SFA
cache stored as FP8 with per-token scales over 128-wide tiles, the products kept in BF16).

Each pin checks the oracle against something other than itself:
  * dequantisation against torch's own casts (float8_e4m3fn -> float32, a float32 multiply, then
    float32 -> bfloat16), over every finite code and random scales;
  * the tile map (which scale serves which column) against a closed form: a row of ones with a
    distinct power-of-two scale per tile;
  * e4m3 values under a unit scale are bf16-exact, so dequantisation is the identity on them;
  * attention over identical selected rows returns that row's value part exactly (softmax of
    equal logits), with lse = z + ln n;
  * the fp8-cache attention equals the bf16 attention over the rows torch dequantises.
"""
import numpy as np
import torch

import workloads as W
from oracle import dequant_kv_fp8, sparse_attn_fp8kv_ref, sparse_attn_ref
from oracle.codecs import bf16_bits_to_f64, e4m3_codes_to_f64


def _torch_dequant(codes, scales):
    c = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float32)
    tile = torch.clamp(torch.arange(codes.shape[-1]) // 128, max=4)
    s = torch.from_numpy(np.ascontiguousarray(scales, np.float32))[..., tile]
    return (c * s).to(torch.bfloat16).view(torch.uint16).numpy()


def test_dequant_matches_torch_all_codes():
    rng = np.random.default_rng(11)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = rng.choice(finite, size=(40, 576)).astype(np.uint8)
    codes[0, :254] = finite
    scales = (rng.standard_normal((40, 8)) * 10.0 ** rng.integers(-6, 4, (40, 8))).astype(np.float32)
    scales = np.abs(scales) + np.float32(1e-30)
    np.testing.assert_array_equal(dequant_kv_fp8(codes, scales), _torch_dequant(codes, scales))


def test_tile_map_closed_form():
    codes = np.full((1, 576), 0x38, np.uint8)                # e4m3 1.0
    assert e4m3_codes_to_f64(codes[:, :1])[0, 0] == 1.0
    scales = np.array([[2.0 ** -3, 2.0 ** 1, 2.0 ** 5, 2.0 ** -7, 2.0 ** 9, 7.0, 7.0, 7.0]], np.float32)
    got = bf16_bits_to_f64(dequant_kv_fp8(codes, scales))[0]
    expect = np.concatenate([np.full(128, 2.0 ** -3), np.full(128, 2.0), np.full(128, 2.0 ** 5),
                             np.full(128, 2.0 ** -7), np.full(64, 2.0 ** 9)])
    np.testing.assert_array_equal(got, expect)


def test_unit_scale_is_identity_on_e4m3_values():
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = np.resize(finite, (3, 576)).astype(np.uint8)
    got = bf16_bits_to_f64(dequant_kv_fp8(codes, np.ones((3, 8), np.float32)))
    np.testing.assert_array_equal(got, e4m3_codes_to_f64(codes))


def test_identical_rows_give_that_row():
    rng = np.random.default_rng(12)
    P, H, n = 3, 4, 70
    row = rng.integers(0, 0x7E, 576).astype(np.uint8)
    codes = np.broadcast_to(row, (P, 64, 576)).copy()
    sc = np.broadcast_to(np.array([0.5, 0.25, 2.0, 1.0, 4.0, 1, 1, 1], np.float32), (P, 64, 8)).copy()
    q = W.f32_to_bf16_bits(rng.standard_normal((1, 1, H, 576)).astype(np.float32) * 0.05)
    bt = np.array([[2, 0]], np.int32)
    lens = np.array([n], np.int32)
    idx = np.full((1, 1, 80), -1, np.int32)
    idx[0, 0, :n] = np.arange(n)
    out, lse = sparse_attn_fp8kv_ref(q, codes, sc, bt, lens, idx, 1 / 24)
    x = bf16_bits_to_f64(dequant_kv_fp8(row[None], sc[0, :1]))[0]
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(x[:512], (H, 512)), rtol=1e-13, atol=1e-15)
    z = (bf16_bits_to_f64(q[0, 0]) @ x) / 24
    np.testing.assert_allclose(lse[0, 0], z + np.log(n), rtol=1e-12)


def test_fp8_attention_is_bf16_attention_on_torch_dequantised_rows():
    spec = W.custom("fp8kv_pin", 2, 2, (300, 190), 8, 64, 64, 16, kv_dtype="fp8")
    c = W.make_case(spec, poison=False)
    rng = np.random.default_rng(13)
    idx = np.full((2, 2, 64), -1, np.int32)
    for b in range(2):
        for t in range(2):
            n = int(c.seq_lens[b]) - 2 + t + 1
            k = min(64, n - 5)
            idx[b, t, :k] = np.sort(rng.choice(n, k, replace=False))
    o1, l1 = sparse_attn_fp8kv_ref(c.q_attn, c.kv_codes, c.kv_scale, c.block_table, c.seq_lens, idx, spec.sm_scale)
    deq = _torch_dequant(c.kv_codes, c.kv_scale)
    o2, l2 = sparse_attn_ref(c.q_attn, deq, c.block_table, c.seq_lens, idx, spec.sm_scale)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_generator_quantiser_round_trip():
    # the generated cache dequantises to within half an e4m3 step of the bf16 rows it came from
    spec = W.custom("fp8kv_rt", 1, 1, (200,), 8, 64, 64, 16, kv_dtype="fp8")
    c = W.make_case(spec, poison=False)
    x = bf16_bits_to_f64(c.kv_cache)
    back = bf16_bits_to_f64(dequant_kv_fp8(c.kv_codes, c.kv_scale))
    tile = np.minimum(np.arange(576) // 128, 4)
    s = c.kv_scale[..., tile].astype(np.float64)
    assert (np.abs(back - x) <= s * 448 * 2.0 ** -4 + np.abs(x) * 2.0 ** -8).all()
    assert np.all(c.kv_scale[..., 5:] == 1)
