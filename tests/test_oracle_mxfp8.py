"""Pins for the oracle's MXFP8 indexer path ("Inference Optimization for Kimi K3.1 Pro", §4: the
Lightning Indexer's Q and K in MXFP8; "Day0 Inference Adaptation for Next-Gen LLMs", §3.3).

MXFP8 as the OCP Microscaling format defines it: E4M3FN elements, each run of 32 consecutive
elements sharing one E8M0 scale 2^(e - 127).  Each pin checks the oracle against something other
than itself:
  * E8M0 decoding against torch's float8_e8m0fnu cast and closed-form values;
  * the generator's quantisation against the format's invariants (per-group scale exponent, codes
    within the E4M3 range, round-trip error within half an E4M3 step);
  * scores against a pure-Python brute force that decodes every code from its bit fields and
    applies the scale of the element's own 32-group (a wrong group index or a dropped scale fails);
  * reduction to the per-tensor fp8 path when every scale byte is 127 (scale 1);
  * the exactness certificate of the integer-grid variant (fp32 scores exact in any order);
  * page-permutation invariance.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import e8m0_to_f64, indexer_scores_ref, indexer_topk_ref


def _case(values="gauss", lens=(130, 257), T=1, HI=4, DI=64, K=40):
    spec = W.custom("mx_small", len(lens), T, lens, HI, DI, K, 16, idx_dtype="mxfp8", values=values)
    return W.make_case(spec)


def _args(c):
    return dict(q_idx=c.q_idx, q_scale=c.q_scale, w=c.w, k_cache=c.k_cache, k_scale=c.k_scale,
                block_table=c.block_table, seq_lens=c.seq_lens)


def test_e8m0_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float32).double().numpy()
    got = e8m0_to_f64(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 1     # only 0xFF
    # torch decodes through float32, which has no 2^-127 (code 0) as a normal number
    assert np.array_equal(ref[1:255], got[1:255])


@pytest.mark.parametrize("code,value", [(127, 1.0), (128, 2.0), (126, 0.5), (0, 2.0 ** -127),
                                        (254, 2.0 ** 127), (117, 2.0 ** -10)])
def test_e8m0_closed_forms(code, value):
    assert e8m0_to_f64(np.array([code], np.uint8))[0] == value


def test_generator_mx_quantisation_invariants():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 128)) * 10.0 ** rng.integers(-3, 3, (64, 1))).astype(np.float32)
    codes, sc = W.f32_to_mxfp8(x)
    assert codes.shape == x.shape and sc.shape == (64, 4)
    from oracle import e4m3_codes_to_f64
    el = e4m3_codes_to_f64(codes).reshape(64, 4, 32)
    scale = e8m0_to_f64(sc)
    g = x.reshape(64, 4, 32).astype(np.float64)
    amax = np.abs(g).max(-1)
    # shared exponent floor(log2(amax)) - 8, so the largest element lands in [256, 512) before
    # saturation to 448
    assert np.array_equal(np.log2(scale), np.floor(np.log2(amax)) - 8)
    assert np.abs(el).max() <= 448
    assert (np.abs(el).max(-1) >= 256).all()
    # round trip within half an E4M3 step (3 mantissa bits: 2^-4 relative) or the saturation
    back = el * scale[..., None]
    err = np.abs(back - g)
    step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(g), 1e-300))) - 3), scale[..., None] * 2.0 ** -9)
    sat = np.abs(g) > 448 * scale[..., None]
    assert (err[~sat] <= step[~sat] / 2 + 1e-300).all()


def _e4m3_from_bits(code):
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    return s * (m / 8.0) * 2.0 ** -6 if e == 0 else s * (1 + m / 8.0) * 2.0 ** (e - 7)


def test_scores_match_brute_force():
    c = _case(lens=(70,), HI=3, DI=64)
    (sc,) = indexer_scores_ref(**_args(c), T=1, dtype="mxfp8", b=0, ts=[0])
    n = 70
    q = [[_e4m3_from_bits(int(c.q_idx[0, 0, h, d])) * 2.0 ** (int(c.q_scale[0, 0, h, d // 32]) - 127)
          for d in range(64)] for h in range(3)]
    ref = []
    for s in range(n):
        p, slot = int(c.block_table[0, s // 64]), s % 64
        k = [_e4m3_from_bits(int(c.k_cache[p, slot, d])) * 2.0 ** (int(c.k_scale[p, slot, d // 32]) - 127)
             for d in range(64)]
        tot = 0.0
        for h in range(3):
            dot = sum(q[h][d] * k[d] for d in range(64))
            tot += float(c.w[0, 0, h]) * max(dot, 0.0)
        ref.append(tot)
    np.testing.assert_allclose(sc, np.array(ref), rtol=1e-12, atol=1e-15)


def test_unit_scales_reduce_to_fp8_path():
    c = _case(lens=(200,))
    ones_q = np.full(c.q_scale.shape, 127, np.uint8)
    ones_k = np.full(c.k_scale.shape, 127, np.uint8)
    a = _args(c)
    (mx,) = indexer_scores_ref(**{**a, "q_scale": ones_q, "k_scale": ones_k}, T=1, dtype="mxfp8",
                               b=0, ts=[0])
    (f8,) = indexer_scores_ref(**{**a, "q_scale": np.ones(c.w.shape, np.float32),
                                  "k_scale": np.ones(c.k_cache.shape[0], np.float32)},
                               T=1, dtype="fp8", b=0, ts=[0])
    np.testing.assert_array_equal(mx, f8)


def test_one_group_scale_changes_only_its_dims():
    """Doubling the scale of one 32-group of one key changes that key's dot products by exactly
    the group's partial dot product (so the scale sits on the right elements)."""
    c = _case(lens=(64,), HI=2, DI=64)
    a = _args(c)
    ks = c.k_scale.copy()
    p, slot = int(c.block_table[0, 0]), 5
    ks[p, slot, 1] += 1
    w1 = np.zeros_like(c.w); w1[0, 0, 0] = 1.0
    qp = c.q_idx.copy(); qm = c.q_idx.copy()
    # with q and -q the ReLU passes one of the two: their difference is the plain dot product
    qm[0, 0] ^= np.uint8(0x80)

    def dot(k_scale):
        (sp,) = indexer_scores_ref(**{**a, "w": w1, "q_idx": qp, "k_scale": k_scale}, T=1, dtype="mxfp8", b=0, ts=[0])
        (sm,) = indexer_scores_ref(**{**a, "w": w1, "q_idx": qm, "k_scale": k_scale}, T=1, dtype="mxfp8", b=0, ts=[0])
        return sp - sm
    d0, d1 = dot(c.k_scale), dot(ks)
    from oracle import e4m3_codes_to_f64
    q = e4m3_codes_to_f64(c.q_idx[0, 0, 0]) * np.repeat(e8m0_to_f64(c.q_scale[0, 0, 0]), 32)
    k = e4m3_codes_to_f64(c.k_cache[p, slot]) * np.repeat(e8m0_to_f64(c.k_scale[p, slot]), 32)
    part = (q[32:64] * k[32:64]).sum()
    assert np.delete(d1 - d0, 5).tolist() == [0.0] * 63
    assert d1[5] - d0[5] == pytest.approx(part, rel=1e-12, abs=1e-15)


def test_mxgrid_exactness_certificate():
    """Integer-grid MXFP8 variant: codes in [-2, 2], q scales 2^-2..2^0, k scales 2^-1..2^1, w in
    sixteenths.  Every product is a multiple of 2^-3 and every weighted term of 2^-7; the bound
    sum_h |w| * sum_d |q k| stays below 2^16, so fp32 partial sums (24 bits) are exact in any
    order."""
    c = _case(values="mxgrid", lens=(300,), HI=64, DI=128)
    (sc,) = indexer_scores_ref(**_args(c), T=1, dtype="mxfp8", b=0, ts=[0])
    assert np.array_equal(sc * 2 ** 7, np.round(sc * 2 ** 7))
    from oracle import e4m3_codes_to_f64
    q = np.abs(e4m3_codes_to_f64(c.q_idx[0, 0])) * np.repeat(e8m0_to_f64(c.q_scale[0, 0]), 32, -1)
    kmax = 2.0 * 2.0       # |code| <= 2, scale <= 2
    bound = (np.abs(c.w[0, 0]) * q.sum(-1) * kmax).sum()
    assert bound < 2 ** 16


def test_page_permutation_invariance_mx():
    c = _case(T=1, lens=(130, 257, 64))
    c2 = W.permute_pages(c)
    i1, e1 = indexer_topk_ref(**_args(c), T=1, K=40, dtype="mxfp8", return_scores=True)
    i2, e2 = indexer_topk_ref(**_args(c2), T=1, K=40, dtype="mxfp8", return_scores=True)
    np.testing.assert_array_equal(i1, i2)
    for key in e1:
        np.testing.assert_array_equal(e1[key][0], e2[key][0])
