"""Pins for the oracle's sparse attention ("Inference Optimization for Kimi K3.1 Pro", §1 step 3;
"Optimizing Kimi K3.1 Pro Sparse Attention Inference", "Inheritance and Extension of Core
Operators").

  * closed forms: one selected row returns that V row exactly; two rows give the logistic mix;
    equal logits give the mean of V and lse = ln K';
  * selecting every visible position equals dense causal attention computed by
    torch.nn.functional.scaled_dot_product_attention in float64 (an independent library routine);
  * invariance to the order of the index list, to -1 padding and to physical page placement.
"""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import sparse_attn_ref
from oracle.codecs import bf16_bits_to_f64


def _case(T=1, lens=(300,), H=16, values="gauss", variant=0):
    spec = W.custom("sfa_pin", len(lens), T, lens, 4, 16, 64, H, values=values, variant=variant,
                    cfg_id=91)
    return W.make_case(spec)


def _rows(c, b, sel):
    sel = np.asarray(sel)
    return bf16_bits_to_f64(c.kv_cache[c.block_table[b, sel // 64], sel % 64])


def _run(c, idx, scale=1.0 / 24):
    return sparse_attn_ref(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx, scale)


def test_single_row_returns_v_row():
    c = _case()
    idx = np.full((1, 1, 8), -1, np.int32)
    idx[0, 0, 0] = 137
    out, lse = _run(c, idx)
    X = _rows(c, 0, [137])[0]
    assert np.array_equal(out[0, 0], np.broadcast_to(X[:512], out[0, 0].shape))
    z = (bf16_bits_to_f64(c.q_attn[0, 0]) @ X) / 24
    np.testing.assert_allclose(lse[0, 0], z, rtol=1e-14, atol=1e-14)


def test_two_rows_logistic_mix():
    c = _case(values="sharp")
    idx = np.array([[[5, 250, -1, -1]]], np.int32)
    out, lse = _run(c, idx, scale=0.3)
    X = _rows(c, 0, [5, 250])
    q = bf16_bits_to_f64(c.q_attn[0, 0])
    z1, z2 = 0.3 * (q @ X[0]), 0.3 * (q @ X[1])
    a = 1.0 / (1.0 + np.exp(z2 - z1))
    ref = a[:, None] * X[0, :512] + (1 - a)[:, None] * X[1, :512]
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.logaddexp(z1, z2), rtol=1e-13)


def test_equal_logits_mean_of_v():
    c = _case()
    q0 = np.zeros_like(c.q_attn)                 # all logits 0
    sel = np.array([3, 64, 65, 199, 299])
    idx = np.full((1, 1, 9), -1, np.int32)
    idx[0, 0, :5] = sel
    out, lse = sparse_attn_ref(q0, c.kv_cache, c.block_table, c.seq_lens, idx, 1 / 24)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(_rows(c, 0, sel)[:, :512].mean(0), (16, 512)),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], np.log(5.0), rtol=1e-14)


def test_empty_selection():
    c = _case()
    out, lse = _run(c, np.full((1, 1, 4), -1, np.int32))
    assert np.all(out == 0) and np.all(lse == -np.inf)


@pytest.mark.parametrize("T", [1, 5])
def test_full_selection_equals_dense_causal_sdpa(T):
    """With every visible position selected, sparse attention is dense causal attention with
    K = the 576-wide latent rows and V = their first 512 columns."""
    L = 150
    c = _case(T=T, lens=(L,), values="sharp")
    idx = np.full((1, T, L), -1, np.int32)
    for t in range(T):
        n = L - T + t + 1
        idx[0, t, :n] = np.arange(n)
    out, lse = _run(c, idx, scale=0.05)
    X = torch.from_numpy(_rows(c, 0, np.arange(L)))                       # [L, 576]
    q = torch.from_numpy(bf16_bits_to_f64(c.q_attn[0]))                   # [T, H, 576]
    qh = q.permute(1, 0, 2)                                               # [H, T, 576]
    kh = X[None].expand(16, L, 576)
    vh = X[None, :, :512].expand(16, L, 512).contiguous()
    mask = torch.zeros(T, L, dtype=torch.bool)
    for t in range(T):
        mask[t, :L - T + t + 1] = True
    ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=0.05)
    np.testing.assert_allclose(out[0], ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-13)
    # lse against torch.logsumexp of the masked logits
    z = (qh @ kh.transpose(1, 2)) * 0.05
    z = z.masked_fill(~mask[None], float("-inf"))
    np.testing.assert_allclose(lse[0], torch.logsumexp(z, -1).permute(1, 0).numpy(), rtol=1e-12)


def test_order_padding_and_page_invariance():
    c = _case(T=2, lens=(260, 190), H=32)
    rng = np.random.default_rng(0)
    idx = np.full((2, 2, 64), -1, np.int32)
    for b in range(2):
        for t in range(2):
            pos = c.seq_lens[b] - 2 + t
            idx[b, t, :40] = np.sort(rng.choice(pos + 1, 40, replace=False))
    o1, l1 = _run(c, idx)
    shuffled = idx.copy()
    for b in range(2):
        for t in range(2):
            shuffled[b, t, :40] = rng.permutation(idx[b, t, :40])
    o2, l2 = _run(c, shuffled)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-15)
    c2 = W.permute_pages(c)
    o3, l3 = sparse_attn_ref(c2.q_attn, c2.kv_cache, c2.block_table, c2.seq_lens, idx, 1 / 24)
    np.testing.assert_array_equal(o1, o3)
    np.testing.assert_array_equal(l1, l3)


def test_rejects_future_or_duplicate_indices():
    c = _case(lens=(100,))
    with pytest.raises(ValueError):
        _run(c, np.array([[[5, 5, -1]]], np.int32))
    with pytest.raises(ValueError):
        _run(c, np.array([[[5, 100, -1]]], np.int32))
