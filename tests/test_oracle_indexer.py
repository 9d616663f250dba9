"""Pins for the oracle's Lightning-Indexer scores and Top-K ("Inference Optimization for Kimi
K3.1 Pro", §1-§2; "Day0 Inference Adaptation for Next-Gen LLMs", §3.1).

Each pin checks the oracle against something other than itself:
  * a hand-derived worked example (tests/golden/indexer_worked_example.json): scores, the ReLU gate,
    the sign of the head weight, page resolution through a permuted block table with decoy pages,
    tie-breaking, -1 padding and causal visibility;
  * identities of the score that fail if a term is dropped or mis-indexed (ReLU split identity,
    head-permutation invariance, positive homogeneity, additivity over heads);
  * page-permutation invariance of indices and scores;
  * Top-K against brute force (Python sorted / heapq with the (score desc, position asc) key);
  * the exactness certificate of the integer-grid workload (fp32 scores exact in any order).
"""
import heapq
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import indexer_scores_ref, indexer_topk_ref
from oracle.indexer import select_topk

GOLD = os.path.join(os.path.dirname(__file__), "golden", "indexer_worked_example.json")


def _golden_arrays(g, T):
    P, DI, HI = g["num_pages"], g["DI"], g["HI"]
    k = np.full((P, 64, DI), g["decoy_value"], dtype=np.float32)
    bt = np.array([g["block_table"]], dtype=np.int32)
    for p in g["block_table"]:
        k[p] = 0.0
    for s, vec in g["keys"].items():
        s = int(s)
        k[bt[0, s // 64], s % 64] = vec
    q = np.broadcast_to(np.array(g["q"], np.float32), (1, T, HI, DI)).copy()
    w = np.broadcast_to(np.array(g["w"], np.float32), (1, T, HI)).copy()
    return dict(q_idx=W.f32_to_bf16_bits(q), q_scale=None, w=w, k_cache=W.f32_to_bf16_bits(k),
                k_scale=None, block_table=bt, seq_lens=np.array([g["seq_len"]], np.int32))


def test_worked_example_scores():
    g = json.load(open(GOLD))
    a = _golden_arrays(g, 1)
    (sc,) = indexer_scores_ref(**a, T=1, dtype="bf16", b=0, ts=[0])
    assert sc.shape == (70,)
    for s, v in g["expected_scores_pos69"].items():
        assert sc[int(s)] == v, (s, sc[int(s)], v)
    zero = [s for s in range(70) if str(s) not in g["keys"]]
    assert np.all(sc[zero] == 0.0)


@pytest.mark.parametrize("case", json.load(open(GOLD))["cases"], ids=lambda c: f"T{c['T']}t{c['t']}K{c['K']}")
def test_worked_example_topk(case):
    g = json.load(open(GOLD))
    a = _golden_arrays(g, case["T"])
    if "w_per_query" in case:
        a["w"] = np.array([case["w_per_query"]], np.float32)
    idx = indexer_topk_ref(**a, T=case["T"], K=case["K"], dtype="bf16")
    assert idx[0, case["t"]].tolist() == case["idx"]


def test_worked_example_padding():
    g = json.load(open(GOLD))
    a = _golden_arrays(g, 1)
    a["seq_lens"] = np.array([5], np.int32)       # only positions 0..4 visible
    idx = indexer_topk_ref(**a, T=1, K=8, dtype="bf16")
    assert idx[0, 0].tolist() == [0, 1, 2, 3, 4, -1, -1, -1]


def _small_case(values="gauss", dtype="bf16", T=1, lens=(150, 200), HI=4, DI=16, K=32, variant=0):
    spec = W.custom("pin", len(lens), T, lens, HI, DI, K, 16, idx_dtype=dtype, values=values,
                    variant=variant, cfg_id=90)
    return W.make_case(spec)


def _args(c):
    return dict(q_idx=c.q_idx, q_scale=c.q_scale, w=c.w, k_cache=c.k_cache, k_scale=c.k_scale,
                block_table=c.block_table, seq_lens=c.seq_lens)


def _scores(c, b=0, t=0, **over):
    a = _args(c)
    a.update(over)
    dt = "bf16" if c.spec.idx_dtype == "bf16" else "fp8"
    return indexer_scores_ref(**a, T=c.spec.T, dtype=dt, b=b, ts=[t])[0]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_relu_split_identity(dtype):
    """relu(x) - relu(-x) = x, so I(q) - I(-q) = sum_h w_h (q_h . k): fails if the gate is dropped
    (difference doubles) or applied to the weighted sum instead of each head."""
    c = _small_case(dtype=dtype)
    neg = c.q_idx ^ (np.uint16(0x8000) if dtype == "bf16" else np.uint8(0x80))
    d = _scores(c) - _scores(c, q_idx=neg)
    from oracle.codecs import bf16_bits_to_f64, e4m3_codes_to_f64
    dec = bf16_bits_to_f64 if dtype == "bf16" else e4m3_codes_to_f64
    n = c.seq_lens[0]
    s = np.arange(n)
    pages = c.block_table[0, s // 64]
    k = dec(c.k_cache[pages, s % 64])
    q = dec(c.q_idx[0, 0])
    if dtype == "fp8":
        k = k * c.k_scale[pages][:, None]
        q = q * c.q_scale[0, 0][:, None]
    lin = np.einsum("h,hd,sd->s", c.w[0, 0].astype(np.float64), q, k)
    np.testing.assert_allclose(d, lin, rtol=1e-12, atol=1e-12)


def test_head_permutation_invariance():
    c = _small_case()
    perm = np.random.default_rng(5).permutation(c.spec.HI)
    s1 = _scores(c)
    s2 = _scores(c, q_idx=c.q_idx[:, :, perm], w=c.w[:, :, perm])
    np.testing.assert_allclose(s1, s2, rtol=1e-13, atol=1e-15)


def test_head_additivity_and_homogeneity():
    c = _small_case()
    w1 = c.w.copy(); w1[..., 1:] = 0
    w2 = c.w.copy(); w2[..., :1] = 0
    np.testing.assert_allclose(_scores(c, w=w1) + _scores(c, w=w2), _scores(c), rtol=1e-12, atol=1e-15)
    # doubling every key (exact in bf16: exponent + 1) doubles every score (ReLU is homogeneous)
    k2 = W.f32_to_bf16_bits(
        (c.k_cache.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0))
    np.testing.assert_array_equal(_scores(c, k_cache=k2), 2.0 * _scores(c))
    # a head with zero weight is inert
    w0 = c.w.copy(); w0[..., 2] = 0
    q0 = c.q_idx.copy(); q0[:, :, 2] = W.f32_to_bf16_bits(np.full(c.spec.DI, 3.0, np.float32))
    np.testing.assert_array_equal(_scores(c, w=w0), _scores(c, w=w0, q_idx=q0))


@pytest.mark.parametrize("dtype,values", [("bf16", "gauss"), ("bf16", "grid"), ("fp8", "gauss")])
def test_page_permutation_invariance(dtype, values):
    c = _small_case(values=values, dtype=dtype, T=2, lens=(130, 257, 64))
    c2 = W.permute_pages(c)
    assert not np.array_equal(c.block_table, c2.block_table)
    dt = "bf16" if dtype == "bf16" else "fp8"
    i1, e1 = indexer_topk_ref(**_args(c), T=2, K=40, dtype=dt, return_scores=True)
    i2, e2 = indexer_topk_ref(**_args(c2), T=2, K=40, dtype=dt, return_scores=True)
    np.testing.assert_array_equal(i1, i2)
    for key in e1:
        np.testing.assert_array_equal(e1[key][0], e2[key][0])


def test_causal_visibility_and_poison():
    """Query t of a sequence sees exactly seq_len - T + t + 1 keys; poisoned (NaN) slots past the
    sequence end never reach a score."""
    c = _small_case(T=4, lens=(100, 131), K=200)
    idx, ex = indexer_topk_ref(**_args(c), T=4, K=200, dtype="bf16", return_scores=True)
    for b in range(2):
        for t in range(4):
            n = c.seq_lens[b] - 4 + t + 1
            assert ex[(b, t)][0].shape == (n,)
            assert np.isfinite(ex[(b, t)][0]).all()
            assert idx[b, t].tolist() == list(range(n)) + [-1] * (200 - n)


def _brute_topk(scores, K):
    n = len(scores)
    by_sort = sorted(range(n), key=lambda s: (-scores[s], s))[:min(K, n)]
    by_heap = heapq.nsmallest(min(K, n), range(n), key=lambda s: (-scores[s], s))
    assert by_sort == by_heap
    return sorted(by_sort) + [-1] * (K - min(K, n))


@pytest.mark.parametrize("seed", range(6))
def test_select_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 300))
    # few distinct values -> many exact ties; include -0.0 and +0.0 which must compare equal
    scores = rng.choice(np.array([-1.5, -0.0, 0.0, 0.25, 0.5, 3.0]), size=n)
    for K in (1, 2, 7, n // 2 + 1, n, n + 5):
        assert select_topk(scores, K).tolist() == _brute_topk(list(scores), K)


def test_select_topk_all_ties_and_zero_signs():
    assert select_topk(np.zeros(10), 4).tolist() == [0, 1, 2, 3]
    s = np.array([0.0, -0.0, 0.0, -0.0, 1.0])
    assert select_topk(s, 3).tolist() == [0, 1, 4]


def test_oracle_topk_matches_brute_force_on_case():
    c = _small_case(values="ties", lens=(300,), K=50)
    idx, ex = indexer_topk_ref(**_args(c), T=1, K=50, dtype="bf16", return_scores=True)
    sc = ex[(0, 0)][0]
    assert len(np.unique(sc)) < 100          # the tie-heavy variant really ties
    assert idx[0, 0].tolist() == _brute_topk(list(sc), 50)


def test_grid_exactness_certificate():
    """Integer-grid workload (multiples of 1/16): every score is a multiple of 2^-12 and every
    partial sum stays below 2^12 in magnitude, so an fp32 accumulation in any order is exact."""
    c = W.make_case(W.config(1))
    (sc,) = indexer_scores_ref(**_args(c), T=1, dtype="bf16", b=0, ts=[0])
    assert np.array_equal(sc * 4096, np.round(sc * 4096))
    from oracle.codecs import bf16_bits_to_f64
    q = bf16_bits_to_f64(c.q_idx[0, 0])
    kmax = np.abs(bf16_bits_to_f64(c.k_cache[np.isfinite(bf16_bits_to_f64(c.k_cache))])).max()
    bound_dot = np.abs(q).sum(axis=1).max() * kmax
    bound = np.abs(c.w[0, 0]).sum() * bound_dot
    assert bound < 4096 and bound_dot < 2 ** 16


def test_fp8_grid_exact_scores_are_dyadic():
    c = _small_case(values="fp8grid", dtype="fp8", lens=(200,))
    sc = _scores(c)
    # integer codes * power-of-two scales * 1/16 weights: multiples of 2^-16, bounded
    assert np.array_equal(sc * 2 ** 16, np.round(sc * 2 ** 16))
    assert np.abs(sc).max() < 2 ** 20
