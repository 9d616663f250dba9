"""Mutation checks for the pins of the indexer and sparse-attention oracle ("Inference
Optimization for Kimi K3.1 Pro", §1-§2; "Optimizing Kimi K3.1 Pro Sparse Attention Inference",
"Inheritance and Extension of Core Operators"; "Day0 Inference Adaptation for Next-Gen LLMs",
§3.1).

Each pin is written once as a check that takes an implementation.  The oracle passes every pin;
each planted mistake (a small re-implementation of the definition with one plausible error, built
here on the CPU) must fail at least one pin, so the pins would catch that mistake in the oracle.

Indexer pins: the hand-derived worked example (tests/golden/indexer_worked_example.json), a
pure-Python brute force on tiny inputs (loops for the dots, sorted() for the selection), the
doubling of one physical page's fp8 scale (doubles exactly the scores of the keys on that page),
page-permutation invariance and the causal visible counts.
Attention pins: one selected row returns its V row exactly, the two-row logistic closed form,
dense causal attention from torch's scaled_dot_product_attention in float64, -1 padding and page
placement invariance.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import indexer_topk_ref, sparse_attn_ref
from oracle.codecs import bf16_bits_to_f64, e4m3_codes_to_f64

GOLD = os.path.join(os.path.dirname(__file__), "golden", "indexer_worked_example.json")
PAGE = 64


# ================================================================ indexer
def _dec(x, dtype):
    return bf16_bits_to_f64(x) if dtype == "bf16" else e4m3_codes_to_f64(x)


def make_indexer(relu="head", page="table", ties="low", vis=1, order="asc", kscale="phys", wrow="own"):
    """The definition with switchable mistakes; the defaults are the definition itself."""
    def fn(q_idx, q_scale, w, k_cache, k_scale, block_table, seq_lens, T, K, dtype):
        B = seq_lens.shape[0]
        idx = np.full((B, T, K), -1, np.int32)
        scores = {}
        for b in range(B):
            for t in range(T):
                n = int(seq_lens[b]) - T + t + vis
                s = np.arange(n)
                lp = s // PAGE if page != "shift" else np.minimum((s + 1) // PAGE, block_table.shape[1] - 1)
                pg = block_table[b, lp] if page != "identity" else lp
                k = _dec(k_cache[pg, s % PAGE], dtype)
                q = _dec(q_idx[b, t], dtype)
                if dtype == "fp8":
                    ks = k_scale[pg] if kscale == "phys" else k_scale[s // PAGE]
                    k = k * ks.astype(np.float64)[:, None]
                    q = q * q_scale[b, t].astype(np.float64)[:, None]
                wt = w[b, t if wrow == "own" else 0].astype(np.float64)
                dots = q @ k.T
                if relu == "head":
                    sc = wt @ np.maximum(dots, 0.0)
                elif relu == "none":
                    sc = wt @ dots
                else:                                    # gate after the head sum
                    sc = np.maximum(wt @ dots, 0.0)
                kp = min(K, n)
                pos_key = np.arange(n) if ties == "low" else -np.arange(n)
                sel = np.sort(np.lexsort((pos_key, -sc))[:kp])
                if order == "desc":
                    sel = sel[::-1]
                idx[b, t, :kp] = sel
                scores[(b, t)] = sc
        return idx, scores
    return fn


def oracle_indexer(q_idx, q_scale, w, k_cache, k_scale, block_table, seq_lens, T, K, dtype):
    idx, ex = indexer_topk_ref(q_idx, q_scale, w, k_cache, k_scale, block_table, seq_lens, T, K, dtype,
                               return_scores=True)
    return idx, {key: v[0] for key, v in ex.items()}


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


def pin_golden(fn):
    g = json.load(open(GOLD))
    _, sc = fn(**_golden_arrays(g, 1), T=1, K=4, dtype="bf16")
    for s, v in g["expected_scores_pos69"].items():
        if sc[(0, 0)].shape[0] != 70 or sc[(0, 0)][int(s)] != v:
            return False
    for case in g["cases"]:
        a = _golden_arrays(g, case["T"])
        if "w_per_query" in case:
            a["w"] = np.array([case["w_per_query"]], np.float32)
        idx, _ = fn(**a, T=case["T"], K=case["K"], dtype="bf16")
        if idx[0, case["t"]].tolist() != case["idx"]:
            return False
    return True


def _tiny(dtype="bf16", T=2, lens=(150, 97), K=12, values="gauss", HI=3, DI=8, variant=0):
    spec = W.custom("mut", len(lens), T, lens, HI, DI, K, 16, idx_dtype=dtype, values=values,
                    variant=variant, cfg_id=92)
    return W.make_case(spec)


def _args(c):
    return dict(q_idx=c.q_idx, q_scale=c.q_scale, w=c.w, k_cache=c.k_cache, k_scale=c.k_scale,
                block_table=c.block_table, seq_lens=c.seq_lens)


def _brute(c, dtype):
    """Plain Python: dot products by loops, page lookups one key at a time, sorted() selection."""
    spec = c.spec
    out = np.full((spec.B, spec.T, spec.K), -1, np.int32)
    for b in range(spec.B):
        for t in range(spec.T):
            n = int(c.seq_lens[b]) - spec.T + t + 1
            q = _dec(c.q_idx[b, t], dtype)
            if dtype == "fp8":
                q = q * c.q_scale[b, t].astype(np.float64)[:, None]
            score = []
            for s in range(n):
                p = int(c.block_table[b, s // PAGE])
                k = _dec(c.k_cache[p, s % PAGE], dtype)
                if dtype == "fp8":
                    k = k * float(c.k_scale[p])
                tot = 0.0
                for h in range(spec.HI):
                    d = 0.0
                    for j in range(spec.DI):
                        d += float(q[h, j]) * float(k[j])
                    tot += float(c.w[b, t, h]) * max(d, 0.0)
                score.append(tot)
            best = sorted(range(n), key=lambda s: (-score[s], s))[:min(spec.K, n)]
            out[b, t, :len(best)] = sorted(best)
    return out


def pin_brute_force(fn):
    for dtype, values in (("bf16", "gauss"), ("bf16", "ties"), ("fp8", "gauss")):
        c = _tiny(dtype=dtype, values=values)
        idx, _ = fn(**_args(c), T=c.spec.T, K=c.spec.K, dtype=dtype)
        if not np.array_equal(idx, _brute(c, dtype)):
            return False
    return True


def pin_page_scale_doubling(fn):
    """fp8 keys: doubling the scale of one physical page doubles exactly the scores of the keys
    stored on it (ReLU is positively homogeneous) and leaves every other score unchanged."""
    c = _tiny(dtype="fp8", T=1, lens=(200,))
    _, s1 = fn(**_args(c), T=1, K=8, dtype="fp8")
    page = int(c.block_table[0, 1])                  # the page that holds positions 64..127
    a = _args(c)
    a["k_scale"] = c.k_scale.copy()
    a["k_scale"][page] *= 2
    _, s2 = fn(**a, T=1, K=8, dtype="fp8")
    on = (np.arange(200) // PAGE) == 1
    if s1[(0, 0)].shape != (200,) or s2[(0, 0)].shape != (200,):
        return False
    return (np.array_equal(s2[(0, 0)][on], 2 * s1[(0, 0)][on]) and
            np.array_equal(s2[(0, 0)][~on], s1[(0, 0)][~on]))


def pin_page_permutation(fn):
    c = _tiny(T=2, lens=(130, 200))
    c2 = W.permute_pages(c)
    i1, _ = fn(**_args(c), T=2, K=12, dtype="bf16")
    i2, _ = fn(**_args(c2), T=2, K=12, dtype="bf16")
    return np.array_equal(i1, i2)


def pin_visible_counts(fn):
    """Query t of a sequence of length L with T queries keeps min(K, L - T + t + 1) positions, all
    at or below its own position, ascending, then -1."""
    c = _tiny(T=4, lens=(9, 40), K=12)
    idx, _ = fn(**_args(c), T=4, K=12, dtype="bf16")
    for b in range(2):
        for t in range(4):
            pos = int(c.seq_lens[b]) - 4 + t
            row = idx[b, t]
            kp = min(12, pos + 1)
            sel = row[:kp]
            if not (np.all(row[kp:] == -1) and np.all(sel >= 0) and np.all(sel <= pos)
                    and np.all(np.diff(sel) > 0)):
                return False
    return True


INDEXER_PINS = [pin_golden, pin_brute_force, pin_page_scale_doubling, pin_page_permutation, pin_visible_counts]

INDEXER_MUTANTS = {
    "ReLU dropped": make_indexer(relu="none"),
    "ReLU after the head sum": make_indexer(relu="sum"),
    "logical page used as physical": make_indexer(page="identity"),
    "page of the next position": make_indexer(page="shift"),
    "ties to the higher position": make_indexer(ties="high"),
    "visibility one short": make_indexer(vis=0),
    "descending output": make_indexer(order="desc"),
    "fp8 scale of the logical page": make_indexer(kscale="logical"),
    "head weights of the first query": make_indexer(wrow="first"),
}


def test_indexer_definition_matches_oracle():
    for dtype in ("bf16", "fp8"):
        c = _tiny(dtype=dtype)
        a, _ = make_indexer()(**_args(c), T=2, K=12, dtype=dtype)
        b, _ = oracle_indexer(**_args(c), T=2, K=12, dtype=dtype)
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("pin", INDEXER_PINS, ids=lambda p: p.__name__)
def test_indexer_pins_pass_on_the_oracle(pin):
    assert pin(oracle_indexer)


@pytest.mark.parametrize("name", list(INDEXER_MUTANTS))
def test_indexer_pins_catch(name):
    fn = INDEXER_MUTANTS[name]
    assert not all(pin(fn) for pin in INDEXER_PINS), name


# ================================================================ sparse attention
def make_attn(vcols=(0, 512), scale_mul=1.0, lse_base="e", skip_pad=True, page="table", norm=True,
              axis="keys", qrow="own"):
    """The definition with switchable mistakes; the defaults are the definition itself."""
    def fn(q_attn, kv_cache, block_table, seq_lens, idx, sm_scale):
        B, T, H, _ = q_attn.shape
        out = np.zeros((B, T, H, 512))
        lse = np.full((B, T, H), -np.inf)
        for b in range(B):
            for t in range(T):
                sel = idx[b, t]
                if skip_pad:
                    sel = sel[sel >= 0]
                sel = sel.astype(np.int64)
                if sel.size == 0:
                    continue
                pg = block_table[b, sel // PAGE] if page == "table" else sel // PAGE
                X = bf16_bits_to_f64(kv_cache[pg, sel % PAGE])
                q = bf16_bits_to_f64(q_attn[b, t if qrow == "own" else 0])
                z = sm_scale * scale_mul * (q @ X.T)
                ax = 1 if axis == "keys" else 0
                m = z.max(axis=ax, keepdims=True)
                e = np.exp(z - m)
                l = e.sum(axis=ax, keepdims=True)
                o = e @ X[:, vcols[0]:vcols[1]]
                out[b, t] = o / (l if axis == "keys" else 1.0) if norm else o
                ls = (m + np.log(l)).reshape(-1)[:H] if axis == "keys" else np.log(l.sum()) * np.ones(H)
                lse[b, t] = ls / math.log(2) if lse_base == "2" else ls
        return out, lse
    return fn


def oracle_attn(q_attn, kv_cache, block_table, seq_lens, idx, sm_scale):
    return sparse_attn_ref(q_attn, kv_cache, block_table, seq_lens, idx, sm_scale)


def _acase(T=1, lens=(300,), H=16, values="gauss"):
    spec = W.custom("mut_attn", len(lens), T, lens, 4, 16, 64, H, values=values, cfg_id=93)
    return W.make_case(spec)


def _kv_rows(c, b, sel):
    sel = np.asarray(sel)
    return bf16_bits_to_f64(c.kv_cache[c.block_table[b, sel // 64], sel % 64])


def pin_single_row(fn):
    c = _acase(T=2, lens=(300,))
    idx = np.full((1, 2, 8), -1, np.int32)
    idx[0, 0, 0] = 137
    idx[0, 1, 0] = 70
    out, lse = fn(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx, 1 / 24)
    for t, s in ((0, 137), (1, 70)):
        X = _kv_rows(c, 0, [s])[0]
        if not np.array_equal(out[0, t], np.broadcast_to(X[:512], out[0, t].shape)):
            return False
        z = (bf16_bits_to_f64(c.q_attn[0, t]) @ X) / 24
        if not np.allclose(lse[0, t], z, rtol=1e-13, atol=1e-13):
            return False
    return True


def pin_two_rows(fn):
    c = _acase(values="sharp")
    idx = np.array([[[5, 250, -1, -1]]], np.int32)
    out, lse = fn(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx, 0.3)
    X = _kv_rows(c, 0, [5, 250])
    q = bf16_bits_to_f64(c.q_attn[0, 0])
    z1, z2 = 0.3 * (q @ X[0]), 0.3 * (q @ X[1])
    a = 1.0 / (1.0 + np.exp(z2 - z1))
    ref = a[:, None] * X[0, :512] + (1 - a)[:, None] * X[1, :512]
    return (np.allclose(out[0, 0], ref, rtol=1e-11, atol=1e-12) and
            np.allclose(lse[0, 0], np.logaddexp(z1, z2), rtol=1e-12))


def pin_dense_sdpa(fn):
    L, T = 120, 3
    c = _acase(T=T, lens=(L,), values="sharp")
    idx = np.full((1, T, L + 4), -1, np.int32)
    for t in range(T):
        n = L - T + t + 1
        idx[0, t, :n] = np.arange(n)
    out, lse = fn(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx, 0.05)
    X = torch.from_numpy(_kv_rows(c, 0, np.arange(L)))
    qh = torch.from_numpy(bf16_bits_to_f64(c.q_attn[0])).permute(1, 0, 2)
    kh = X[None].expand(16, L, 576)
    vh = X[None, :, :512].expand(16, L, 512).contiguous()
    mask = torch.zeros(T, L, dtype=torch.bool)
    for t in range(T):
        mask[t, :L - T + t + 1] = True
    ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=0.05)
    z = ((qh @ kh.transpose(1, 2)) * 0.05).masked_fill(~mask[None], float("-inf"))
    return (np.allclose(out[0], ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12) and
            np.allclose(lse[0], torch.logsumexp(z, -1).permute(1, 0).numpy(), rtol=1e-11))


def pin_padding_and_pages(fn):
    c = _acase(T=2, lens=(260, 190), H=16)
    rng = np.random.default_rng(3)
    idx = np.full((2, 2, 48), -1, np.int32)
    for b in range(2):
        for t in range(2):
            pos = int(c.seq_lens[b]) - 2 + t
            idx[b, t, :40] = np.sort(rng.choice(pos + 1, 40, replace=False))
    o1, l1 = fn(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx, 1 / 24)
    o2, l2 = fn(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, np.ascontiguousarray(idx[:, :, :40]), 1 / 24)
    c2 = W.permute_pages(c)
    o3, l3 = fn(c2.q_attn, c2.kv_cache, c2.block_table, c2.seq_lens, idx, 1 / 24)
    return (np.allclose(o1, o2, rtol=1e-12, atol=1e-15) and np.allclose(l1, l2, rtol=1e-12) and
            np.array_equal(o1, o3) and np.array_equal(l1, l3))


ATTN_PINS = [pin_single_row, pin_two_rows, pin_dense_sdpa, pin_padding_and_pages]

ATTN_MUTANTS = {
    "V from the last 512 columns": make_attn(vcols=(64, 576)),
    "softmax scale dropped": make_attn(scale_mul=24.0),
    "lse in base 2": make_attn(lse_base="2"),
    "-1 entries taken as positions": make_attn(skip_pad=False),
    "logical page used as physical": make_attn(page="identity"),
    "output not normalised": make_attn(norm=False),
    "softmax over heads": make_attn(axis="heads"),
    "query of the first token": make_attn(qrow="first"),
}


def test_attn_definition_matches_oracle():
    c = _acase(T=2, lens=(260, 190))
    rng = np.random.default_rng(4)
    idx = np.full((2, 2, 32), -1, np.int32)
    for b in range(2):
        for t in range(2):
            pos = int(c.seq_lens[b]) - 2 + t
            idx[b, t, :30] = np.sort(rng.choice(pos + 1, 30, replace=False))
    a = make_attn()(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx, 1 / 24)
    b = oracle_attn(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx, 1 / 24)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12)


@pytest.mark.parametrize("pin", ATTN_PINS, ids=lambda p: p.__name__)
def test_attn_pins_pass_on_the_oracle(pin):
    assert pin(oracle_attn)


@pytest.mark.parametrize("name", list(ATTN_MUTANTS))
def test_attn_pins_catch(name):
    fn = ATTN_MUTANTS[name]
    assert not all(pin(fn) for pin in ATTN_PINS), name
