"""GPU parity of the per-page fp8 indexer-K cache append ("Inference Optimization for Kimi K3.1 Pro",
§3: the indexer prolog writes each step's new keys into the cache; the fp8 indexer keys carry one
fp32 scale per page) through the C ABI, against the CPU oracle.  Codes and scales are byte
outputs: bit-exact after every call.

Call sequences mix prefill-sized appends over fresh pages, appends that start mid-page and cross
page boundaries, single-key decode appends, keys whose growing magnitude raises a page's scale
(the held codes are re-encoded), pages of zeros (scale 1), signed zeros, and a stale scale left
in a page that holds no key yet.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_15_amd as dsa
import workloads as W
from oracle.quant import indexer_cache_append_fp8_ref
from tests._gpu import DEV, check_indices_band, to_np, up

pytestmark = pytest.mark.gpu
PAGE = 64


def _bf16_bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, np.float32))


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


class Cache:
    """One paged fp8 cache on the device and its oracle copy, checked after every append."""

    def __init__(self, B, D, max_len, seed, spare=5):
        rng = np.random.default_rng(seed)
        self.mp = (max_len + PAGE - 1) // PAGE
        self.P = B * self.mp + spare
        perm = rng.permutation(self.P).astype(np.int32)
        self.bt = perm[:B * self.mp].reshape(B, self.mp)
        self.max_len = max_len
        # contents before the first append: NaN codes and a stale scale everywhere
        self.kc = np.full((self.P, PAGE, D), 0x7F, np.uint8)
        self.ks = np.full(self.P, np.float32(3.0), np.float32)
        self.kc_d, self.ks_d, self.bt_d = up(self.kc), up(self.ks), up(self.bt)

    def append(self, bits, lens, rows=None):
        """bits [b, T, D] bf16 keys for the sequences `rows` (default all) at lengths `lens`."""
        rows = list(range(self.bt.shape[0])) if rows is None else rows
        T = bits.shape[1]
        lens = np.asarray(lens, np.int32)
        bt = self.bt[rows]
        dsa.dsa_indexer_cache_append_fp8(up(bits), self.kc_d, self.ks_d, up(bt), up(lens),
                                         max_seq_len=self.max_len, num_pages=self.P)
        self.kc, self.ks = indexer_cache_append_fp8_ref(_f32(bits), self.kc, self.ks, bt, lens, T)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(self.ks_d).view(np.uint32), self.ks.view(np.uint32))
        np.testing.assert_array_equal(to_np(self.kc_d), self.kc)


def _keys(rng, B, L, D):
    """bf16 keys whose magnitude drifts upwards along the sequence, so page scales keep growing."""
    x = rng.standard_normal((B, L, D)) * np.exp(np.linspace(-2, 2, L))[None, :, None]
    x *= np.exp(rng.standard_normal((B, L, 1)) * 0.5)
    x[:, ::97] = 0.0                                   # zero keys
    x[:, 5::41, 3] = -0.0
    return _bf16_bits(x)


@pytest.mark.parametrize("D", [128, 64])
def test_append_sequence_bit_exact(D):
    B = 5
    rng = np.random.default_rng(D)
    start = np.array([1, 63, 64, 130, 700])
    plan = [1, 3, 64, 130, 1, 700, 1, 17]               # T of each batched call after the prefixes
    max_len = int(start.max() + sum(plan))
    keys = _keys(rng, B, max_len, D)
    keys[2, :start[2]] = 0                              # a sequence whose first page holds only zeros
    c = Cache(B, D, max_len, seed=D + 1)
    for b in range(B):                                  # prefixes: one sequence per call
        print(f"[case] fp8 page append D={D} prefix b={b} T={start[b]}", flush=True)
        c.append(keys[b:b + 1, :start[b]], [start[b]], rows=[b])
    lens = start.copy()
    for T in plan:
        lens = lens + T
        print(f"[case] fp8 page append D={D} T={T} lens={lens.tolist()}", flush=True)
        c.append(np.stack([keys[b, lens[b] - T:lens[b]] for b in range(B)]), lens)


def test_worked_example_on_the_device():
    """The hand-derived example (tests/golden/fp8_page_append_worked_example.json, 4-dim keys) in
    the first 4 of 64 columns, the rest zero: every call matches the oracle, and the 4 columns the
    example's expected codes and scales."""
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp8_page_append_worked_example.json")))
    D = 64
    bt = np.array([g["block_table"]], np.int32)
    kc = np.full((g["num_pages"], PAGE, D), g["initial_code"], np.uint8)
    ks = np.full(g["num_pages"], g["initial_scale"], np.float32)
    kc_d, ks_d = up(kc), up(ks)
    for call in g["calls"]:
        L, T = call["seq_len"], call["T"]
        print(f"[case] fp8 page worked example len={L} T={T}", flush=True)
        new = np.zeros((1, T, D), np.float32)
        for pos, v in call["keys"].items():
            new[0, int(pos) - (L - T), :4] = v
        bits = _bf16_bits(new)
        dsa.dsa_indexer_cache_append_fp8(up(bits), kc_d, ks_d, up(bt), up(np.array([L], np.int32)),
                                         max_seq_len=128, num_pages=g["num_pages"])
        kc, ks = indexer_cache_append_fp8_ref(_f32(bits), kc, ks, bt, np.array([L]), T)
        torch.cuda.synchronize()
        got_c, got_s = to_np(kc_d), to_np(ks_d)
        np.testing.assert_array_equal(got_c, kc)
        np.testing.assert_array_equal(got_s.view(np.uint32), ks.view(np.uint32))
        for page, bits_hex in call["expect_scale_bits"].items():
            assert got_s[int(page)].view(np.uint32) == int(bits_hex, 16)
        for page, rows in call["expect_codes"].items():
            for slot, hexrow in enumerate(rows):
                assert bytes(got_c[int(page), slot, :4]).hex().upper() == hexrow


def test_append_then_fp8_indexer_end_to_end():
    """Keys written through the library (a prefill-sized append, then decode appends) and queries
    quantised by the library are scored by the fp8 indexer: its indices equal the oracle's on the
    library-written cache (which the tests above show equal the oracle's own append)."""
    rng = np.random.default_rng(21)
    B, D, HI, K = 2, 128, 64, 2048
    lens0 = np.array([3000, 4500])
    steps = 6
    max_len = int(lens0.max()) + steps
    keys = _bf16_bits(rng.standard_normal((B, max_len, D)) / np.sqrt(D))
    c = Cache(B, D, max_len, seed=22)
    for b in range(B):
        c.append(keys[b:b + 1, :lens0[b]], [lens0[b]], rows=[b])
    lens = lens0.copy()
    for _ in range(steps):
        lens = lens + 1
        c.append(np.stack([keys[b, lens[b] - 1:lens[b]] for b in range(B)]), lens)
    q_bits = _bf16_bits(rng.standard_normal((B, 1, HI, D)) / np.sqrt(D))
    q_codes, q_sc = dsa.dsa_fp8_quantize_heads(up(q_bits))
    w = (rng.standard_normal((B, 1, HI)) / 8).astype(np.float32)
    idx = dsa.dsa_indexer_topk(q_codes, q_sc, up(w), c.kc_d, c.ks_d, c.bt_d, up(lens.astype(np.int32)),
                               T=1, top_k=K, max_seq_len=max_len, fp8=True, num_pages=c.P)
    torch.cuda.synchronize()
    ref, extra = oracle.indexer_topk_ref(q_idx=to_np(q_codes), q_scale=to_np(q_sc), w=w, k_cache=c.kc,
                                         k_scale=c.ks, block_table=c.bt, seq_lens=lens, T=1, K=K,
                                         dtype="fp8", return_scores=True)
    check_indices_band(to_np(idx), ref, extra, K, lens, 1)
    dsa.dsa_debug_status()


def test_length_below_T_writes_nothing_and_is_reported():
    """A sequence whose length is below T has no certain positions: its pages stay as they were,
    the other sequences are appended, and the length check is reported."""
    rng = np.random.default_rng(23)
    B, D, T = 3, 128, 20
    c = Cache(B, D, 256, seed=24)
    keys = _keys(rng, B, 256, D)
    for b in range(B):
        c.append(keys[b:b + 1, :50], [50], rows=[b])
    try:
        dsa.dsa_debug_status()
    except dsa.DsaError:
        pass
    before = to_np(c.kc_d).copy(), to_np(c.ks_d).copy()
    lens = np.array([70, 10, 70], np.int32)               # sequence 1: 10 < T
    new = np.stack([keys[b, 50:70] for b in range(B)])
    dsa.dsa_indexer_cache_append_fp8(up(new), c.kc_d, c.ks_d, c.bt_d, up(lens), max_seq_len=256,
                                     num_pages=c.P)
    with pytest.raises(dsa.DsaError, match="seq_lens"):
        dsa.dsa_debug_status()
    got_c, got_s = to_np(c.kc_d), to_np(c.ks_d)
    for j in range(c.mp):                               # sequence 1's pages unchanged
        p = c.bt[1, j]
        np.testing.assert_array_equal(got_c[p], before[0][p])
        assert got_s[p].view(np.uint32) == before[1][p].view(np.uint32)
    ok = [0, 2]
    ref_c, ref_s = indexer_cache_append_fp8_ref(_f32(new[ok]), before[0], before[1], c.bt[ok], lens[ok], T)
    for b in ok:
        for j in range(2):
            p = c.bt[b, j]
            np.testing.assert_array_equal(got_c[p], ref_c[p])
            assert got_s[p].view(np.uint32) == ref_s[p].view(np.uint32)


def test_append_at_bench_size_every_page():
    """The append at the benchmark's size (8 sequences x 65536 new keys x 128 dims into 8193
    permuted pages, the launch bench.py times), then a decode step of 32 sequences appending one
    key each to pages that hold keys: every page's codes and scale bit-exact against the oracle."""
    B, T, D = 8, 65536, 128
    P = B * T // 64 + 1
    gen = torch.Generator(device=DEV).manual_seed(17)
    perm = torch.randperm(P, device=DEV, generator=gen).to(torch.int32)
    bt = perm[:B * T // 64].view(B, T // 64).contiguous()
    sl = torch.full((B,), T, dtype=torch.int32, device=DEV)
    src = (torch.randn(B, T, D, device=DEV, generator=gen) / np.sqrt(D)).to(torch.bfloat16)
    kc = torch.full((P, 64, D), 0x7F, dtype=torch.uint8, device=DEV)
    ks = torch.full((P,), 3.0, dtype=torch.float32, device=DEV)
    kc0, ks0 = to_np(kc).copy(), to_np(ks).copy()
    print("[case] fp8 page append bench size", flush=True)
    dsa.dsa_indexer_cache_append_fp8(src, kc, ks, bt, sl, max_seq_len=T, num_pages=P)
    torch.cuda.synchronize()
    btn = bt.cpu().numpy()
    ref_c, ref_s = indexer_cache_append_fp8_ref(src.float().cpu().numpy(), kc0, ks0, btn, np.full(B, T), T)
    np.testing.assert_array_equal(to_np(ks).view(np.uint32), ref_s.view(np.uint32))
    np.testing.assert_array_equal(to_np(kc), ref_c)
    # decode step: sequence b holds lens[b] - 1 keys and appends one (the bench's decode leg)
    Bd = 32
    lens = np.array([1000 + 197 * b for b in range(Bd)], np.int32)
    bt_d = perm[:Bd * 112].view(Bd, 112).contiguous()
    new = (torch.randn(Bd, 1, D, device=DEV, generator=gen) / np.sqrt(D) * 3).to(torch.bfloat16)
    print("[case] fp8 page append bench decode step", flush=True)
    dsa.dsa_indexer_cache_append_fp8(new, kc, ks, bt_d, up(lens), max_seq_len=112 * 64, num_pages=P)
    torch.cuda.synchronize()
    ref_c, ref_s = indexer_cache_append_fp8_ref(new.float().cpu().numpy(), ref_c, ref_s, bt_d.cpu().numpy(), lens, 1)
    np.testing.assert_array_equal(to_np(ks).view(np.uint32), ref_s.view(np.uint32))
    np.testing.assert_array_equal(to_np(kc), ref_c)
