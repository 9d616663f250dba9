"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

Sizes span several score chunks (1024 keys), select scan steps (16384 keys), attention tiles (32 rows)
and splits, with ragged tails (lengths not multiples of 64).  Exact-arithmetic cases (integer grids,
exact fp8 grid) must match the oracle's indices bit for bit; Gaussian cases use the near-tie band.
Attention is always compared on one shared index tensor (the GPU's own indices).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_15_amd as dsa
import workloads as W
from tests._gpu import Dev, check_attn, check_indices_band, oracle_args, to_np, up

pytestmark = pytest.mark.gpu


def _run(spec, exact, sfa_rows=None, check_sfa=True):
    print(f"[case] {spec.name} B={spec.B} T={spec.T} lens={spec.lens[:4]} K={spec.K} "
          f"{spec.idx_dtype}/{spec.values}", flush=True)
    c = W.make_case(spec)
    d = Dev(c)
    idx_t = d.indexer()
    torch.cuda.synchronize()
    idx = to_np(idx_t)
    ref, extra = oracle.indexer_topk_ref(**oracle_args(c), T=spec.T, K=spec.K, dtype=spec.idx_dtype,
                                         return_scores=True)
    if exact:
        bad = np.nonzero((idx != ref).any(axis=-1))
        assert np.array_equal(idx, ref), f"index mismatch in rows {list(zip(*bad))[:5]}"
    else:
        check_indices_band(idx, ref, extra, spec.K, c.seq_lens, spec.T)
    if check_sfa:
        out, lse = d.attn(idx_t)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.sparse_attn_ref(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx,
                                              spec.sm_scale, rows=sfa_rows)
        check_attn(to_np(out), to_np(lse), o_ref, l_ref, rows=sfa_rows)
    return c, d, idx


# ---------------------------------------------------------------- the five workloads (small size)
def test_cfg1_decode_grid_exact():
    _run(W.config(1), exact=True)


def test_cfg2_small_ragged_decode():
    _run(W.config(2, "small"), exact=False)


def test_cfg3_small_causal_prefill():
    spec = W.config(3, "small")
    rows = [(0, t) for t in (0, 1, 63, 64, 100, 1000, 2046, 2047, 2048, 2049, 2200, 2303)]
    _run(spec, exact=False, sfa_rows=rows)


def test_cfg4_small_fp8_decode():
    _run(W.config(4, "small"), exact=False)


def test_cfg5_small_verify():
    _run(W.config(5, "small"), exact=False)


def test_mx_small_verify():
    _run(W.config(8, "small"), exact=False)


# ---------------------------------------------------------------- exact-arithmetic variants
@pytest.mark.parametrize("T,lens", [(1, (3000, 5000)), (4, (2600, 4500)), (3, (2049, 2051, 3333)),
                                    (4, (2050, 2051, 9000))])
def test_wide_grid_exact(T, lens):
    spec = W.custom("grid8_wide", len(lens), T, lens, 64, 128, 2048, 128, values="grid8")
    _run(spec, exact=True)


@pytest.mark.parametrize("T", [1, 4])
def test_large_batch_grid_exact(T):
    """More than 512 sequences: decode and verify leave the persistent score kernels for the
    chunked one; the whole index tensor must still equal the oracle's."""
    lens = np.random.default_rng([15, 77, T]).integers(100, 1200, size=520)
    lens[:3] = (T, 257, 1199)
    spec = W.custom("grid8_b520", len(lens), T, lens, 64, 128, 256, 32, values="grid8")
    _run(spec, exact=True, sfa_rows=[(0, 0), (1, T - 1), (2, 0), (519, T - 1)])


def test_tie_heavy_exact():
    spec = W.custom("ties_wide", 2, 1, (3500, 6000), 64, 128, 2048, 128, values="ties")
    _run(spec, exact=True, check_sfa=False)


def _key_u32(x):
    """Order-preserving uint32 image of float32 values (-0 folded onto +0)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).copy()
    u[(u << 1) == 0] = 0
    return np.where((u & 0x80000000) != 0, ~u, u | 0x80000000).astype(np.uint32)


def _threshold_populations(extra, rows):
    """Per row: keys sharing the K'-th key's top 11 bits, top 22 bits, and all 32 bits."""
    out = []
    for r in rows:
        sc, th = extra[r]
        k, kt = _key_u32(sc), _key_u32([th])[0]
        out.append(tuple(int(np.sum((k >> s) == (kt >> s))) for s in (21, 10, 0)))
    return out


# Scores squeezed into one coarse bin (17 exact values, thousands of ties each) and a two-value
# tie flood: the threshold bin exceeds the 8192 candidates the select stages in LDS, so it takes
# the extra histogram passes (narrow at 70001 keys needs two); ties2 rows 0 and 70000 keep more
# than 8192 exact ties at the threshold, so the selection is emitted straight from the keys.
@pytest.mark.parametrize("values,lens,expect", [
    ("narrow", (60000, 30000), [lambda p: p[0] > 8192 and p[1] <= 8192] * 2),
    ("ties2", (20000, 12000), [lambda p: p[2] > 8192, lambda p: p[0] <= 8192]),
    ("ties2", (70000,), [lambda p: p[2] > 8192]),
    ("narrow", (70001,), [lambda p: p[1] > 8192 and p[2] <= 8192]),
])
def test_select_crowded_threshold_exact(values, lens, expect):
    spec = W.custom(values, len(lens), 1, lens, 64, 128, 2048, 16, values=values)
    print(f"[case] {spec.name} lens={lens}", flush=True)
    c = W.make_case(spec)
    d = Dev(c)
    idx = to_np(d.indexer())
    ref, extra = oracle.indexer_topk_ref(**oracle_args(c), T=1, K=2048, dtype="bf16",
                                         return_scores=True)
    pops = _threshold_populations(extra, [(b, 0) for b in range(len(lens))])
    assert all(f(p) for f, p in zip(expect, pops)), pops
    assert np.array_equal(idx, ref)


# The same floods in launches whose rows all have at most 8192 keys, which run the 256-thread
# select (2040 candidates staged in LDS): narrow and ties take one extra histogram pass, ties2
# keeps more than 2040 exact ties and is emitted straight from the keys.
@pytest.mark.parametrize("values,lens,expect", [
    ("narrow", (8192, 5000), [lambda p: p[0] > 2040 and p[1] <= 2040] * 2),
    ("ties", (8192, 7000), [lambda p: p[0] > 2040 and p[1] <= 2040] * 2),
    ("ties2", (8192, 6000), [lambda p: p[2] > 2040] * 2),
])
def test_select_crowded_threshold_short_rows_exact(values, lens, expect):
    test_select_crowded_threshold_exact(values, lens, expect)


def test_select_shapes_agree_at_the_boundary():
    """Rows of up to 8192 keys give the same indices whether the launch runs the 256-thread select
    (max_seq_len 8192) or the 1024-thread one (the same rows with a block table one page wider and
    max_seq_len 8256), and both equal the oracle's."""
    spec = W.custom("grid8_boundary", 3, 1, (8192, 5000, 8191), 64, 128, 2048, 16, values="grid8")
    print(f"[case] {spec.name}", flush=True)
    c = W.make_case(spec)
    d = Dev(c)
    short = to_np(d.indexer())
    wide = np.concatenate([c.block_table, c.block_table[:, :1]], axis=1)
    long_ = to_np(dsa.dsa_indexer_topk(d.q_idx, None, d.w, d.k, None, up(wide), d.sl, T=1, top_k=spec.K,
                                       max_seq_len=8256, num_pages=c.num_pages))
    ref = oracle.indexer_topk_ref(**oracle_args(c), T=1, K=spec.K, dtype="bf16")
    assert np.array_equal(short, ref)
    assert np.array_equal(long_, ref)


# Rows longer than one select segment (two scan steps of 16384 keys for rows up to 32768 keys, one
# step beyond) are split over several workgroups whose lists meet in global memory; rows longer
# than 65536 keys are emitted in several bitmap chunks.
@pytest.mark.parametrize("T,lens", [(1, (16385, 32768, 32769, 70000)), (4, (33000, 20000))])
def test_multi_segment_rows_exact(T, lens):
    spec = W.custom("grid8_long", len(lens), T, lens, 64, 128, 2048, 16, values="grid8")
    _run(spec, exact=True, check_sfa=False)


@pytest.mark.parametrize("T,fmt", [(1, "bf16"), (4, "bf16"), (1, "fp8"), (1, "mxfp8")])
def test_maximum_length_rows_exact(T, fmt):
    """A sequence at the library's maximum length (2^20 keys: the select's 32 segments of two scan
    steps each, 16 bitmap chunks) beside a 300001-key one, decode and verify, each indexer format
    on its exact grid: the indices equal the oracle's, and the attention over them matches."""
    values = {"bf16": "grid8", "fp8": "fp8grid", "mxfp8": "mxgrid"}[fmt]
    spec = W.custom("maxlen", 2, T, (1 << 20, 300001), 8, 64, 2048, 16, idx_dtype=fmt, values=values)
    _run(spec, exact=True)


@pytest.mark.parametrize("T", [1, 4])
def test_fp8_grid_exact(T):
    spec = W.custom("fp8grid", 2, T, (2500, 4100), 64, 128, 2048, 128, idx_dtype="fp8",
                    values="fp8grid")
    _run(spec, exact=True)


@pytest.mark.parametrize("HI,DI,T", [(8, 64, 1), (16, 128, 4), (32, 64, 2), (64, 64, 4), (8, 128, 3)])
def test_fp8_grid_other_shapes_exact(HI, DI, T):
    """The per-page fp8 indexer at other head counts and dims (decode, two rows, verify), on the
    exact fp8 grid: the indices equal the oracle's bit for bit."""
    spec = W.custom(f"fp8grid_{HI}x{DI}", 3, T, (2500, 777, 4100), HI, DI, 300, 16, idx_dtype="fp8",
                    values="fp8grid")
    _run(spec, exact=True, check_sfa=False)


@pytest.mark.parametrize("HI,DI,K", [(8, 64, 256), (16, 128, 100), (32, 64, 512), (64, 64, 1)])
def test_other_indexer_shapes_exact(HI, DI, K):
    spec = W.custom(f"grid_{HI}x{DI}", 2, 2, (1500, 777), HI, DI, K, 16, values="grid8")
    _run(spec, exact=True)


# ---------------------------------------------------------------- edge cases
@pytest.mark.parametrize("T,lens,K", [
    (1, (100, 2048, 2049, 1), 2048),     # n < K, n == K, n == K + 1, a single token
    (4, (5, 70, 4), 8),                  # T = 4 with tiny contexts (n = 1 .. 70)
    (2, (65, 129, 4095, 4097), 64),      # page and slice boundaries
])
def test_edge_lengths_exact(T, lens, K):
    spec = W.custom("edges", len(lens), T, lens, 64, 128, K, 32, values="grid8")
    _run(spec, exact=True)


def test_page_permutation_and_determinism():
    spec = W.config(2, "small")
    c = W.make_case(spec)
    d1 = Dev(c)
    i1 = d1.indexer(); o1, l1 = d1.attn(i1)
    i1b = d1.indexer(); o1b, l1b = d1.attn(i1b)
    d2 = Dev(W.permute_pages(c))
    i2 = d2.indexer(); o2, l2 = d2.attn(i2)
    torch.cuda.synchronize()
    for x, y in [(i1, i1b), (o1, o1b), (l1, l1b), (i1, i2), (o1, o2), (l1, l2)]:
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


# ---------------------------------------------------------------- attention closed forms
def _attn_case(H=128, lens=(700, 300), T=1, values="sharp"):
    return W.make_case(W.custom("attn", len(lens), T, lens, 8, 64, 64, H, values=values,
                                sharp_c=3.0))


def test_attn_single_row_is_v_row_bitexact():
    c = _attn_case()
    d = Dev(c)
    idx = np.full((2, 1, 64), -1, np.int32)
    idx[0, 0, 0] = 650
    idx[1, 0, 0] = 3
    out, lse = d.attn(idx)
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for b, s in [(0, 650), (1, 3)]:
        row = c.kv_cache[c.block_table[b, s // 64], s % 64, :512]
        assert np.array_equal(o[b, 0], np.broadcast_to(row, o[b, 0].shape))


def test_attn_empty_rows_and_equal_logits():
    c = _attn_case(H=48, values="gauss")
    c.q_attn[1] = 0                       # sequence 1: all logits 0 -> mean of V
    d = Dev(c)
    idx = np.full((2, 1, 96), -1, np.int32)
    sel = np.array([0, 5, 64, 65, 128, 200, 299])
    idx[1, 0, :7] = sel
    out, lse = d.attn(idx)
    torch.cuda.synchronize()
    o, l = to_np(out), to_np(lse)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    ref = oracle.sparse_attn_ref(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx, 1 / 24)
    check_attn(o[1:], l[1:], ref[0][1:], ref[1][1:])
    np.testing.assert_allclose(l[1], np.log(7.0), rtol=1e-5)


def test_attn_logit_spread_restarts():
    """Logits that jump far above the first tile's max inside one split (the softmax reference
    has to move twice) still give the exact softmax."""
    B, L, K = 64, 3000, 2048
    c = W.make_case(W.custom("attn_spread", B, 1, (L,) * B, 8, 64, K, 32, values="sharp",
                             sharp_c=1.0))
    one = W.f32_to_bf16_bits(np.float32(1.0))
    big = {1300: 8.0, 1400: 64.0, 700: 2.0}   # logits 8*576/24, 64*576/24, 2*576/24
    for b in (0, 1):
        c.q_attn[b, 0] = one
        for pos, v in big.items():
            c.kv_cache[c.block_table[b, pos // 64], pos % 64] = W.f32_to_bf16_bits(np.float32(v))
    idx = np.broadcast_to(np.arange(K, dtype=np.int32), (B, 1, K)).copy()
    d = Dev(c)
    out, lse = d.attn(idx)
    torch.cuda.synchronize()
    rows = [(0, 0), (1, 0), (2, 0)]
    o_ref, l_ref = oracle.sparse_attn_ref(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx,
                                          c.spec.sm_scale, rows=rows)
    check_attn(to_np(out)[:3], to_np(lse)[:3], o_ref[:3], l_ref[:3])
    assert np.all(to_np(out)[:2] == 64.0)


@pytest.mark.parametrize("B,K", [(1, 2048), (3, 1000), (300, 64)])
def test_attn_random_index_sets_sharp(B, K):
    """Random unique index sets (several splits when B is small, none when B is large)."""
    rng = np.random.default_rng(B)
    lens = tuple(int(x) for x in rng.integers(K, K + 3000, B))
    c = W.make_case(W.custom("attn_rand", B, 1, lens, 8, 64, K, 128, values="sharp", sharp_c=1.0))
    idx = np.full((B, 1, K), -1, np.int32)
    for b in range(B):
        m = int(rng.integers(1, K + 1))
        idx[b, 0, :m] = np.sort(rng.choice(lens[b], m, replace=False))
    d = Dev(c)
    out, lse = d.attn(idx)
    torch.cuda.synchronize()
    rows = [(b, 0) for b in range(min(B, 40))]
    o_ref, l_ref = oracle.sparse_attn_ref(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx,
                                          1 / 24, rows=rows)
    check_attn(to_np(out), to_np(lse), o_ref, l_ref, rows=rows)


@pytest.mark.parametrize("H", [32, 48, 64, 96])
def test_attn_head_counts(H):
    """Head counts that give one wave per workgroup (32), two (48: the second group half full; 64)
    and two head chunks of two groups with the last one empty (96), on random index sets with
    several splits per row."""
    rng = np.random.default_rng(H)
    B, K = 3, 700
    lens = (K + 10, 2500, 4100)
    c = W.make_case(W.custom(f"attn_h{H}", B, 1, lens, 8, 64, K, H, values="sharp", sharp_c=1.0))
    idx = np.full((B, 1, K), -1, np.int32)
    for b in range(B):
        m = int(rng.integers(1, K + 1))
        idx[b, 0, :m] = np.sort(rng.choice(lens[b], m, replace=False))
    print(f"[case] attention heads {H}", flush=True)
    d = Dev(c)
    out, lse = d.attn(idx)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.sparse_attn_ref(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx, 1 / 24)
    check_attn(to_np(out), to_np(lse), o_ref, l_ref)
