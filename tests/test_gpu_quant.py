"""GPU parity of the MXFP8 quantiser and the paged cache append ("Inference Optimization for Kimi
K3.1 Pro", §3: the indexer prolog writes the new keys into the cache; §4: MXFP8 indexer storage)
through the C ABI, against the CPU oracle.  Codes and scale bytes are byte outputs: bit-exact.

Inputs mix group magnitudes over many octaves, all-zero groups, groups whose small elements land
on E4M3 subnormals or round to (signed) zero, elements near 448 * scale, and exact ties.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_15_amd as dsa
import workloads as W
from oracle.quant import cache_append_ref, mxfp8_quantize_rows
from tests._gpu import DEV, Dev, oracle_args, to_np, up

pytestmark = pytest.mark.gpu


def _bf16_rows(shape, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * 10.0 ** rng.integers(-6, 5, shape[:-1] + (shape[-1] // 32, 1)).repeat(32, -1).reshape(shape)
    x = x.astype(np.float32)
    flat = x.reshape(-1, 32)
    flat[::7] = 0.0                                        # all-zero groups
    flat[1::11, 1:] *= 1e-4                                # one large element: the rest near/below the subnormals
    flat[2::13, 3] = -0.0
    flat[3::17, :] = np.float32(448.0) * np.float32(2.0 ** -5)   # exact powers: amax on a binade edge
    return W.f32_to_bf16_bits(x)


def _decode_bf16(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("rows,dim", [(1, 32), (333, 128), (4096, 64), (20, 4096)])
def test_quantize_rows_bit_exact(rows, dim):
    print(f"[case] quantize rows={rows} dim={dim}", flush=True)
    bits = _bf16_rows((rows, dim), seed=rows + dim)
    codes, scales = dsa.dsa_mxfp8_quantize(up(bits))
    torch.cuda.synchronize()
    ref_c, ref_s = mxfp8_quantize_rows(_decode_bf16(bits))
    np.testing.assert_array_equal(to_np(scales), ref_s)
    np.testing.assert_array_equal(to_np(codes), ref_c)


@pytest.mark.parametrize("T,lens", [(1, (130, 64, 4097)), (4, (4, 200, 1000)), (64, (64, 128))])
def test_cache_append_bit_exact(T, lens):
    print(f"[case] append T={T} lens={lens}", flush=True)
    spec = W.custom("append", len(lens), T, lens, 8, 128, 64, 16, idx_dtype="mxfp8")
    c = W.make_case(spec)
    rng = np.random.default_rng(7)
    # the cache holds other contents (noise) everywhere; only the appended slots may change
    kc = rng.integers(0, 256, c.k_cache.shape).astype(np.uint8)
    ks = rng.integers(0, 256, c.k_scale.shape).astype(np.uint8)
    new = _bf16_rows((len(lens), T, 128), seed=T)
    kc_d, ks_d = up(kc), up(ks)
    dsa.dsa_indexer_cache_append(up(new), kc_d, ks_d, up(c.block_table), up(c.seq_lens),
                                 max_seq_len=spec.max_len, num_pages=c.num_pages)
    torch.cuda.synchronize()
    ref_c, ref_s = cache_append_ref(_decode_bf16(new), kc, ks, c.block_table, c.seq_lens, T)
    np.testing.assert_array_equal(to_np(ks_d), ref_s)
    np.testing.assert_array_equal(to_np(kc_d), ref_c)


def test_prolog_then_indexer_end_to_end():
    """Quantise the queries and append every key through the library, then run the MXFP8 indexer:
    its indices equal the oracle's on the library-written codes (which the tests above show equal
    the oracle's own quantisation)."""
    spec = W.custom("prolog", 2, 1, (3000, 4500), 64, 128, 2048, 16, idx_dtype="mxfp8")
    c = W.make_case(spec)
    B, L = 2, 4500     # keys drawn for the longer context
    q_bits = _bf16_rows((B, 1, 64, 128), seed=11)
    k_bits = _bf16_rows((B, L, 128), seed=12)
    q_codes, q_sc = dsa.dsa_mxfp8_quantize(up(q_bits))
    kc = torch.zeros(c.k_cache.shape, dtype=torch.uint8, device=DEV)
    ks = torch.zeros(c.k_scale.shape, dtype=torch.uint8, device=DEV)
    bt, sl = up(c.block_table), up(c.seq_lens)
    # two appends write every key of both contexts (3000 and 4500): sequence 1's last 3000 with
    # sequence 0's whole context, then sequence 1's first 1500 with sequence 0's last 1500 again
    n0, n1 = 3000, 4500
    new1 = np.stack([k_bits[0, :n0], k_bits[1, n1 - n0:n1]])
    dsa.dsa_indexer_cache_append(up(new1), kc, ks, bt, up(np.array([n0, n1], np.int32)),
                                 max_seq_len=L, num_pages=c.num_pages)
    new2 = np.stack([k_bits[0, n0 - 1500:n0], k_bits[1, :1500]])
    dsa.dsa_indexer_cache_append(up(new2), kc, ks, bt, up(np.array([n0, 1500], np.int32)),
                                 max_seq_len=L, num_pages=c.num_pages)
    idx = dsa.dsa_indexer_topk(q_codes, q_sc, up(c.w), kc, ks, bt, sl, T=1, top_k=spec.K,
                               max_seq_len=spec.max_len, mx=True, num_pages=c.num_pages)
    torch.cuda.synchronize()
    got = to_np(idx)
    args = dict(oracle_args(c), q_idx=to_np(q_codes), q_scale=to_np(q_sc), k_cache=to_np(kc),
                k_scale=to_np(ks))
    ref, extra = oracle.indexer_topk_ref(**args, T=1, K=spec.K, dtype="mxfp8", return_scores=True)
    from tests._gpu import check_indices_band
    check_indices_band(got, ref, extra, spec.K, c.seq_lens, 1)


# ---------------------------------------------------------------- FP8 latent-cache append
from oracle.quant import latent_cache_append_fp8_ref  # noqa: E402


def _latent_rows(B, T, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((B, T, 576)) * 10.0 ** rng.integers(-5, 3, (B, T, 5)).repeat(
        [128, 128, 128, 128, 64], axis=-1)).astype(np.float32)
    x[0, 0, :128] = 0.0                                   # an all-zero tile
    x[0, -1, 512:] *= 1e-5                                # rope tile far below the value tiles
    x[-1, 0, 3] = -0.0
    x[-1, -1, 130] = np.float32(448.0) * np.float32(2.0 ** -7)
    return W.f32_to_bf16_bits(x)


@pytest.mark.parametrize("B,T,lens", [(3, 1, (70, 1, 3000)), (2, 5, (64, 4100)), (1, 300, (300,))])
def test_latent_fp8_append_bit_exact(B, T, lens):
    print(f"[case] latent fp8 append B={B} T={T} lens={lens}", flush=True)
    spec = W.custom("kv8_append", B, 1, lens, 8, 64, 64, 16, kv_dtype="fp8")
    c = W.make_case(spec, poison=False)
    new = _latent_rows(B, T, seed=B * 7 + T)
    codes_d, scale_d = up(c.kv_codes), up(c.kv_scale)
    dsa.dsa_latent_cache_append_fp8(up(new), codes_d, scale_d, up(c.block_table), up(c.seq_lens),
                                    max_seq_len=spec.max_len, num_pages=c.num_pages)
    torch.cuda.synchronize()
    kc_ref, ks_ref = latent_cache_append_fp8_ref(_decode_bf16(new).astype(np.float32), c.kv_codes,
                                                 c.kv_scale, c.block_table, c.seq_lens, T)
    np.testing.assert_array_equal(codes_d.cpu().numpy(), kc_ref)
    np.testing.assert_array_equal(scale_d.cpu().numpy().view(np.uint32), ks_ref.view(np.uint32))


def test_latent_fp8_append_then_attend():
    """Appended rows are read back by the FP8-cache attention like the generator's own rows."""
    spec = W.custom("kv8_append_attn", 2, 1, (2600, 4100), 8, 64, 64, 128, kv_dtype="fp8")
    c = W.make_case(spec, poison=False)
    T = 40
    # unit-scale rows like the generator's (N(0, 1) / 24): the attention gates assume that scale
    rng0 = np.random.default_rng(5)
    new = W.f32_to_bf16_bits((rng0.standard_normal((2, T, 576)) / 24).astype(np.float32))
    codes_d, scale_d = up(c.kv_codes), up(c.kv_scale)
    dsa.dsa_latent_cache_append_fp8(up(new), codes_d, scale_d, up(c.block_table), up(c.seq_lens),
                                    max_seq_len=spec.max_len, num_pages=c.num_pages)
    kc, ks = latent_cache_append_fp8_ref(_decode_bf16(new).astype(np.float32), c.kv_codes, c.kv_scale,
                                         c.block_table, c.seq_lens, T)
    rng = np.random.default_rng(6)
    idx = np.full((2, 1, 64), -1, np.int32)
    for b in range(2):
        n = int(c.seq_lens[b])
        idx[b, 0] = np.sort(np.r_[np.arange(n - T, n), rng.choice(n - T, 24, replace=False)])
    out, lse = dsa.dsa_sparse_attn_fp8kv(up(c.q_attn), codes_d, scale_d, up(idx), up(c.block_table),
                                         up(c.seq_lens), sm_scale=spec.sm_scale, max_seq_len=spec.max_len,
                                         num_pages=c.num_pages)
    torch.cuda.synchronize()
    from tests._gpu import check_attn
    o_ref, l_ref = oracle.sparse_attn_fp8kv_ref(c.q_attn, kc, ks, c.block_table, c.seq_lens, idx, spec.sm_scale)
    check_attn(to_np(out), to_np(lse), o_ref, l_ref)


# ---------------------------------------------------------------- per-head fp8 queries
from oracle.quant import fp8_quantize_heads  # noqa: E402


@pytest.mark.parametrize("rows,dim", [(1, 64), (37, 128), (4099, 64), (2050, 128)])
def test_fp8_heads_bit_exact(rows, dim):
    print(f"[case] fp8 heads rows={rows} dim={dim}", flush=True)
    rng = np.random.default_rng(rows + dim)
    x = (rng.standard_normal((rows, dim)) * 10.0 ** rng.integers(-6, 4, (rows, 1))).astype(np.float32)
    x[::9] = 0.0
    x[1::7, 1:] *= 1e-5
    x[2::11, 5] = -0.0
    bits = W.f32_to_bf16_bits(x)
    codes, sc = dsa.dsa_fp8_quantize_heads(up(bits))
    torch.cuda.synchronize()
    c_ref, s_ref = fp8_quantize_heads(_decode_bf16(bits).astype(np.float32))
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)
    np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_fp8_heads_feed_the_fp8_indexer():
    """Queries quantised on the device drive the fp8 indexer to the oracle's selection on the same
    codes and scales."""
    spec = W.config(4, "small")
    c = W.make_case(spec)
    rng = np.random.default_rng(41)
    qf = W.f32_to_bf16_bits((rng.standard_normal((spec.B, spec.T, spec.HI, spec.DI)) / np.sqrt(spec.DI)).astype(np.float32))
    codes, sq = dsa.dsa_fp8_quantize_heads(up(qf))
    d = Dev(c)
    d.q_idx, d.q_scale = codes, sq
    idx = to_np(d.indexer())
    torch.cuda.synchronize()
    import dataclasses
    c2 = dataclasses.replace(c, q_idx=codes.cpu().numpy(), q_scale=sq.cpu().numpy())
    ref, extra = oracle.indexer_topk_ref(**oracle_args(c2), T=1, K=spec.K, dtype="fp8", return_scores=True)
    from tests._gpu import check_indices_band
    check_indices_band(idx, ref, extra, spec.K, c.seq_lens, 1)


def test_latent_fp8_append_bench_size_every_row():
    """The append at the benchmark's size (8 sequences x 16384 rows into 2049 permuted pages, the
    launch bench.py times): every row's codes and scales bit-exact against the oracle's quantiser."""
    B, T, D = 8, 16384, 576
    P = B * T // 64 + 1
    gen = torch.Generator(device=DEV).manual_seed(16)
    perm = torch.randperm(P, device=DEV, generator=gen).to(torch.int32)
    bt = perm[:B * T // 64].view(B, T // 64).contiguous()
    sl = torch.full((B,), T, dtype=torch.int32, device=DEV)
    src = (torch.randn(B, T, D, device=DEV, generator=gen) / 24).to(torch.bfloat16)
    kc = torch.zeros(P, 64, D, dtype=torch.uint8, device=DEV)
    ks = torch.zeros(P, 64, 8, dtype=torch.float32, device=DEV)
    print("[case] latent fp8 append bench size", flush=True)
    dsa.dsa_latent_cache_append_fp8(src, kc, ks, bt, sl, max_seq_len=T, num_pages=P)
    torch.cuda.synchronize()
    from oracle.quant import latent_fp8_quantize_rows
    c_ref, s_ref = latent_fp8_quantize_rows(src.float().cpu().numpy())
    pages = bt.cpu().numpy()                       # sequence b's token t sits at page t // 64
    np.testing.assert_array_equal(to_np(kc)[pages].reshape(B, T, D), c_ref)
    got_s = to_np(ks)[pages].reshape(B, T, 8)
    np.testing.assert_array_equal(got_s[..., :5].view(np.uint32), s_ref[..., :5].view(np.uint32))
    assert (got_s[..., 5:] == 1.0).all()


def test_cache_append_bench_size_every_row():
    """The MXFP8 append at the benchmark's size (8 sequences x 65536 new keys x 128 dims into 8193
    permuted pages, the launch bench.py times): every code and scale byte against the oracle."""
    B, T, D = 8, 65536, 128
    P = B * T // 64 + 1
    gen = torch.Generator(device=DEV).manual_seed(15)
    perm = torch.randperm(P, device=DEV, generator=gen).to(torch.int32)
    bt = perm[:B * T // 64].view(B, T // 64).contiguous()
    sl = torch.full((B,), T, dtype=torch.int32, device=DEV)
    src = torch.randn(B, T, D, device=DEV, generator=gen).to(torch.bfloat16)
    kc = torch.zeros(P, 64, D, dtype=torch.uint8, device=DEV)
    ks = torch.zeros(P, 64, D // 32, dtype=torch.uint8, device=DEV)
    print("[case] mxfp8 append bench size", flush=True)
    dsa.dsa_indexer_cache_append(src, kc, ks, bt, sl, max_seq_len=T, num_pages=P)
    torch.cuda.synchronize()
    ref_c, ref_s = mxfp8_quantize_rows(src.float().cpu().numpy().astype(np.float64))
    pages = bt.cpu().numpy()                       # [B, T / 64]: sequence b's token t at page t // 64
    got_c = to_np(kc)[pages].reshape(B, T, D)
    got_s = to_np(ks)[pages].reshape(B, T, D // 32)
    np.testing.assert_array_equal(got_s, ref_s)
    np.testing.assert_array_equal(got_c, ref_c)
