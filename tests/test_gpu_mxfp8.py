"""GPU parity of the MXFP8 indexer ("Inference Optimization for Kimi K3.1 Pro", §4: the Lightning
Indexer's Q and K in MXFP8) through the C ABI, against the CPU oracle.

The exact integer-grid variant (codes in [-2, 2], power-of-two group scales, weights in sixteenths)
makes every fp32 partial sum exact, so its indices must match the oracle bit for bit; it runs at
both indexer head dims, which place 4 and 2 scale bytes per key.  The Gaussian cases (rows
quantised to MXFP8 as the OCP Microscaling format defines it) use the near-tie band.  Sizes span
several 128-key tiles, score workgroups and select scan steps, with ragged tails.  Decode runs the
decode score kernel, 2-4 query rows per sequence the verify kernel; causal prefill and more than 4
query rows per sequence run the chunked grid.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._gpu import Dev, check_attn, check_indices_band, oracle_args, to_np

pytestmark = pytest.mark.gpu


def _run(spec, exact, check_sfa=False, case=None):
    print(f"[case] {spec.name} B={spec.B} lens={spec.lens[:4]} HI={spec.HI} DI={spec.DI} K={spec.K} "
          f"{spec.idx_dtype}/{spec.values}", flush=True)
    c = case if case is not None else W.make_case(spec)
    d = Dev(c)
    idx_t = d.indexer()
    torch.cuda.synchronize()
    idx = to_np(idx_t)
    ref, extra = oracle.indexer_topk_ref(**oracle_args(c), T=1, K=spec.K, dtype="mxfp8",
                                         return_scores=True)
    if exact:
        bad = np.nonzero((idx != ref).any(axis=-1))
        assert np.array_equal(idx, ref), f"index mismatch in rows {list(zip(*bad))[:5]}"
    else:
        check_indices_band(idx, ref, extra, spec.K, c.seq_lens, 1)
    if check_sfa:
        out, lse = d.attn(idx_t)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.sparse_attn_ref(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx,
                                              spec.sm_scale)
        check_attn(to_np(out), to_np(lse), o_ref, l_ref)
    return c, idx


@pytest.mark.parametrize("HI,DI,K,lens", [(64, 128, 2048, (3000, 5000, 4545)),
                                          (8, 64, 256, (4096, 1000)),
                                          (32, 64, 300, (2100, 777))])
def test_mx_grid_exact(HI, DI, K, lens):
    spec = W.custom("mxgrid", len(lens), 1, lens, HI, DI, K, 16, idx_dtype="mxfp8", values="mxgrid")
    _run(spec, exact=True)


def test_mx_small_gaussian_decode():
    _run(W.config(6, "small"), exact=False, check_sfa=True)


def test_mx_ragged_rows_and_short_rows():
    # one row shorter than K (all positions), others with partial last pages
    spec = W.custom("mx_ragged", 4, 1, (1500, 2049, 2113, 6001), 64, 128, 2048, 16, idx_dtype="mxfp8")
    _run(spec, exact=False)


def test_mx_page_permutation_bit_identical():
    spec = W.custom("mx_perm", 2, 1, (2600, 4100), 64, 128, 2048, 16, idx_dtype="mxfp8")
    c = W.make_case(spec)
    c2 = W.permute_pages(c)
    i1 = to_np(Dev(c).indexer())
    i2 = to_np(Dev(c2).indexer())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(i1, i2)


# ---------------------------------------------------------------- chunked grid: prefill and T > 4
def _run_rows(spec, rows, exact):
    print(f"[case] {spec.name} T={spec.T} lens={spec.lens} rows={rows[:6]} {spec.values}", flush=True)
    c = W.make_case(spec)
    idx = to_np(Dev(c).indexer())
    torch.cuda.synchronize()
    ref, extra = oracle.indexer_topk_ref(**oracle_args(c), T=spec.T, K=spec.K, dtype="mxfp8",
                                         rows=rows, return_scores=True)
    if exact:
        for b, t in rows:
            np.testing.assert_array_equal(idx[b, t], ref[b, t], err_msg=f"row {(b, t)}")
    else:
        check_indices_band(idx, ref, extra, spec.K, c.seq_lens, spec.T, rows=rows)


def test_mx_prefill_grid_exact_rows():
    L = 2304
    spec = W.custom("mxgrid_prefill", 1, L, (L,), 64, 128, 2048, 16, idx_dtype="mxfp8",
                    values="mxgrid")
    rows = [(0, t) for t in (0, 1, 63, 64, 1000, 2046, 2047, 2048, 2049, 2200, 2303)]
    _run_rows(spec, rows, exact=True)


def test_mx_multi_query_grid_exact():
    # T = 6 rows per sequence is past the verify kernel: the chunked grid runs it
    spec = W.custom("mxgrid_T6", 2, 6, (3000, 4100), 64, 128, 2048, 16, idx_dtype="mxfp8",
                    values="mxgrid")
    _run_rows(spec, [(b, t) for b in range(2) for t in range(6)], exact=True)


def test_mx_small_prefill_gaussian():
    spec = W.config(7, "small")
    rows = [(0, t) for t in (0, 5, 511, 512, 800, 1099)]
    _run_rows(spec, rows, exact=False)


# ---------------------------------------------------------------- verify kernel: 2-4 rows per sequence
@pytest.mark.parametrize("T,lens", [(4, (3000, 4100, 2051)), (2, (2600, 70, 4545)), (3, (2300, 5000))])
def test_mx_verify_grid_exact(T, lens):
    spec = W.custom(f"mxgrid_verify_T{T}", len(lens), T, lens, 64, 128, 2048, 16, idx_dtype="mxfp8",
                    values="mxgrid")
    _run_rows(spec, [(b, t) for b in range(len(lens)) for t in range(T)], exact=True)


def test_mx_verify_grid_exact_dim64():
    spec = W.custom("mxgrid_verify_d64", 2, 4, (2100, 777), 32, 64, 300, 16, idx_dtype="mxfp8",
                    values="mxgrid")
    _run_rows(spec, [(b, t) for b in range(2) for t in range(4)], exact=True)


def test_mx_verify_gaussian():
    spec = W.custom("mx_verify", 3, 4, (5000, 2049, 6001), 64, 128, 2048, 16, idx_dtype="mxfp8")
    _run_rows(spec, [(b, t) for b in range(3) for t in range(4)], exact=False)
