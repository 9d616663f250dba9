"""GPU parity at the five workloads' full sizes (and their MXFP8-indexer and FP8-latent-cache
variants), in the launch configuration bench.py times.

Decode and verify workloads are compared with the oracle on every query row (near-tie index gate,
then the attention gates on the GPU's own indices); the causal prefill chunks on 256 rows spread
over t, first and last included.  Every row is also checked for the properties that hold at any
size: K' = min(K, n) distinct positions inside [0, n), strictly ascending, then -1 padding.  The
output and workspace buffers carry canary regions that must be untouched after each call.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._gpu import Dev, attn_ref, check_attn, check_indices_band, oracle_args, to_np

pytestmark = pytest.mark.gpu


def _row_properties(idx, spec, seq_lens):
    for b in range(spec.B):
        for t in range(spec.T):
            n = int(seq_lens[b]) - spec.T + t + 1
            kp = min(spec.K, n)
            r = idx[b, t]
            assert np.all(r[kp:] == -1), (b, t)
            v = r[:kp]
            assert np.all(v >= 0) and np.all(v < n), (b, t)
            assert np.all(np.diff(v) > 0), (b, t)


PREFILL_ROWS = sorted({int(t) for t in np.linspace(0, 8191, 254)} | {2047, 2048})


@pytest.mark.parametrize("cfg,rows", [
    (2, "all"), (4, "all"), (5, "all"), (6, "all"), (8, "all"), (9, "all"),
    (3, [(0, t) for t in PREFILL_ROWS]),
    (7, [(0, t) for t in PREFILL_ROWS]),
])
def test_full_size_rows(cfg, rows):
    spec = W.config(cfg)
    if rows == "all":
        rows = [(b, t) for b in range(spec.B) for t in range(spec.T)]
    print(f"[case] full {spec.name}: {len(rows)} rows", flush=True)
    c = W.make_case(spec)
    d = Dev(c)
    idx_t = d.indexer()
    out_t, lse_t = d.attn(idx_t)
    torch.cuda.synchronize()
    idx = to_np(idx_t)
    _row_properties(idx, spec, c.seq_lens)
    ref, extra = oracle.indexer_topk_ref(**oracle_args(c), T=spec.T, K=spec.K, dtype=spec.idx_dtype,
                                         rows=rows, return_scores=True)
    swaps = check_indices_band(idx, ref, extra, spec.K, c.seq_lens, spec.T, rows=rows)
    print(f"[case] band swaps over {len(rows)} rows: {swaps}", flush=True)
    o_ref, l_ref = attn_ref(c, idx, rows=rows)
    bi = [r[0] for r in rows]
    ti = [r[1] for r in rows]
    check_attn(to_np(out_t[bi, ti]), to_np(lse_t[bi, ti]), o_ref[bi, ti], l_ref[bi, ti])


def test_full_size_mxfp8_grid_exact_rows():
    """The exact MXFP8 grid at the MXFP8 workload's full shape (8 x 131072 keys): sampled rows must
    match the oracle bit for bit on every row (every fp32 partial sum is exact)."""
    spec = W.custom("mxgrid_full", 8, 1, (131072,) * 8, 64, 128, 2048, 128, idx_dtype="mxfp8",
                    values="mxgrid", cfg_id=6)
    rows = [(b, 0) for b in range(8)]
    print(f"[case] full {spec.name} rows {rows}", flush=True)
    c = W.make_case(spec)
    idx = to_np(Dev(c).indexer())
    torch.cuda.synchronize()
    _row_properties(idx, spec, c.seq_lens)
    ref = oracle.indexer_topk_ref(**oracle_args(c), T=1, K=spec.K, dtype="mxfp8", rows=rows)
    for b, t in rows:
        np.testing.assert_array_equal(idx[b, t], ref[b, t])
