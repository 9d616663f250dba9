"""GPU parity at the five workloads' full sizes, in the launch configuration bench.py times.

The oracle cannot score every row at these sizes in seconds, so it checks sampled rows completely
(near-tie index gate, attention gates on the GPU's own indices) and every row is checked for the
properties that hold at any size: K' = min(K, n) distinct positions inside [0, n), strictly
ascending, then -1 padding.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._gpu import Dev, check_attn, check_indices_band, oracle_args, to_np

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


@pytest.mark.parametrize("cfg,rows", [
    (2, [(0, 0), (7, 0), (19, 0), (31, 0)]),
    (4, [(0, 0), (5, 0)]),
    (5, [(0, 0), (0, 3), (9, 1), (15, 2)]),
    (3, [(0, 0), (0, 2047), (0, 2048), (0, 5000), (0, 8191)]),
])
def test_full_size_sampled(cfg, rows):
    spec = W.config(cfg)
    print(f"[case] full {spec.name} rows {rows}", flush=True)
    c = W.make_case(spec)
    d = Dev(c)
    idx_t = d.indexer()
    out_t, lse_t = d.attn(idx_t)
    torch.cuda.synchronize()
    idx = to_np(idx_t)
    _row_properties(idx, spec, c.seq_lens)
    dt = "fp8" if spec.idx_dtype == "fp8" else "bf16"
    ref, extra = oracle.indexer_topk_ref(**oracle_args(c), T=spec.T, K=spec.K, dtype=dt, rows=rows,
                                         return_scores=True)
    swaps = check_indices_band(idx, ref, extra, spec.K, c.seq_lens, spec.T, rows=rows)
    print(f"[case] band swaps on sampled rows: {swaps}", flush=True)
    o_ref, l_ref = oracle.sparse_attn_ref(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx,
                                          spec.sm_scale, rows=rows)
    bi = [r[0] for r in rows]
    ti = [r[1] for r in rows]
    check_attn(to_np(out_t[bi, ti]), to_np(lse_t[bi, ti]), o_ref[bi, ti], l_ref[bi, ti])
