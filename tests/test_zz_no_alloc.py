"""dsa_sparse_attn_noalloc (the attention entry point that uses the library's static per-GPU
scratch instead of a caller workspace) against dsa_sparse_attn on the same inputs: two calls in a
row, the second on a smaller input, each bitwise equal to the workspace call (same kernels, same
split plan, deterministic merge) and within the attention gates of the oracle on sampled rows."""
import numpy as np
import pytest
import torch

import sparse_attention_15_amd as dsa
import workloads as W
from tests._gpu import Dev, attn_ref, check_attn, to_np

pytestmark = pytest.mark.gpu


def _both(d, idx):
    s = d.c.spec
    out_ws, lse_ws = d.attn(idx)
    out_na, lse_na = dsa.dsa_sparse_attn_noalloc(d.q_attn, d.kv, idx, d.bt, d.sl, sm_scale=s.sm_scale,
                                                 max_seq_len=s.max_len, num_pages=d.c.num_pages)
    torch.cuda.synchronize()
    return out_ws, lse_ws, out_na, lse_na


@pytest.mark.parametrize("calls", [[(2, "full", [(0, 0), (17, 0), (31, 0)]),
                                    (5, "small", [(0, 0), (1, 3)])]])
def test_noalloc_matches_workspace_call(calls):
    for cfg, size, rows in calls:
        spec = W.config(cfg, size)
        print(f"[case] noalloc {spec.name}", flush=True)
        c = W.make_case(spec)
        d = Dev(c)
        idx = d.indexer()
        out_ws, lse_ws, out_na, lse_na = _both(d, idx)
        assert torch.equal(out_ws.view(torch.int16), out_na.view(torch.int16)), spec.name
        assert torch.equal(lse_ws.view(torch.int32), lse_na.view(torch.int32)), spec.name
        idx_np = to_np(idx)
        o_ref, l_ref = attn_ref(c, idx_np, rows=rows)
        bi = [r[0] for r in rows]
        ti = [r[1] for r in rows]
        check_attn(to_np(out_na[bi, ti]), to_np(lse_na[bi, ti]), o_ref[bi, ti], l_ref[bi, ti])
        dsa.dsa_debug_status()
