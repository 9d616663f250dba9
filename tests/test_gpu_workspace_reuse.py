"""Indexer workspace reuse across calls.

The select leaves every row's histogram and counters zero once it has read them, and the decode /
grouped score kernels read a started row before clearing it, clearing only a row they find dirty
(the first call on a workspace, or one that a call of another shape or a caller left dirty).
These tests drive one workspace through dirty, clean, scribbled and re-laid-out states and check
every result against the oracle; the results of one case must also be identical call to call."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_15_amd as dsa
import workloads as W
from tests._gpu import Dev, check_indices_band, oracle_args, to_np

pytestmark = pytest.mark.gpu


def _ref(c, T):
    return oracle.indexer_topk_ref(**oracle_args(c), T=T, K=c.spec.K, dtype="bf16", return_scores=True)


def _need(d):
    s = d.c.spec
    lay = dsa.make_layout(d.bt, d.sl, d.c.num_pages, s.max_len)
    return dsa.dsa_indexer_workspace_size(lay, dsa.IndexerShape(s.T, s.HI, s.DI, s.K, dsa.DSA_BF16))


@pytest.mark.parametrize("T", [1, 4])
def test_workspace_dirty_clean_scribbled_relaid(T):
    # rows of 2600..40000 keys: one-segment rows and a three-segment row (its last segment clears)
    c = W.make_case(W.custom("wsreuse", 3, T, (2600, 9000, 40000), 64, 128, 2048, 16))
    c2 = W.make_case(W.custom("wsreuse2", 5, T, (3000, 2100, 7000, 12000, 2500), 64, 128, 2048, 16))
    d, d2 = Dev(c), Dev(c2)
    ws = torch.full((max(_need(d), _need(d2)),), 0xA5, dtype=torch.uint8, device="cuda:0")
    ref, extra = _ref(c, T)
    ref2, extra2 = _ref(c2, T)

    first = to_np(d.indexer(workspace=ws))                       # dirty workspace: rows cleared
    check_indices_band(first, ref, extra, 2048, c.seq_lens, T)
    again = to_np(d.indexer(workspace=ws))                       # rows left clear by the select
    assert np.array_equal(again, first)
    ws.random_(0, 256)                                           # a caller scribbles over it
    assert np.array_equal(to_np(d.indexer(workspace=ws)), first)
    other = to_np(d2.indexer(workspace=ws))                      # another shape, another layout
    check_indices_band(other, ref2, extra2, 2048, c2.seq_lens, T)
    assert np.array_equal(to_np(d.indexer(workspace=ws)), first)
    assert np.array_equal(to_np(d2.indexer(workspace=ws)), other)
    dsa.dsa_debug_status()


def test_workspace_across_modes():
    """One workspace through decode (T = 1), two query rows (T = 2: cleared by its own launch),
    verify (T = 4) and decode again, each on its own layout of the same memory; every result
    matches the oracle and the repeated decode call its first result."""
    lens = (2600, 9000, 40000)
    cases = [W.make_case(W.custom(f"wsmode{T}", 3, T, lens, 64, 128, 2048, 16)) for T in (1, 2, 4)]
    devs = [Dev(c) for c in cases]
    ws = torch.full((max(_need(d) for d in devs),), 0xA5, dtype=torch.uint8, device="cuda:0")
    refs = [_ref(c, c.spec.T) for c in cases]
    got = []
    for d, c, (ref, extra) in zip(devs, cases, refs):
        idx = to_np(d.indexer(workspace=ws))
        check_indices_band(idx, ref, extra, 2048, c.seq_lens, c.spec.T)
        got.append(idx)
    assert np.array_equal(to_np(devs[0].indexer(workspace=ws)), got[0])
    dsa.dsa_debug_status()
