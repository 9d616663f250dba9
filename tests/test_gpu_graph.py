"""Capturing the decode indexer call in a HIP graph.  The call launches no memset and allocates
nothing, so it can be captured; the decode score kernel clears each row's histogram itself and
publishes a per-call tag that the select resets, so replays (which reuse the captured tag) stay
correct.  Each replay runs on new query contents, with eager calls on the same workspace and
synchronisations in between, and is checked against an eager call on the same inputs."""
import numpy as np
import pytest
import torch

import sparse_attention_15_amd as dsa
import workloads as W
from tests._gpu import Dev, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [2, 6])
def test_decode_indexer_graph_replays(cfg):
    spec = W.config(cfg, "small")
    print(f"[case] graph {spec.name}", flush=True)
    c = W.make_case(spec)
    d = Dev(c)
    layout = dsa.make_layout(d.bt, d.sl, c.num_pages, spec.max_len)
    dt = dsa.DSA_MXFP8_E4M3 if d.mx else (dsa.DSA_FP8_E4M3 if d.fp8 else dsa.DSA_BF16)
    shape = dsa.IndexerShape(1, spec.HI, spec.DI, spec.K, dt)
    ws = torch.empty(max(256, dsa.dsa_indexer_workspace_size(layout, shape)), dtype=torch.uint8,
                     device=d.q_idx.device)
    out = torch.empty((spec.B, 1, spec.K), dtype=torch.int32, device=d.q_idx.device)
    q0 = d.q_idx.clone()
    gen = torch.Generator(device="cpu").manual_seed(5)
    variants = [q0] + [q0[:, :, torch.randperm(spec.HI, generator=gen)].contiguous() for _ in range(3)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d.indexer(idx_out=out, workspace=ws)           # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.indexer(idx_out=out, workspace=ws)
    torch.cuda.synchronize()
    for r, qv in enumerate(variants):
        d.q_idx.copy_(qv)
        # eager call on the same workspace, then the replay
        ref = to_np(d.indexer(workspace=ws).clone())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(out), ref, err_msg=f"replay {r}")
        assert (ref[:, 0, :] >= 0).sum() > 0
