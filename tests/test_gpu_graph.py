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


def test_fp8_latent_append_and_attention_graph_replays():
    """The FP8 latent-cache append followed by the FP8-cache attention, captured once and replayed
    on new rows and queries (eager work and synchronisations between replays); every replay must
    equal the eager calls bit for bit."""
    spec = W.custom("kv8_graph", 2, 1, (2600, 4100), 8, 64, 256, 128, kv_dtype="fp8")
    print(f"[case] graph {spec.name}", flush=True)
    c = W.make_case(spec, poison=False)
    d = Dev(c)
    T = 16
    dev = d.q_attn.device
    rng = np.random.default_rng(8)
    idx = np.full((2, 1, spec.K), -1, np.int32)
    for b in range(2):
        n = int(c.seq_lens[b])
        idx[b, 0, :200] = np.sort(np.r_[np.arange(n - T, n), rng.choice(n - T, 184, replace=False)])
    idx_t = torch.from_numpy(idx).to(dev)
    new = torch.empty((2, T, 576), dtype=torch.bfloat16, device=dev)
    out = torch.empty((2, 1, spec.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((2, 1, spec.H), dtype=torch.float32, device=dev)
    layout = dsa.make_layout(d.bt, d.sl, c.num_pages, spec.max_len)
    ws = torch.empty(max(256, dsa.dsa_sparse_attn_workspace_size(
        layout, dsa.AttnShape(1, spec.H, 576, 512, spec.K, spec.sm_scale))), dtype=torch.uint8, device=dev)

    def calls(o, l):
        dsa.dsa_latent_cache_append_fp8(new, d.kv, d.kv_scale, d.bt, d.sl, max_seq_len=spec.max_len,
                                        num_pages=c.num_pages)
        d.attn(idx_t, out=o, lse=l, workspace=ws)

    gen = torch.Generator(device="cpu").manual_seed(9)
    new.copy_((torch.randn((2, T, 576), generator=gen) / 24).to(torch.bfloat16))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls(out, lse)                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(out, lse)
    torch.cuda.synchronize()
    q0 = d.q_attn.clone()
    for r in range(4):
        new.copy_((torch.randn((2, T, 576), generator=gen) / 24).to(torch.bfloat16))
        d.q_attn.copy_(q0 * (1.0 + 0.25 * r))
        o_ref = torch.empty_like(out)
        l_ref = torch.empty_like(lse)
        calls(o_ref, l_ref)                               # eager on the same buffers
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16)), f"replay {r}"
        assert torch.equal(lse, l_ref), f"replay {r}"


@pytest.mark.parametrize("cfg", [5, 3])
def test_indexer_and_attention_step_graph_replays(cfg):
    """A whole step (indexer, then attention on its indices) of the verify (T = 4) and causal
    prefill shapes, captured once and replayed on new queries with eager steps on the same
    buffers in between; every replay equals the eager step bit for bit."""
    spec = W.config(cfg, "small")
    print(f"[case] graph step {spec.name}", flush=True)
    c = W.make_case(spec)
    d = Dev(c)
    dev = d.q_idx.device
    layout = dsa.make_layout(d.bt, d.sl, c.num_pages, spec.max_len)
    ishape = dsa.IndexerShape(spec.T, spec.HI, spec.DI, spec.K, dsa.DSA_BF16)
    ashape = dsa.AttnShape(spec.T, spec.H, 576, 512, spec.K, spec.sm_scale)
    iws = torch.empty(max(256, dsa.dsa_indexer_workspace_size(layout, ishape)), dtype=torch.uint8, device=dev)
    aws = torch.empty(max(256, dsa.dsa_sparse_attn_workspace_size(layout, ashape)), dtype=torch.uint8, device=dev)
    idx = torch.empty((spec.B, spec.T, spec.K), dtype=torch.int32, device=dev)
    out = torch.empty((spec.B, spec.T, spec.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((spec.B, spec.T, spec.H), dtype=torch.float32, device=dev)

    def step(i_out, o, l):
        d.indexer(idx_out=i_out, workspace=iws)
        d.attn(i_out, out=o, lse=l, workspace=aws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(idx, out, lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(idx, out, lse)
    torch.cuda.synchronize()
    qi0, qa0 = d.q_idx.clone(), d.q_attn.clone()
    gen = torch.Generator(device="cpu").manual_seed(7)
    for r in range(3):
        perm = torch.randperm(spec.HI, generator=gen)
        d.q_idx.copy_(qi0[:, :, perm].contiguous())
        d.q_attn.copy_(qa0 * (1.0 + 0.5 * r))
        i_ref = torch.empty_like(idx)
        o_ref = torch.empty_like(out)
        l_ref = torch.empty_like(lse)
        step(i_ref, o_ref, l_ref)                          # eager, same workspaces
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, i_ref), f"replay {r}: indices"
        assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16)), f"replay {r}: out"
        assert torch.equal(lse, l_ref), f"replay {r}: lse"


def test_fp8_cache_append_and_indexer_graph_replays():
    """The per-page fp8 cache append followed by the fp8 indexer, captured once and replayed on new
    keys and queries from the same starting cache (the eager calls and synchronisations in between);
    codes, page scales and indices of every replay equal the eager calls' bit for bit.  The new
    keys grow from replay to replay, so page scales rise and held keys are re-encoded."""
    spec = W.custom("fp8page_graph", 2, 1, (2600, 4100), 64, 128, 256, 16, idx_dtype="fp8")
    print(f"[case] graph {spec.name}", flush=True)
    c = W.make_case(spec, poison=False)
    d = Dev(c)
    T = 40
    dev = d.q_idx.device
    k0, s0 = d.k.clone(), d.k_scale.clone()
    new = torch.empty((2, T, spec.DI), dtype=torch.bfloat16, device=dev)
    out = torch.empty((2, 1, spec.K), dtype=torch.int32, device=dev)
    layout = dsa.make_layout(d.bt, d.sl, c.num_pages, spec.max_len)
    shape = dsa.IndexerShape(1, spec.HI, spec.DI, spec.K, dsa.DSA_FP8_E4M3)
    ws = torch.empty(max(256, dsa.dsa_indexer_workspace_size(layout, shape)), dtype=torch.uint8, device=dev)

    def calls(o):
        dsa.dsa_indexer_cache_append_fp8(new, d.k, d.k_scale, d.bt, d.sl, max_seq_len=spec.max_len,
                                         num_pages=c.num_pages)
        d.indexer(idx_out=o, workspace=ws)

    gen = torch.Generator(device="cpu").manual_seed(10)

    def fresh(r):
        return (torch.randn((2, T, spec.DI), generator=gen) * (0.1 * 4.0 ** r)).to(torch.bfloat16)

    new.copy_(fresh(0))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls(out)                                        # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(out)
    torch.cuda.synchronize()
    q0 = d.q_idx.clone()
    raised = False
    for r in range(4):
        new.copy_(fresh(r))
        d.q_idx.copy_(q0[:, :, torch.randperm(spec.HI, generator=gen)])
        d.k.copy_(k0)
        d.k_scale.copy_(s0)
        ref = torch.empty_like(out)
        calls(ref)                                        # eager, from the starting cache
        torch.cuda.synchronize()
        ref_k, ref_s = d.k.clone(), d.k_scale.clone()
        d.k.copy_(k0)
        d.k_scale.copy_(s0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.k, ref_k), f"replay {r}: codes"
        assert torch.equal(d.k_scale.view(torch.int32), ref_s.view(torch.int32)), f"replay {r}: scales"
        assert torch.equal(out, ref), f"replay {r}: indices"
        raised |= bool((ref_s != s0).any())
    assert raised
