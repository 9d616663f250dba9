"""GPU parity of sparse attention over an FP8 latent cache ("Inference Optimization for Kimi K3.1
Pro", §4: the SFA cache in FP8 with per-token scales over 128-wide tiles, BF16 products) through the
C ABI, against the CPU oracle.

The kernel dequantises each gathered tile into the same bf16 tile the bf16 cache is gathered into,
so besides the oracle gates (attention tolerances on the GPU's own indices) the fp8 call must
match, bit for bit, the bf16 call over the cache the oracle dequantises.  Cases span one, two and
four 32-head waves per workgroup, one and several splits, ragged index tails, rows with fewer
visible positions than K and the verify shape.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests._gpu import Dev, attn_ref, check_attn, to_np, up

pytestmark = pytest.mark.gpu


def _indices(c, seed=0):
    """Valid sorted index rows: K' = min(K, n) - 3 distinct visible positions, -1 padded."""
    s = c.spec
    rng = np.random.default_rng(seed)
    idx = np.full((s.B, s.T, s.K), -1, np.int32)
    for b in range(s.B):
        for t in range(s.T):
            n = int(c.seq_lens[b]) - s.T + t + 1
            k = max(min(s.K, n) - 3, 1)
            idx[b, t, :k] = np.sort(rng.choice(n, k, replace=False))
    return idx


def _run(spec, idx=None):
    print(f"[case] {spec.name} B={spec.B} T={spec.T} H={spec.H} K={spec.K} lens={spec.lens[:4]} kv fp8",
          flush=True)
    c = W.make_case(spec)
    d = Dev(c)
    if idx is None:
        idx_t = d.indexer()
    else:
        idx_t = up(idx)
    out, lse = d.attn(idx_t)
    torch.cuda.synchronize()
    idx_np = to_np(idx_t)
    o_ref, l_ref = attn_ref(c, idx_np)
    check_attn(to_np(out), to_np(lse), o_ref, l_ref)
    # bit-identical to the bf16 path over the oracle's dequantised cache
    deq = oracle.dequant_kv_fp8(c.kv_codes, c.kv_scale)
    kv16 = up(deq)
    out16, lse16 = d.attn_bf16(idx_t, kv16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out16.view(torch.int16)), "fp8 cache != bf16 of its dequantisation"
    assert torch.equal(lse, lse16)
    return c


def test_kv8_small_decode_with_indexer():
    _run(W.config(9, "small"))


@pytest.mark.parametrize("H", [16, 64, 128])
def test_kv8_heads_and_ragged_k(H):
    spec = W.custom(f"kv8_h{H}", 3, 1, (700, 2500, 4100), 8, 64, 300, H, kv_dtype="fp8")
    c = W.make_case(spec)
    _run(spec, _indices(c, 1))


def test_kv8_verify_rows():
    spec = W.custom("kv8_verify", 2, 4, (3000, 5000), 64, 128, 2048, 128, kv_dtype="fp8")
    _run(spec)


def test_kv8_short_rows_and_padding():
    # rows with fewer visible positions than K: -1 padding inside and past the last tile
    spec = W.custom("kv8_short", 3, 1, (40, 100, 2049), 8, 64, 2048, 128, kv_dtype="fp8")
    c = W.make_case(spec)
    _run(spec, _indices(c, 2))


def test_kv8_page_permutation_bit_identical():
    spec = W.custom("kv8_perm", 2, 1, (2600, 4100), 64, 128, 2048, 128, kv_dtype="fp8")
    c = W.make_case(spec)
    c2 = W.permute_pages(c)
    idx = up(_indices(c, 3))
    o1, l1 = Dev(c).attn(idx)
    o2, l2 = Dev(c2).attn(idx)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
