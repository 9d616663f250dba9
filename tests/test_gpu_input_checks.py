"""Device-side precondition checks (dsa_debug_status).

The kernels clamp or skip inputs that violate a device-side precondition, so such inputs never
address outside the buffers, and record which kind they met; valid inputs record nothing.  Every
input here is handled by those in-kernel checks (a page id is clamped into the pool, an index past
the visible range is skipped)."""
import pytest
import torch

import sparse_attention_15_amd as dsa
import workloads as W
from tests._gpu import Dev

pytestmark = pytest.mark.gpu


def _clear():
    try:
        dsa.dsa_debug_status()
    except dsa.DsaError:
        pass


def test_valid_inputs_record_nothing():
    c = W.make_case(W.config(1))
    d = Dev(c)
    _clear()
    idx = d.indexer()
    d.attn(idx)
    dsa.dsa_debug_status()                       # raises if anything was recorded


def test_attention_index_past_the_visible_range_is_skipped_and_reported():
    c = W.make_case(W.config(1))
    d = Dev(c)
    idx = d.indexer()
    torch.cuda.synchronize()
    _clear()
    bad = idx.clone()
    bad[0, 0, 5] = int(c.seq_lens[0]) + 7        # not a visible position of row (0, 0)
    d.attn(bad)
    with pytest.raises(dsa.DsaError, match="attention index"):
        dsa.dsa_debug_status()
    dsa.dsa_debug_status()                       # reading cleared the record


def test_block_table_entry_outside_the_pool_is_clamped_and_reported():
    c = W.make_case(W.config(1))
    d = Dev(c)
    _clear()
    d.bt = d.bt.clone()
    d.bt[0, 1] = c.num_pages + 3                 # the page of positions 64..127
    d.indexer()
    with pytest.raises(dsa.DsaError, match="block_table"):
        dsa.dsa_debug_status()


def test_fp8_cache_paths_record_nothing_on_valid_inputs():
    spec = W.custom("kv8_checks", 2, 1, (300, 700), 8, 64, 64, 16, kv_dtype="fp8")
    c = W.make_case(spec, poison=False)
    d = Dev(c)
    _clear()
    new = torch.zeros((2, 3, 576), dtype=torch.bfloat16, device=d.kv.device)
    dsa.dsa_latent_cache_append_fp8(new, d.kv, d.kv_scale, d.bt, d.sl, max_seq_len=spec.max_len,
                                    num_pages=c.num_pages)
    d.attn(d.indexer())
    dsa.dsa_debug_status()


def test_latent_append_clamps_and_reports_bad_length_and_page():
    """A sequence length past max_seq_len is clamped to it, a page id outside the pool into it;
    both land inside the cache and are reported."""
    spec = W.custom("kv8_bad", 2, 1, (300, 700), 8, 64, 64, 16, kv_dtype="fp8")
    c = W.make_case(spec, poison=False)
    d = Dev(c)
    new = torch.zeros((2, 2, 576), dtype=torch.bfloat16, device=d.kv.device)
    _clear()
    sl = d.sl.clone()
    sl[1] = spec.max_len + 50
    dsa.dsa_latent_cache_append_fp8(new, d.kv, d.kv_scale, d.bt, sl, max_seq_len=spec.max_len,
                                    num_pages=c.num_pages)
    with pytest.raises(dsa.DsaError, match="seq_lens"):
        dsa.dsa_debug_status()
    bt = d.bt.clone()
    bt[0, 4] = c.num_pages + 9                   # the page of positions 256..319 (sequence 0 ends at 299)
    dsa.dsa_latent_cache_append_fp8(new, d.kv, d.kv_scale, bt, d.sl, max_seq_len=spec.max_len,
                                    num_pages=c.num_pages)
    with pytest.raises(dsa.DsaError, match="block_table"):
        dsa.dsa_debug_status()
    dsa.dsa_debug_status()


@pytest.mark.parametrize("T", [1, 4])
def test_decode_tag_wait_timeout_emits_minus_one_rows(monkeypatch, T):
    """The decode score kernel's bounded wait for a row's histogram clear, forced from the host:
    the clearing workgroups publish no tag and the waits give up after 64 sleeps.  Every kernel
    still exits; rows with n > K come out all -1 (never a selection from an uncleared histogram),
    rows with n <= K are unaffected, the handshake check is reported, and the next call without
    the hooks is correct again."""
    import numpy as np
    import oracle
    from tests._gpu import check_indices_band, oracle_args, to_np
    # T = 4: the first sequence's rows see 1497..1500 keys (all n <= K), the others more than K
    spec = W.custom("tagwait", 3, T, (1500, 2600, 4100), 64, 128, 2048, 16)
    c = W.make_case(spec)
    d = Dev(c)
    _clear()
    monkeypatch.setenv("DSA_TEST_WITHHOLD_TAG", "1")
    monkeypatch.setenv("DSA_TEST_SYNC_SPIN_CAP", "64")
    idx = to_np(d.indexer())
    monkeypatch.delenv("DSA_TEST_WITHHOLD_TAG")
    monkeypatch.delenv("DSA_TEST_SYNC_SPIN_CAP")
    for t in range(T):
        n = 1500 - T + 1 + t
        assert np.array_equal(idx[0, t], np.r_[np.arange(n), -np.ones(2048 - n)].astype(np.int32))
    assert (idx[1:] == -1).all()
    with pytest.raises(dsa.DsaError, match="handshake"):
        dsa.dsa_debug_status()
    idx = to_np(d.indexer())
    ref, extra = oracle.indexer_topk_ref(**oracle_args(c), T=T, K=2048, dtype="bf16", return_scores=True)
    check_indices_band(idx, ref, extra, 2048, c.seq_lens, T)
    dsa.dsa_debug_status()
