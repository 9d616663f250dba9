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
