"""Helpers shared by the GPU parity tests: upload a synthetic case, run the HIP path through the
C ABI, and the comparison gates.

Gates (written here, used by every parity test):
  * indices, exact-arithmetic cases (integer grids): the whole [B,T,K] int32 array must match the
    oracle, order and -1 padding included;
  * indices, Gaussian cases: with theta the oracle's K'-th score and
    tau = max(1e-3 |theta|, 1e-6 max|I|), the GPU row must hold K' distinct positions in [0, pos],
    contain every s with I[s] > theta + tau and none with I[s] < theta - tau (rows with
    n <= K must equal 0..n-1 exactly);
  * attention (always on one shared index tensor): G1 |o - o_ref| <= 2e-2 + 2e-2 |o_ref|
    elementwise; G2 max_d |o - o_ref| <= 2e-2 max_d |o_ref| per (b, t, h); G3
    |lse - lse_ref| <= 1e-3 max(1, |lse_ref|).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_attention_15_amd as dsa

DEV = torch.device("cuda:0")


def up(a: np.ndarray, dtype=None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


GUARD = 4096          # bytes of canary before and after every guarded buffer
CANARY = 0xA5


class Guarded:
    """A device buffer with GUARD canary bytes on both sides (the interior keeps 256-byte
    alignment); intact() tells whether a call wrote outside the interior."""

    def __init__(self, shape, dtype, nbytes=None):
        item = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * item if nbytes is None else int(nbytes)
        n = max(n, item)
        self.raw = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.uint8, device=DEV)
        inner = self.raw[GUARD:GUARD + n]
        self.t = inner.view(dtype).view(shape) if nbytes is None else inner
        self.nbytes = n

    def intact(self) -> bool:
        return bool((self.raw[:GUARD] == CANARY).all()) and bool((self.raw[-GUARD:] == CANARY).all())


def check_guards(*bufs):
    torch.cuda.synchronize()
    for name, g in bufs:
        assert g.intact(), f"write outside {name}"


class Dev:
    """A case's tensors in device memory.  Calls made without explicit output or workspace
    buffers run on guarded buffers, and the canaries around each are checked after the call."""

    def __init__(self, c):
        self.c = c
        s = c.spec
        self.bt = up(c.block_table)
        self.sl = up(c.seq_lens)
        self.q_idx = up(c.q_idx)
        self.w = up(c.w)
        self.k = up(c.k_cache)
        self.q_scale = None if c.q_scale is None else up(c.q_scale)
        self.k_scale = None if c.k_scale is None else up(c.k_scale)
        self.q_attn = up(c.q_attn)
        self.kv8 = s.kv_dtype == "fp8"
        self.kv = up(c.kv_codes if self.kv8 else c.kv_cache)
        self.kv_scale = up(c.kv_scale) if self.kv8 else None
        self.fp8 = s.idx_dtype == "fp8"
        self.mx = s.idx_dtype == "mxfp8"

    def indexer(self, **kw) -> torch.Tensor:
        s = self.c.spec
        if not kw:
            g_out = Guarded((s.B, s.T, s.K), torch.int32)
            lay = dsa.make_layout(self.bt, self.sl, self.c.num_pages, s.max_len)
            dt = dsa.DSA_MXFP8_E4M3 if self.mx else (dsa.DSA_FP8_E4M3 if self.fp8 else dsa.DSA_BF16)
            need = dsa.dsa_indexer_workspace_size(lay, dsa.IndexerShape(s.T, s.HI, s.DI, s.K, dt))
            g_ws = Guarded(None, torch.uint8, nbytes=need)
            r = self.indexer(idx_out=g_out.t, workspace=g_ws.t)
            check_guards(("idx_out", g_out), ("indexer workspace", g_ws))
            return r
        return dsa.dsa_indexer_topk(self.q_idx, self.q_scale, self.w, self.k, self.k_scale, self.bt,
                                    self.sl, T=s.T, top_k=s.K, max_seq_len=s.max_len, fp8=self.fp8,
                                    mx=self.mx, num_pages=self.c.num_pages, **kw)

    def attn(self, idx, **kw):
        s = self.c.spec
        if isinstance(idx, np.ndarray):
            idx = up(idx.astype(np.int32))
        if not kw:
            g_o = Guarded((s.B, s.T, s.H, 512), torch.bfloat16)
            g_l = Guarded((s.B, s.T, s.H), torch.float32)
            lay = dsa.make_layout(self.bt, self.sl, self.c.num_pages, s.max_len)
            need = dsa.dsa_sparse_attn_workspace_size(lay, dsa.AttnShape(s.T, s.H, 576, 512, idx.shape[-1],
                                                                         float(s.sm_scale)))
            g_ws = Guarded(None, torch.uint8, nbytes=need)
            r = self.attn(idx, out=g_o.t, lse=g_l.t, workspace=g_ws.t)
            check_guards(("out", g_o), ("lse", g_l), ("attention workspace", g_ws))
            return r
        if self.kv8:
            return dsa.dsa_sparse_attn_fp8kv(self.q_attn, self.kv, self.kv_scale, idx, self.bt, self.sl,
                                             sm_scale=s.sm_scale, max_seq_len=s.max_len,
                                             num_pages=self.c.num_pages, **kw)
        return dsa.dsa_sparse_attn(self.q_attn, self.kv, idx, self.bt, self.sl, sm_scale=s.sm_scale,
                                   max_seq_len=s.max_len, num_pages=self.c.num_pages, **kw)

    def attn_bf16(self, idx, kv16, **kw):
        """The bf16-cache call over another cache of the same geometry (kv16 [P,64,576] bf16)."""
        s = self.c.spec
        return dsa.dsa_sparse_attn(self.q_attn, kv16, idx, self.bt, self.sl, sm_scale=s.sm_scale,
                                   max_seq_len=s.max_len, num_pages=self.c.num_pages, **kw)


def attn_ref(c, idx, rows=None):
    """The oracle's attention for case c (bf16 or fp8 latent cache) on indices idx."""
    s = c.spec
    if s.kv_dtype == "fp8":
        return oracle.sparse_attn_fp8kv_ref(c.q_attn, c.kv_codes, c.kv_scale, c.block_table, c.seq_lens,
                                            idx, s.sm_scale, rows=rows)
    return oracle.sparse_attn_ref(c.q_attn, c.kv_cache, c.block_table, c.seq_lens, idx, s.sm_scale,
                                  rows=rows)


def oracle_args(c):
    return dict(q_idx=c.q_idx, q_scale=c.q_scale, w=c.w, k_cache=c.k_cache, k_scale=c.k_scale,
                block_table=c.block_table, seq_lens=c.seq_lens)


def check_indices_band(got: np.ndarray, ref: np.ndarray, extra: dict, K: int, seq_lens, T: int,
                       rows=None) -> int:
    """Near-tie gate for Gaussian cases; returns the number of band swaps."""
    swaps = 0
    B = got.shape[0]
    rows = rows if rows is not None else [(b, t) for b in range(B) for t in range(T)]
    for b, t in rows:
        n = int(seq_lens[b]) - T + t + 1
        g = got[b, t]
        if n <= K:
            assert np.array_equal(g, np.r_[np.arange(n), -np.ones(K - n)].astype(np.int32)), (b, t)
            continue
        sc, theta = extra[(b, t)]
        assert np.all(g >= 0) and np.all(g < n), f"row ({b},{t}): positions outside [0, {n})"
        assert np.all(np.diff(g) > 0), f"row ({b},{t}): not strictly ascending"
        tau = max(1e-3 * abs(theta), 1e-6 * float(np.abs(sc).max()))
        must = np.nonzero(sc > theta + tau)[0]
        never = sc < theta - tau
        gs = set(g.tolist())
        assert set(must.tolist()) <= gs, f"row ({b},{t}): missing clear winners"
        assert not never[g].any(), f"row ({b},{t}): selected a clear loser"
        swaps += len(gs.symmetric_difference(set(ref[b, t].tolist()))) // 2
    return swaps


def check_attn(o: np.ndarray, lse: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray, rows=None):
    if rows is not None:
        bi = np.array([r[0] for r in rows]); ti = np.array([r[1] for r in rows])
        o, lse, o_ref, lse_ref = o[bi, ti], lse[bi, ti], o_ref[bi, ti], lse_ref[bi, ti]
    assert np.isfinite(o).all(), "non-finite attention output"
    err = np.abs(o - o_ref)
    assert np.all(err <= 2e-2 + 2e-2 * np.abs(o_ref)), f"G1 max err {err.max()}"
    scale = np.abs(o_ref).max(axis=-1, keepdims=True)
    assert np.all(err.max(axis=-1, keepdims=True) <= 2e-2 * scale + 1e-30), \
        f"G2 worst ratio {(err.max(-1) / np.maximum(scale[..., 0], 1e-30)).max()}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.all(np.abs(lse[fin] - lse_ref[fin]) <= 1e-3 * np.maximum(1.0, np.abs(lse_ref[fin]))), \
        f"G3 max err {np.abs(lse[fin] - lse_ref[fin]).max()}"


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()
