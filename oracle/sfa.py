"""Sparse attention over the selected latent rows, by definition (test infrastructure only).

Follows [P1] §1 (DSA step 3: read the KV cache at the indices the indexer selected and attend over
them), [P1] §2 (indices resolve through the paged cache) and [P2] "Inheritance and Extension of
Core Operators" (blockwise attention whose cross-block reduction reproduces the global softmax, so
the definition is the exact softmax).  Readings where the pages are silent:
  * one index set per query token, shared by all attention heads; -1 entries are skipped;
  * each selected row is an MLA latent row of width 576; V is its first 512 columns;
  * z[h,j] = sm_scale * q[h,:] . X[j,:];  o[h] = sum_j softmax(z[h])_j V[j];  lse = log sum_j e^z;
  * an empty selection gives o = 0 and lse = -inf.
Arithmetic is float64 on the decoded bf16 inputs.
"""
import numpy as np

from .codecs import bf16_bits_to_f64

PAGE = 64
DV = 512


def sparse_attn_ref(q_attn, kv_cache, block_table, seq_lens, idx, sm_scale, rows=None):
    """q_attn [B,T,H,576] bf16 bits, kv_cache [P,64,576] bf16 bits, idx [B,T,K] int32.
    Returns (out float64 [B,T,H,512], lse float64 [B,T,H]); rows limits the (b, t) computed
    (others are NaN)."""
    B, T, H, _ = q_attn.shape
    out = np.full((B, T, H, DV), np.nan)
    lse = np.full((B, T, H), np.nan)
    if rows is None:
        rows = [(b, t) for b in range(B) for t in range(T)]
    for b, t in rows:
        sel = idx[b, t]
        sel = sel[sel >= 0].astype(np.int64)
        pos = int(seq_lens[b]) - T + t
        if sel.size and (np.unique(sel).size != sel.size or sel.max() > pos):
            raise ValueError(f"row ({b},{t}): indices must be unique and <= {pos}")
        if sel.size == 0:
            out[b, t] = 0.0
            lse[b, t] = -np.inf
            continue
        X = bf16_bits_to_f64(kv_cache[block_table[b, sel // PAGE], sel % PAGE])   # [K', 576]
        q = bf16_bits_to_f64(q_attn[b, t])                                         # [H, 576]
        z = sm_scale * (q @ X.T)                                                   # [H, K']
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        l = e.sum(axis=1, keepdims=True)
        out[b, t] = (e @ X[:, :DV]) / l
        lse[b, t] = (m + np.log(l))[:, 0]
    return out, lse
