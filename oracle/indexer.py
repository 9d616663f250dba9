"""Lightning-Indexer scores and Top-K selection, by definition (test infrastructure only).

Follows [P1] §1 (DSA steps 1 and 2), [P1] §2 ("Inlined Top-K Selection": only the selected indices
are output; they address the paged cache) and [P3] §3.1 (relevance scoring, head-weight summation
and Top-K; the paged K cache is read in place).  Readings where the pages are silent:
  * score I[t,s] = sum_h w[t,h] * max(0, q[t,h,:] . k[s,:]); one key vector per position, shared by
    the indexer heads; no softmax or extra scale (any scale is folded into w);
  * fp8 path: q = q_scale[t,h] * e4m3(q_code), k = k_scale[page] * e4m3(k_code);
  * mxfp8 path (MXFP8, [P1] §4, [P3] §3.3): every run of 32 consecutive elements of a q row or
    of a cached key row shares one E8M0 scale: q[t,h,d] = e8m0(q_scale[t,h,d // 32]) *
    e4m3(q_code[t,h,d]) and k[s,d] = e8m0(k_scale[page, slot, d // 32]) * e4m3(k_code[s,d]);
  * queries are the last T positions of their sequence: query t of sequence b sits at
    pos = seq_len[b] - T + t and sees keys 0..pos (its own key included);
  * K' = min(K, pos + 1) positions are kept: the K' largest scores, ties to the lower position;
  * output: those positions in ascending order, then -1 up to K.
Arithmetic is float64 on the decoded inputs; a score of -0 compares equal to +0.
"""
import numpy as np

from .codecs import bf16_bits_to_f64, e4m3_codes_to_f64, e8m0_to_f64

PAGE = 64


def visible_positions(seq_len: int, T: int, t: int) -> int:
    """Number of keys query t sees (its position + 1)."""
    return int(seq_len) - int(T) + int(t) + 1


MX_GROUP = 32   # elements per shared scale in the MX formats


def _decode(x, dtype):
    return bf16_bits_to_f64(x) if dtype == "bf16" else e4m3_codes_to_f64(x)


def _mx_scales(scale_bytes, dim):
    """Per-element scale of MX rows: each E8M0 byte covers MX_GROUP consecutive elements."""
    return np.repeat(e8m0_to_f64(scale_bytes), MX_GROUP, axis=-1)[..., :dim]


def _keys_of_sequence(k_cache, k_scale, block_table, b, n, dtype):
    """Logical key rows 0..n-1 of sequence b, resolved through the block table ([P1] §2: indices
    resolve to page slots on demand)."""
    s = np.arange(n)
    pages = block_table[b, s // PAGE]
    k = _decode(k_cache[pages, s % PAGE], dtype)
    if dtype == "fp8":
        k = k * k_scale[pages].astype(np.float64)[:, None]
    elif dtype == "mxfp8":
        k = k * _mx_scales(k_scale[pages, s % PAGE], k.shape[-1])
    return k


def indexer_scores_ref(q_idx, q_scale, w, k_cache, k_scale, block_table, seq_lens, T, dtype,
                       b, ts):
    """Scores of queries ts (list of t) of sequence b against their visible keys.
    Returns a list of float64 arrays, one per t, of length pos_t + 1."""
    n_max = max(visible_positions(seq_lens[b], T, t) for t in ts)
    k = _keys_of_sequence(k_cache, k_scale, block_table, b, n_max, dtype)       # [n, DI]
    out = []
    for t in ts:
        n = visible_positions(seq_lens[b], T, t)
        q = _decode(q_idx[b, t], dtype)                                          # [HI, DI]
        if dtype == "fp8":
            q = q * q_scale[b, t].astype(np.float64)[:, None]
        elif dtype == "mxfp8":
            q = q * _mx_scales(q_scale[b, t], q.shape[-1])
        dots = q @ k[:n].T                                                       # [HI, n]
        relu = np.maximum(dots, 0.0)
        wt = w[b, t].astype(np.float64)                                          # [HI]
        out.append(wt @ relu)                                                    # [n]
    return out


def select_topk(scores: np.ndarray, K: int) -> np.ndarray:
    """Ascending positions of the min(K, n) largest scores, ties to the lower position; -1 pad."""
    n = scores.shape[0]
    kp = min(K, n)
    order = np.lexsort((np.arange(n), -scores))       # score descending, then position ascending
    sel = np.sort(order[:kp]).astype(np.int32)
    out = np.full(K, -1, dtype=np.int32)
    out[:kp] = sel
    return out


def indexer_topk_ref(q_idx, q_scale, w, k_cache, k_scale, block_table, seq_lens, T, K, dtype,
                     rows=None, return_scores=False, block=64):
    """Indices [B, T, K] (int32).  rows: optional list of (b, t) to compute (others left -1).
    With return_scores, also a dict (b, t) -> (scores float64[n], theta) where theta is the
    K'-th largest score."""
    B = seq_lens.shape[0]
    idx = np.full((B, T, K), -1, dtype=np.int32)
    extra = {}
    if rows is None:
        rows = [(b, t) for b in range(B) for t in range(T)]
    by_seq = {}
    for b, t in rows:
        by_seq.setdefault(int(b), []).append(int(t))
    for b, ts in by_seq.items():
        ts = sorted(set(ts))
        for i in range(0, len(ts), block):
            chunk = ts[i:i + block]
            for t, sc in zip(chunk, indexer_scores_ref(q_idx, q_scale, w, k_cache, k_scale,
                                                       block_table, seq_lens, T, dtype, b, chunk)):
                idx[b, t] = select_topk(sc, K)
                if return_scores:
                    kp = min(K, sc.shape[0])
                    theta = np.sort(sc)[::-1][kp - 1]
                    extra[(b, t)] = (sc, float(theta))
    return (idx, extra) if return_scores else idx
