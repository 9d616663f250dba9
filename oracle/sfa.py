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

FP8 latent cache ([P1] §4: the SFA cache held in FP8 with per-token scales over tiles of 128, the
core products kept in BF16; the dequantised BF16 tile feeds the matrix unit directly).  Readings:
  * one fp32 scale per token and per 128-column tile of the 576-wide row: columns 0-127, 128-255,
    256-383, 384-511 (the value part) and 512-575 (the rope remainder), stored as 8 floats per
    token with entries 5-7 unused;
  * an element is dequantised as e4m3(code) * scale in float32 (round to nearest even), then
    rounded to bf16 (nearest even): the BF16 tile the products read;
  * attention then proceeds exactly as for a bf16 cache holding those rows.
"""
import numpy as np

from .codecs import bf16_bits_to_f64, e4m3_codes_to_f64

PAGE = 64
DV = 512


def sparse_attn_ref(q_attn, kv_cache, block_table, seq_lens, idx, sm_scale, rows=None, rows_of=None):
    """q_attn [B,T,H,576] bf16 bits, kv_cache [P,64,576] bf16 bits, idx [B,T,K] int32.
    Returns (out float64 [B,T,H,512], lse float64 [B,T,H]); rows limits the (b, t) computed
    (others are NaN).  rows_of(pages, slots) -> bf16 bits replaces the cache lookup when given."""
    if rows_of is None:
        rows_of = lambda pg, sl: kv_cache[pg, sl]   # noqa: E731
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
        X = bf16_bits_to_f64(rows_of(block_table[b, sel // PAGE], sel % PAGE))     # [K', 576]
        q = bf16_bits_to_f64(q_attn[b, t])                                         # [H, 576]
        z = sm_scale * (q @ X.T)                                                   # [H, K']
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        l = e.sum(axis=1, keepdims=True)
        out[b, t] = (e @ X[:, :DV]) / l
        lse[b, t] = (m + np.log(l))[:, 0]
    return out, lse


KV_TILE = 128
KV_SCALES = 8          # floats stored per token (5 used)


def f32_to_bf16_rne(x) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), r)


def dequant_kv_fp8(codes, scales) -> np.ndarray:
    """E4M3 latent rows [..., 576] and their tile scales [..., 8] (fp32) -> bf16 bits [..., 576]:
    bf16(float32(e4m3(code) * scale of the column's 128-wide tile))."""
    codes = np.asarray(codes, np.uint8)
    tile = np.minimum(np.arange(codes.shape[-1]) // KV_TILE, 4)
    vals = e4m3_codes_to_f64(codes).astype(np.float32)          # exact: e4m3 values fit float32
    s = np.asarray(scales, np.float32)[..., tile]
    return f32_to_bf16_rne(vals * s)                             # float32 product, then bf16


def sparse_attn_fp8kv_ref(q_attn, kv_codes, kv_scale, block_table, seq_lens, idx, sm_scale, rows=None):
    """sparse_attn_ref over an FP8 latent cache: kv_codes [P,64,576] uint8 (E4M3), kv_scale
    [P,64,8] float32; each selected row is dequantised to bf16 as dequant_kv_fp8 defines."""
    return sparse_attn_ref(q_attn, None, block_table, seq_lens, idx, sm_scale, rows,
                           rows_of=lambda pg, sl: dequant_kv_fp8(kv_codes[pg, sl], kv_scale[pg, sl]))
