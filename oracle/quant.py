"""MXFP8 quantisation of key and query rows, by definition (test infrastructure only).

Follows the indexer's quantised storage ([P1] §4: the Lightning Indexer's Q and K in MXFP8; [P1] §3
and [P3] §3.3: the indexer prolog writes the new keys into the cache), with MXFP8 as the OCP
Microscaling format defines it.  Each run of 32 consecutive elements V_0..V_31 of a row:
  * shared exponent s = floor(log2(max_i |V_i|)) - 8 (8 = the largest E4M3 exponent), clamped to
    [-127, 127]; a run of zeros takes s = -127;
  * scale byte e = s + 127 (E8M0: value 2^(e - 127));
  * element codes: V_i / 2^s rounded to the nearest E4M3 value, ties to even, magnitudes above 448
    clamped to 448; the sign of a result that rounds to zero is the sign of V_i.
Finite inputs only.  Arithmetic in float64 (every step is exact there: the inputs are bf16).

FP8 latent rows ([P1] §4: the SFA cache in FP8 with per-token scales over tiles of 128; reading of
how the prolog fills it): per token and per 128-column tile of the 576-wide row (columns 0-127,
..., 384-511, 512-575), scale = amax / 448 in float32 (1 for an all-zero tile), element code =
E4M3 of float32(x / scale) (nearest even, clamped to +-448).  Both divisions are single float32
operations, rounded to nearest even.

Per-head fp8 queries ([P1] §3: the prolog quantises the indexer q and folds the head weights in;
reading): per query row and head, sq = amax / 448 in float32 (1 for an all-zero head), code = E4M3
of float32(q / sq); the indexer then weights head h by w[t, h] * sq[t, h].

Per-page fp8 indexer-K cache append ([P1] §3: the prolog writes the new keys into the cache; the
fp8 indexer keeps one float32 scale per 64-token page; reading).  The pages fix no rule for a page
that fills over several steps; the reading taken: a page's scale only grows, and equals the
largest |key| the page has received, divided by 448.  For every page that receives new keys:
  * m = max |new key element| landing in the page; candidate = float32(m / 448);
  * s_old = the stored scale if the page already holds keys of this sequence (positions before
    seq_len - T), else 0; s = max(s_old, candidate), and 1 if that is 0 (a page of zeros);
  * if the page holds keys and s > s_old, each held code c is re-encoded:
    E4M3(float32(float32(e4m3(c) * s_old) / s)) (a second rounding of those keys);
  * new codes are E4M3(float32(x / s)); the page's scale becomes s.
A page filled by one call gets exactly the one-shot rule of the fp8 workloads (scale = amax / 448
of the page's keys).  E4M3 rounding is nearest even, clamped to +-448, throughout.
"""
import numpy as np

from .codecs import e4m3_table

MX_GROUP = 32
E4M3_MAX = 448.0


def _e4m3_rne(x: np.ndarray) -> np.ndarray:
    """E4M3FN codes of float64 values: round to nearest (ties to even), clamp to +-448."""
    a = np.abs(x)
    # spacing of the representable values around |x|: 2^(E - 3) for normal E >= -6, 2^-9 below
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.ldexp(1.0, (np.maximum(e, -6) - 3).astype(np.int64))
    q = np.round(a / step) * step            # numpy rounds halves to even
    q = np.minimum(q, E4M3_MAX)
    # code of each magnitude from the format's own value table (positive codes 0x00..0x7E)
    tab = e4m3_table()[:0x7F]
    idx = np.searchsorted(tab, q)
    assert np.array_equal(tab[idx], q), "rounded value not representable"
    neg = np.signbit(x)
    return (idx + np.where(neg, 0x80, 0)).astype(np.uint8)


def mxfp8_quantize_rows(v: np.ndarray):
    """v [..., D] (D a multiple of 32), finite -> (codes uint8 [..., D], scale bytes uint8 [..., D/32])."""
    v = np.asarray(v, dtype=np.float64)
    g = v.reshape(*v.shape[:-1], v.shape[-1] // MX_GROUP, MX_GROUP)
    amax = np.abs(g).max(axis=-1)
    s = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
    s = np.clip(s, -127, 127).astype(np.int64)
    codes = _e4m3_rne(g / np.ldexp(1.0, s)[..., None]).reshape(v.shape)
    return codes, (s + 127).astype(np.uint8)


def cache_append_ref(k_new, k_cache, k_scale, block_table, seq_lens, T):
    """The paged MXFP8 K cache after appending k_new [B, T, D] (already decoded to float):
    token t of sequence b is logical position seq_lens[b] - T + t, stored at page
    block_table[b, pos // 64], slot pos % 64.  Returns new (k_cache, k_scale) copies."""
    kc, ks = k_cache.copy(), k_scale.copy()
    codes, sc = mxfp8_quantize_rows(k_new)
    B = k_new.shape[0]
    for b in range(B):
        for t in range(T):
            pos = int(seq_lens[b]) - T + t
            p, slot = int(block_table[b, pos // 64]), pos % 64
            kc[p, slot] = codes[b, t]
            ks[p, slot] = sc[b, t]
    return kc, ks


KV_TILE = 128


def latent_fp8_quantize_rows(x):
    """x [..., 576] finite (bf16 values) -> (codes uint8 [..., 576], scales float32 [..., 8]; entries
    5-7 = 1)."""
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    codes = np.empty(x.shape, np.uint8)
    scales = np.ones(x.shape[:-1] + (8,), np.float32)
    for i in range((D + KV_TILE - 1) // KV_TILE):
        t = x[..., KV_TILE * i:KV_TILE * (i + 1)]
        amax = np.abs(t).max(axis=-1)
        sc = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[..., i] = sc
        y = (t / sc[..., None]).astype(np.float32)          # float32 division, nearest even
        codes[..., KV_TILE * i:KV_TILE * (i + 1)] = _e4m3_rne(y.astype(np.float64))
    return codes, scales


def latent_cache_append_fp8_ref(kv_new, kv_codes, kv_scale, block_table, seq_lens, T):
    """The FP8 latent cache after appending kv_new [B, T, 576] (bf16 values as float): token t of
    sequence b goes to logical position seq_lens[b] - T + t.  Returns new (codes, scales) copies."""
    kc, ks = kv_codes.copy(), kv_scale.copy()
    codes, sc = latent_fp8_quantize_rows(kv_new)
    for b in range(kv_new.shape[0]):
        for t in range(T):
            pos = int(seq_lens[b]) - T + t
            p, slot = int(block_table[b, pos // 64]), pos % 64
            kc[p, slot] = codes[b, t]
            ks[p, slot] = sc[b, t]
    return kc, ks


def fp8_quantize_heads(x):
    """x [..., d] finite (one head row per leading index) -> (codes uint8 [..., d], scales float32
    [...]): per row sq = amax / 448 (1 for zeros), code = E4M3 of float32(x / sq)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    sq = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / sq[..., None]).astype(np.float32)
    return _e4m3_rne(y.astype(np.float64)), sq


def indexer_cache_append_fp8_ref(k_new, k_cache, k_scale, block_table, seq_lens, T):
    """The per-page fp8 indexer-K cache after appending k_new [B, T, D] (bf16 values as float):
    k_cache [P, 64, D] E4M3 codes, k_scale [P] float32, one scale per page.  Token t of sequence b
    is logical position seq_lens[b] - T + t (page block_table[b, pos // 64], slot pos % 64).
    Returns new (k_cache, k_scale) copies; codes of held keys must be finite."""
    kc, ks = k_cache.copy(), np.asarray(k_scale, np.float32).copy()
    x = np.asarray(k_new, np.float32)
    f32 = np.float32
    for b in range(x.shape[0]):
        L = int(seq_lens[b])
        first = L - T                                    # position of the first new key
        for j in range(first // 64, (L - 1) // 64 + 1):
            page = int(block_table[b, j])
            lo, hi = max(first, 64 * j), min(L, 64 * j + 64)
            held = lo - 64 * j                           # slots 0..held-1 already hold keys
            new = x[b, lo - first:hi - first]
            cand = f32(f32(np.abs(new).max()) / f32(E4M3_MAX))
            s_old = ks[page] if held > 0 else f32(0.0)
            s = max(s_old, cand)
            if s == 0:
                s = f32(1.0)
            if held > 0 and s > s_old:
                dec = (e4m3_table()[kc[page, :held]].astype(f32) * s_old).astype(f32)
                kc[page, :held] = _e4m3_rne((dec / s).astype(f32).astype(np.float64))
            kc[page, held:held + hi - lo] = _e4m3_rne((new / s).astype(f32).astype(np.float64))
            ks[page] = s
    return kc, ks
