"""Seeded synthetic inputs for the DSA Lightning-Indexer + Sparse-Flash-Attention path.

This module is shared by the tests, the benchmark and the CPU oracle's callers.  It holds none of
the method's arithmetic: it draws random numbers, rounds them to the storage formats (bf16 by
round-to-nearest-even, OCP E4M3FN codes through torch's float8 cast) and lays them out in paged
caches addressed through a block table.  Nothing here scores, selects or attends.

Workload shapes follow the long-context decode, speculative-verify and prefill workloads that the
pages discuss ("Inference Optimization for Kimi K3.1 Pro: Decoding Architecture Evolution and
Systems Engineering Practices", §2 and §5.3; "Optimizing Kimi K3.1 Pro Sparse Attention Inference",
"Interleaved KDA and DSA Modules"); the exact sizes are this library's five named workloads below.

Storage conventions (every array is a numpy array in host memory):
  * bf16 tensors are np.uint16 bit patterns; e4m3 tensors are np.uint8 codes.
  * Paged caches are [num_pages, PAGE, dim]; logical token s of sequence b lives in physical page
    block_table[b, s // PAGE], slot s % PAGE.  Physical page ids are a seeded random permutation.
  * Slots past a sequence's length and the spare pages are poisoned with NaN codes
    (bf16 0x7FC0, e4m3 0x7F) so a kernel that reads outside the valid range shows NaN.
  * Unused block-table entries point at a poisoned spare page (never at an invalid page id).
  * An FP8 latent cache (kv_dtype "fp8") quantises the bf16 latent rows per token and 128-column
    tile: scale amax / 448 (fp32), codes through torch's E4M3 cast; poisoned slots get NaN codes
    and NaN scales.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

PAGE = 64
DQK = 576          # MLA latent row: 512 "nope" + 64 rope
DV = 512           # V = first 512 columns of the latent row
BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
E8M0_NAN = np.uint8(0xFF)   # NaN scale byte
MX_GROUP = 32               # elements per MX shared scale
E4M3_MAX = 448.0
_SEED_ROOT = 15
_CHUNK = 1 << 22   # elements per independently seeded generation chunk


@dataclasses.dataclass(frozen=True)
class CaseSpec:
    """Everything that defines one synthetic case."""
    name: str
    cfg_id: int
    B: int
    T: int
    lens: tuple            # per-sequence cache length (tokens, including the T query tokens)
    HI: int                # indexer heads
    DI: int                # indexer head dim
    K: int                 # top-k
    H: int                 # attention heads
    idx_dtype: str = "bf16"   # "bf16" | "fp8" | "mxfp8"
    kv_dtype: str = "bf16"    # latent cache: "bf16" | "fp8" (E4M3 + fp32 scale per token and 128-column tile)
    values: str = "gauss"     # "gauss" | "grid" | "grid8" | "ties" | "ties2" | "narrow" | "fp8grid" | "mxgrid" | "sharp"
    sharp_c: float = 1.0
    variant: int = 0
    spare_pages: int = 1
    sm_scale: float = 1.0 / 24.0   # 1/sqrt(576)

    @property
    def max_len(self) -> int:
        return int(max(self.lens))

    @property
    def max_pages(self) -> int:
        return (self.max_len + PAGE - 1) // PAGE

    @property
    def rows(self) -> int:
        return self.B * self.T


@dataclasses.dataclass
class Case:
    spec: CaseSpec
    seq_lens: np.ndarray      # [B] int32
    block_table: np.ndarray   # [B, max_pages] int32
    num_pages: int
    q_idx: np.ndarray         # [B,T,HI,DI] uint16 (bf16) | uint8 (e4m3)
    q_scale: np.ndarray | None  # [B,T,HI] f32 (fp8) | [B,T,HI,DI/32] uint8 E8M0 (mxfp8)
    w: np.ndarray             # [B,T,HI] f32
    k_cache: np.ndarray       # [P,PAGE,DI] uint16 | uint8
    k_scale: np.ndarray | None  # [P] f32 (fp8) | [P,PAGE,DI/32] uint8 E8M0 (mxfp8)
    q_attn: np.ndarray        # [B,T,H,DQK] uint16
    kv_cache: np.ndarray      # [P,PAGE,DQK] uint16
    kv_codes: np.ndarray | None = None   # fp8 latent cache: [P,PAGE,DQK] uint8 E4M3
    kv_scale: np.ndarray | None = None   # fp8 latent cache: [P,PAGE,8] float32 (5 tile scales used)


# ----------------------------------------------------------------------------- named workloads
def _ragged(cfg_id: int, variant: int, B: int, lo: int, hi: int) -> tuple:
    rng = np.random.default_rng([_SEED_ROOT, cfg_id, variant, 0])
    return tuple(int(x) for x in rng.integers(lo, hi, size=B, endpoint=True))


def config(cfg_id: int, size: str = "full", variant: int = 0) -> CaseSpec:
    """The five named workloads.  size="full" is the real shape; "small" keeps every structural
    feature (paging, raggedness, multi-query, causal, fp8) at a size the CPU oracle finishes in
    seconds, still spanning several kernel tiles and a ragged tail."""
    full = size == "full"
    if cfg_id == 1:   # decode, integer grid, exact fp32 scores
        return CaseSpec("cfg1_decode_L4096_grid", 1, 1, 1, (4096,), 8, 64, 256, 16,
                        values="grid", variant=variant)
    if cfg_id == 2:   # decode, batch 32, ragged 8k..32k
        if full:
            return CaseSpec("cfg2_decode_B32_L8k-32k", 2, 32, 1, _ragged(2, variant, 32, 8192, 32768),
                            64, 128, 2048, 128, variant=variant)
        return CaseSpec("cfg2s_decode_B3_ragged", 2, 3, 1, _ragged(2, variant + 100, 3, 2100, 5000),
                        64, 128, 2048, 128, variant=variant)
    if cfg_id == 3:   # causal prefill chunk over its own context
        L = 8192 if full else 2304
        return CaseSpec(f"cfg3{'' if full else 's'}_prefill_T{L}", 3, 1, L, (L,), 64, 128, 2048, 128,
                        variant=variant)
    if cfg_id == 4:   # long-context decode, fp8 indexer
        if full:
            return CaseSpec("cfg4_decode_B8_L131072_fp8", 4, 8, 1, (131072,) * 8, 64, 128, 2048, 128,
                            idx_dtype="fp8", variant=variant)
        return CaseSpec("cfg4s_decode_B2_fp8", 4, 2, 1, (3000, 4545), 64, 128, 2048, 128,
                        idx_dtype="fp8", variant=variant)
    if cfg_id == 6:   # long-context decode, MXFP8 indexer (the fp8 workload's shape)
        if full:
            return CaseSpec("mx_decode_B8_L131072_mxfp8", 6, 8, 1, (131072,) * 8, 64, 128, 2048, 128,
                            idx_dtype="mxfp8", variant=variant)
        return CaseSpec("mxs_decode_B2_mxfp8", 6, 2, 1, (3000, 4545), 64, 128, 2048, 128,
                        idx_dtype="mxfp8", variant=variant)
    if cfg_id == 7:   # causal prefill chunk, MXFP8 indexer (workload 3's shape)
        L = 8192 if full else 1100
        return CaseSpec(f"mx_prefill{'' if full else 's'}_T{L}_mxfp8", 7, 1, L, (L,), 64, 128, 2048, 128,
                        idx_dtype="mxfp8", variant=variant)
    if cfg_id == 8:   # speculative verify, MXFP8 indexer (workload 5's shape)
        if full:
            return CaseSpec("mx_verify_B16_T4_L65536_mxfp8", 8, 16, 4, (65536,) * 16, 64, 128, 2048, 128,
                            idx_dtype="mxfp8", variant=variant)
        return CaseSpec("mxs_verify_B2_T4_mxfp8", 8, 2, 4, (2500, 4100), 64, 128, 2048, 128,
                        idx_dtype="mxfp8", variant=variant)
    if cfg_id == 9:   # workload 2 with an FP8 latent cache
        if full:
            return CaseSpec("kv8_decode_B32_L8k-32k", 9, 32, 1, _ragged(2, variant, 32, 8192, 32768),
                            64, 128, 2048, 128, kv_dtype="fp8", variant=variant)
        return CaseSpec("kv8s_decode_B3_ragged", 9, 3, 1, _ragged(2, variant + 100, 3, 2100, 5000),
                        64, 128, 2048, 128, kv_dtype="fp8", variant=variant)
    if cfg_id == 5:   # speculative verify: 4 causal drafts per sequence
        if full:
            return CaseSpec("cfg5_verify_B16_T4_L65536", 5, 16, 4, (65536,) * 16, 64, 128, 2048, 128,
                            variant=variant)
        return CaseSpec("cfg5s_verify_B2_T4", 5, 2, 4, (2500, 4100), 64, 128, 2048, 128,
                        variant=variant)
    raise ValueError(f"unknown workload {cfg_id}")


# ----------------------------------------------------------------------------- storage rounding
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


KV_TILE = 128


def bf16_rows_to_fp8_tiles(rows_bits: np.ndarray) -> tuple:
    """Latent rows [..., 576] (bf16 bits) to an FP8 cache: per row and per 128-column tile
    (columns 0-127, ..., 384-511, 512-575) the fp32 scale amax / 448 (1 for an all-zero tile) and
    E4M3 codes of x / scale (torch's cast: nearest even).  Returns (codes uint8 [..., 576],
    scales float32 [..., 8], entries 5-7 = 1)."""
    import torch
    x = torch.from_numpy((rows_bits.astype(np.uint32) << 16).view(np.float32))
    D = x.shape[-1]
    nt = (D + KV_TILE - 1) // KV_TILE
    sc = torch.ones(x.shape[:-1] + (8,), dtype=torch.float32)
    codes = torch.empty(x.shape, dtype=torch.uint8)
    for i in range(nt):
        t = x[..., KV_TILE * i:KV_TILE * (i + 1)]
        amax = t.abs().amax(dim=-1)
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        sc[..., i] = s
        y = (t / s.unsqueeze(-1)).clamp(-448.0, 448.0)
        codes[..., KV_TILE * i:KV_TILE * (i + 1)] = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.numpy(), sc.numpy()


def f32_to_mxfp8(x: np.ndarray) -> tuple:
    """Quantise the last axis (a multiple of 32) to MXFP8 as the OCP Microscaling format defines it:
    each run of 32 elements shares the E8M0 exponent floor(log2(amax)) - 8 (8 = the largest E4M3
    exponent), clamped to the E8M0 range; elements are x / scale rounded to E4M3 (RNE, saturated).
    Returns (codes uint8, scale bytes uint8 with the last axis divided by 32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    g = x.reshape(*x.shape[:-1], x.shape[-1] // MX_GROUP, MX_GROUP)
    amax = np.abs(g).max(axis=-1)
    e = np.where(amax > 0, np.floor(np.log2(np.maximum(amax, 1e-38))) - 8, -127)
    e = np.clip(e, -127, 127).astype(np.int64)
    scaled = (g.astype(np.float64) / np.ldexp(1.0, e)[..., None]).astype(np.float32)
    codes = f32_to_e4m3_codes(scaled).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8)


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 to OCP E4M3FN codes (RNE, saturated to +-448) through torch's float8 cast."""
    import torch
    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


# ----------------------------------------------------------------------------- random draws
def _normal_f32(key: list, n: int, scale: float) -> np.ndarray:
    """n float32 normals * scale, drawn in fixed-size independently seeded chunks (thread-count
    independent, so the same key always yields the same values)."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        rng = np.random.default_rng(key + [c])
        v = rng.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            v *= np.float32(scale)
        out[lo:hi] = v

    threads = min(nchunks, max(1, min(16, len(os.sched_getaffinity(0)))))
    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(work, range(nchunks)))
    else:
        for c in range(nchunks):
            work(c)
    return out


def _gauss_bf16(key: list, shape: tuple, scale: float) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 26
    for i, lo in enumerate(range(0, n, step)):
        hi = min(n, lo + step)
        out[lo:hi] = f32_to_bf16_bits(_normal_f32(key + [i], hi - lo, scale))
    return out.reshape(shape)


def _grid_bf16(rng: np.random.Generator, shape: tuple, lo: int = -16, hi: int = 16) -> np.ndarray:
    vals = rng.integers(lo, hi, size=shape, endpoint=True).astype(np.float32) / np.float32(16.0)
    return f32_to_bf16_bits(vals)


# ----------------------------------------------------------------------------- builder
def make_case(spec: CaseSpec, poison: bool = True) -> Case:
    B, T, HI, DI, H = spec.B, spec.T, spec.HI, spec.DI, spec.H
    lens = np.asarray(spec.lens, dtype=np.int64)
    if len(lens) != B or (lens < T).any():
        raise ValueError("need one length per sequence, each >= T")
    key0 = [_SEED_ROOT, spec.cfg_id, spec.variant]

    # paging: pages used + spare, physical ids are a random permutation of the pool
    pages_per = (lens + PAGE - 1) // PAGE
    used = int(pages_per.sum())
    P = used + spec.spare_pages
    perm = np.random.default_rng(key0 + [1]).permutation(P).astype(np.int32)
    spare = perm[used:]
    bt = np.full((B, spec.max_pages), spare[0], dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :pages_per[b]] = perm[off:off + pages_per[b]]
        off += pages_per[b]
    # mask of valid (page, slot) cells in physical order
    valid = np.zeros((P, PAGE), dtype=bool)
    for b in range(B):
        L = int(lens[b])
        for j in range(int(pages_per[b])):
            valid[bt[b, j], :min(PAGE, L - j * PAGE)] = True

    rngq = np.random.default_rng(key0 + [2])
    rngk = np.random.default_rng(key0 + [3])
    rngw = np.random.default_rng(key0 + [4])
    rngs = np.random.default_rng(key0 + [5])
    rngv = np.random.default_rng(key0 + [6])
    q_scale = k_scale = None
    v = spec.values

    # ---- indexer q / k / w
    if spec.idx_dtype == "bf16":
        if v in ("grid", "grid8", "ties", "ties2", "narrow"):
            # grid: multiples of 1/16 in [-1, 1]; grid8: in [-1/2, 1/2], which keeps the wide
            # (64 heads x 128 dims) scores below 2^11 so fp32 sums are exact in any order
            lim = 16 if v == "grid" else 8
            q_idx = _grid_bf16(rngq, (B, T, HI, DI), -lim, lim)
            if v in ("ties", "ties2"):
                # few distinct key rows copied to many positions: many exact score ties
                nd = 7 if v == "ties" else 2
                base = _grid_bf16(rngk, (nd, DI), -lim, lim)
                k_cache = base[rngk.integers(0, nd, size=(P, PAGE))]
            else:
                k_cache = _grid_bf16(rngk, (P, PAGE, DI), -lim, lim)
            if v == "narrow":
                # every q and k row is 1/2 in all but the last dim: all scores sit in a narrow
                # band (one coarse histogram bin) with a few exact values, each tied many times
                half = f32_to_bf16_bits(np.float32(0.5))
                q_idx[..., :-1] = half
                k_cache[..., :-1] = half
            w = (rngw.integers(0, 16, size=(B, T, HI), endpoint=True) / 16.0).astype(np.float32)
        else:
            q_idx = _gauss_bf16(key0 + [2], (B, T, HI, DI), 1.0 / np.sqrt(DI))
            k_cache = _gauss_bf16(key0 + [3], (P, PAGE, DI), 1.0 / np.sqrt(DI))
            w = _normal_f32(key0 + [4], B * T * HI, 1.0 / np.sqrt(64.0)).reshape(B, T, HI)
        if poison:
            k_cache = k_cache.copy()
            k_cache[~valid] = BF16_NAN
    elif spec.idx_dtype == "fp8":
        if v == "fp8grid":
            # integer codes in [-4, 4] (exact in e4m3) with power-of-two scales, q scales <= 1:
            # every fp32 partial sum of the score is exact in any order
            q_idx = f32_to_e4m3_codes(rngq.integers(-4, 4, size=(B, T, HI, DI), endpoint=True))
            k_cache = f32_to_e4m3_codes(rngk.integers(-4, 4, size=(P, PAGE, DI), endpoint=True))
            q_scale = (2.0 ** rngq.integers(-3, 0, size=(B, T, HI), endpoint=True)).astype(np.float32)
            k_scale = (2.0 ** rngk.integers(-3, 3, size=P, endpoint=True)).astype(np.float32)
            w = (rngw.integers(0, 16, size=(B, T, HI), endpoint=True) / 16.0).astype(np.float32)
        else:
            qf = _normal_f32(key0 + [2], B * T * HI * DI, 1.0 / np.sqrt(DI)).reshape(B, T, HI, DI)
            amax = np.abs(qf).max(axis=-1)
            q_scale = (np.maximum(amax, 1e-30) / E4M3_MAX).astype(np.float32)
            q_idx = f32_to_e4m3_codes(qf / q_scale[..., None])
            kf = _normal_f32(key0 + [3], P * PAGE * DI, 1.0 / np.sqrt(DI)).reshape(P, PAGE, DI)
            kf[~valid] = 0.0
            amax = np.abs(kf).max(axis=(1, 2))
            k_scale = (np.maximum(amax, 1e-30) / E4M3_MAX).astype(np.float32)
            k_scale[amax == 0] = 1.0
            k_cache = f32_to_e4m3_codes(kf / k_scale[:, None, None])
            w = _normal_f32(key0 + [4], B * T * HI, 1.0 / np.sqrt(64.0)).reshape(B, T, HI)
        if poison:
            k_cache = k_cache.copy()
            k_cache[~valid] = E4M3_NAN
    elif spec.idx_dtype == "mxfp8":
        if DI % MX_GROUP:
            raise ValueError("MXFP8 rows need a multiple of 32 elements")
        G = DI // MX_GROUP
        if v == "mxgrid":
            # integer codes in [-2, 2] (exact in e4m3), q scales 2^-2..2^0, k scales 2^-1..2^1,
            # w multiples of 1/16 in [0, 1]: every fp32 partial sum of a 64 x 128 score is a
            # multiple of 2^-7 below 2^16, so exact in any order
            q_idx = f32_to_e4m3_codes(rngq.integers(-2, 2, size=(B, T, HI, DI), endpoint=True))
            k_cache = f32_to_e4m3_codes(rngk.integers(-2, 2, size=(P, PAGE, DI), endpoint=True))
            q_scale = (127 + rngq.integers(-2, 0, size=(B, T, HI, G), endpoint=True)).astype(np.uint8)
            k_scale = (127 + rngk.integers(-1, 1, size=(P, PAGE, G), endpoint=True)).astype(np.uint8)
            w = (rngw.integers(0, 16, size=(B, T, HI), endpoint=True) / 16.0).astype(np.float32)
        else:
            qf = _normal_f32(key0 + [2], B * T * HI * DI, 1.0 / np.sqrt(DI)).reshape(B, T, HI, DI)
            q_idx, q_scale = f32_to_mxfp8(qf)
            kf = _normal_f32(key0 + [3], P * PAGE * DI, 1.0 / np.sqrt(DI)).reshape(P, PAGE, DI)
            k_cache, k_scale = f32_to_mxfp8(kf)
            w = _normal_f32(key0 + [4], B * T * HI, 1.0 / np.sqrt(64.0)).reshape(B, T, HI)
        if poison:
            k_cache = k_cache.copy()
            k_cache[~valid] = E4M3_NAN
            k_scale = k_scale.copy()
            k_scale[~valid] = E8M0_NAN
    else:
        raise ValueError(spec.idx_dtype)

    # ---- attention q / kv
    if v in ("grid", "grid8", "ties", "ties2", "narrow", "fp8grid", "mxgrid"):
        q_attn = _grid_bf16(rngs, (B, T, H, DQK))
        kv_cache = _grid_bf16(rngv, (P, PAGE, DQK))
    elif v == "sharp":
        q_attn = _gauss_bf16(key0 + [5], (B, T, H, DQK), spec.sharp_c)
        kv_cache = _gauss_bf16(key0 + [6], (P, PAGE, DQK), 1.0)
    else:
        q_attn = _gauss_bf16(key0 + [5], (B, T, H, DQK), 1.0 / np.sqrt(DQK))
        kv_cache = _gauss_bf16(key0 + [6], (P, PAGE, DQK), 1.0 / np.sqrt(DQK))
    kv_codes = kv_scale = None
    if spec.kv_dtype == "fp8":
        kv_codes, kv_scale = bf16_rows_to_fp8_tiles(kv_cache)
    elif spec.kv_dtype != "bf16":
        raise ValueError(spec.kv_dtype)
    if poison:
        kv_cache[~valid] = BF16_NAN
        if kv_codes is not None:
            kv_codes[~valid] = E4M3_NAN
            kv_scale[~valid] = np.nan

    return Case(spec=spec, seq_lens=lens.astype(np.int32), block_table=bt, num_pages=P,
                q_idx=np.ascontiguousarray(q_idx), q_scale=q_scale, w=np.ascontiguousarray(w, np.float32),
                k_cache=np.ascontiguousarray(k_cache), k_scale=k_scale,
                q_attn=np.ascontiguousarray(q_attn), kv_cache=np.ascontiguousarray(kv_cache),
                kv_codes=kv_codes, kv_scale=kv_scale)


def custom(name: str, B: int, T: int, lens, HI: int, DI: int, K: int, H: int, **kw) -> CaseSpec:
    """A free-form case (edge cases in tests); cfg_id 0 keeps its seeds apart from the named ones."""
    return CaseSpec(name, kw.pop("cfg_id", 0), B, T, tuple(int(x) for x in lens), HI, DI, K, H, **kw)


def permute_pages(case: Case, seed: int = 99) -> Case:
    """Same logical contents, different physical page placement (for invariance tests)."""
    P = case.num_pages
    perm = np.random.default_rng([_SEED_ROOT, 1000, seed]).permutation(P).astype(np.int32)
    # physical page p moves to perm[p]
    def move(a):
        if a is None:
            return None
        out = np.empty_like(a)
        out[perm] = a
        return out
    return dataclasses.replace(case, block_table=perm[case.block_table], k_cache=move(case.k_cache),
                               k_scale=move(case.k_scale), kv_cache=move(case.kv_cache),
                               kv_codes=move(case.kv_codes), kv_scale=move(case.kv_scale))
