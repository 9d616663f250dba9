"""ctypes binding of libdsa.so (C ABI in include/dsa.h).

Argument marshalling only: torch tensors become device pointers plus sizes, and the current HIP
stream is passed through.  Every step of the computation runs in the HIP kernels behind the C ABI;
nothing here computes.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

DSA_OK = 0
DSA_BF16 = 0
DSA_FP8_E4M3 = 1
DSA_MXFP8_E4M3 = 2
PAGE_SIZE = 64
DIM_QK = 576
DIM_V = 512
_STATUS = {0: "DSA_OK", 1: "DSA_ERR_NULL", 2: "DSA_ERR_SHAPE", 3: "DSA_ERR_ALIGN",
           4: "DSA_ERR_UNSUPPORTED", 5: "DSA_ERR_WORKSPACE", 6: "DSA_ERR_HIP"}


class Layout(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32)]


class IndexerShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("heads", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("dtype", ctypes.c_int)]


class AttnShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("heads", ctypes.c_int32), ("dim_qk", ctypes.c_int32),
                ("dim_v", ctypes.c_int32), ("top_k", ctypes.c_int32), ("sm_scale", ctypes.c_float)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


class DsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None

EXPORTS = ["dsa_indexer_workspace_size", "dsa_indexer_topk", "dsa_sparse_attn_workspace_size",
           "dsa_sparse_attn", "dsa_sparse_attn_noalloc", "dsa_sparse_attn_fp8kv", "dsa_mxfp8_quantize", "dsa_indexer_cache_append", "dsa_indexer_cache_append_fp8", "dsa_latent_cache_append_fp8", "dsa_fp8_quantize_heads", "dsa_profile_start",
           "dsa_profile_stop", "dsa_last_error", "dsa_version", "dsa_debug_status"]


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not found: build it first "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.dsa_indexer_workspace_size.argtypes = [ctypes.POINTER(Layout), ctypes.POINTER(IndexerShape)]
    L.dsa_indexer_workspace_size.restype = sz
    L.dsa_indexer_topk.argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(Layout),
                                   ctypes.POINTER(IndexerShape), vp, vp, sz, vp]
    L.dsa_indexer_topk.restype = ctypes.c_int
    L.dsa_sparse_attn_workspace_size.argtypes = [ctypes.POINTER(Layout), ctypes.POINTER(AttnShape)]
    L.dsa_sparse_attn_workspace_size.restype = sz
    L.dsa_sparse_attn.argtypes = [vp, vp, vp, ctypes.POINTER(Layout), ctypes.POINTER(AttnShape),
                                  vp, vp, vp, sz, vp]
    L.dsa_sparse_attn.restype = ctypes.c_int
    L.dsa_sparse_attn_noalloc.argtypes = [vp, vp, vp, ctypes.POINTER(Layout), ctypes.POINTER(AttnShape),
                                          vp, vp, vp]
    L.dsa_sparse_attn_noalloc.restype = ctypes.c_int
    L.dsa_sparse_attn_fp8kv.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Layout), ctypes.POINTER(AttnShape),
                                        vp, vp, vp, sz, vp]
    L.dsa_sparse_attn_fp8kv.restype = ctypes.c_int
    L.dsa_mxfp8_quantize.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]
    L.dsa_mxfp8_quantize.restype = ctypes.c_int
    L.dsa_indexer_cache_append.argtypes = [vp, ctypes.POINTER(Layout), ctypes.c_int32, ctypes.c_int32,
                                           vp, vp, vp]
    L.dsa_indexer_cache_append.restype = ctypes.c_int
    L.dsa_indexer_cache_append_fp8.argtypes = [vp, ctypes.POINTER(Layout), ctypes.c_int32, ctypes.c_int32,
                                               vp, vp, vp]
    L.dsa_indexer_cache_append_fp8.restype = ctypes.c_int
    L.dsa_latent_cache_append_fp8.argtypes = [vp, ctypes.POINTER(Layout), ctypes.c_int32, vp, vp, vp]
    L.dsa_latent_cache_append_fp8.restype = ctypes.c_int
    L.dsa_fp8_quantize_heads.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]
    L.dsa_fp8_quantize_heads.restype = ctypes.c_int
    L.dsa_last_error.argtypes = []
    L.dsa_last_error.restype = ctypes.c_char_p
    L.dsa_debug_status.argtypes = [vp]
    L.dsa_debug_status.restype = ctypes.c_int
    L.dsa_version.argtypes = []
    L.dsa_version.restype = ctypes.c_int
    L.dsa_profile_start.argtypes = []
    L.dsa_profile_start.restype = ctypes.c_int
    L.dsa_profile_stop.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int]
    L.dsa_profile_stop.restype = ctypes.c_int
    _lib = L
    return L


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(status: int):
    if status != DSA_OK:
        raise DsaError(status, lib().dsa_last_error().decode())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def make_layout(block_table: torch.Tensor, seq_lens: torch.Tensor, num_pages: int,
                max_seq_len: int) -> Layout:
    B, max_pages = block_table.shape
    return Layout(block_table.data_ptr(), seq_lens.data_ptr(), B, max_pages, PAGE_SIZE,
                  int(num_pages), int(max_seq_len))


def dsa_indexer_workspace_size(layout: Layout, shape: IndexerShape) -> int:
    return int(lib().dsa_indexer_workspace_size(ctypes.byref(layout), ctypes.byref(shape)))


def dsa_sparse_attn_workspace_size(layout: Layout, shape: AttnShape) -> int:
    return int(lib().dsa_sparse_attn_workspace_size(ctypes.byref(layout), ctypes.byref(shape)))


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch allocations are at least 256-byte aligned
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def dsa_indexer_topk(q, q_scale, w, k_cache, k_scale, block_table, seq_lens, *, T: int, top_k: int,
                     num_pages: int | None = None, max_seq_len: int, fp8: bool = False,
                     mx: bool = False, idx_out=None, workspace=None, stream=None) -> torch.Tensor:
    """Lightning Indexer + Top-K.  q [B,T,HI,DI] (bf16 or uint8 e4m3 codes), w [B,T,HI] fp32,
    k_cache [P,64,DI], block_table [B,max_pages] int32, seq_lens [B] int32 (device tensors).
    fp8: fp32 scales q_scale [B,T,HI] and k_scale [P]; mx (MXFP8): uint8 E8M0 scales
    q_scale [B,T,HI,DI/32] and k_scale [P,64,DI/32].  Returns idx_out [B,T,top_k] int32."""
    B, Tq, HI, DI = q.shape
    assert Tq == T
    P = k_cache.shape[0] if num_pages is None else num_pages
    layout = make_layout(block_table, seq_lens, P, max_seq_len)
    shape = IndexerShape(T, HI, DI, top_k, DSA_MXFP8_E4M3 if mx else (DSA_FP8_E4M3 if fp8 else DSA_BF16))
    if idx_out is None:
        idx_out = torch.empty((B, T, top_k), dtype=torch.int32, device=q.device)
    need = dsa_indexer_workspace_size(layout, shape)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check(lib().dsa_indexer_topk(_ptr(q), _ptr(q_scale), _ptr(w), _ptr(k_cache), _ptr(k_scale),
                                  ctypes.byref(layout), ctypes.byref(shape), _ptr(idx_out),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream)))
    return idx_out


def dsa_mxfp8_quantize(x, codes=None, scales=None, stream=None):
    """MXFP8 quantisation of bf16 rows x [..., dim] (dim a multiple of 32).  Returns (codes uint8
    [..., dim], scales uint8 E8M0 [..., dim / 32])."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    dim = x.shape[-1]
    rows = x.numel() // dim
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((*x.shape[:-1], dim // 32), dtype=torch.uint8, device=x.device)
    _check(lib().dsa_mxfp8_quantize(_ptr(x), rows, dim, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def dsa_indexer_cache_append(k_new, k_cache, k_scale, block_table, seq_lens, *, max_seq_len: int,
                             num_pages: int | None = None, stream=None):
    """Appends k_new [B, T, dim] bf16 (the T newest keys of each sequence) to the paged MXFP8 cache
    k_cache [P, 64, dim] uint8 / k_scale [P, 64, dim / 32] uint8, in place."""
    assert k_new.dtype == torch.bfloat16 and k_new.is_contiguous()
    B, T, dim = k_new.shape
    P = k_cache.shape[0] if num_pages is None else num_pages
    layout = make_layout(block_table, seq_lens, P, max_seq_len)
    _check(lib().dsa_indexer_cache_append(_ptr(k_new), ctypes.byref(layout), T, dim, _ptr(k_cache),
                                          _ptr(k_scale), _stream(stream)))
    return k_cache, k_scale


def dsa_indexer_cache_append_fp8(k_new, k_cache, k_scale, block_table, seq_lens, *, max_seq_len: int,
                                 num_pages: int | None = None, stream=None):
    """Appends k_new [B, T, dim] bf16 (the T newest keys of each sequence) to the per-page fp8
    cache k_cache [P, 64, dim] uint8 / k_scale [P] fp32, in place (a page's scale grows with the
    keys it receives; its held codes are re-encoded when it does)."""
    assert k_new.dtype == torch.bfloat16 and k_new.is_contiguous()
    assert k_scale.dtype == torch.float32
    B, T, dim = k_new.shape
    P = k_cache.shape[0] if num_pages is None else num_pages
    layout = make_layout(block_table, seq_lens, P, max_seq_len)
    _check(lib().dsa_indexer_cache_append_fp8(_ptr(k_new), ctypes.byref(layout), T, dim, _ptr(k_cache),
                                              _ptr(k_scale), _stream(stream)))
    return k_cache, k_scale


def dsa_fp8_quantize_heads(x, codes=None, scales=None, stream=None):
    """Per-head fp8 quantisation of indexer queries x [..., dim] bf16 (dim 64 or 128).  Returns
    (codes uint8 [..., dim], scales fp32 [...]): the q and q_scale of the fp8 indexer."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    dim = x.shape[-1]
    rows = x.numel() // dim
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _check(lib().dsa_fp8_quantize_heads(_ptr(x), rows, dim, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def dsa_latent_cache_append_fp8(kv_new, kv_codes, kv_scale, block_table, seq_lens, *, max_seq_len: int,
                                num_pages: int | None = None, stream=None):
    """Appends kv_new [B, T, 576] bf16 (the T newest latent rows of each sequence) to the FP8 latent
    cache kv_codes [P, 64, 576] uint8 / kv_scale [P, 64, 8] fp32, in place."""
    assert kv_new.dtype == torch.bfloat16 and kv_new.is_contiguous() and kv_new.shape[-1] == 576
    B, T, _ = kv_new.shape
    P = kv_codes.shape[0] if num_pages is None else num_pages
    layout = make_layout(block_table, seq_lens, P, max_seq_len)
    _check(lib().dsa_latent_cache_append_fp8(_ptr(kv_new), ctypes.byref(layout), T, _ptr(kv_codes),
                                             _ptr(kv_scale), _stream(stream)))
    return kv_codes, kv_scale


def dsa_sparse_attn(q, kv_cache, idx, block_table, seq_lens, *, sm_scale: float, max_seq_len: int,
                    num_pages: int | None = None, out=None, lse=None, want_lse: bool = True,
                    workspace=None, stream=None):
    """Sparse attention.  q [B,T,H,576] bf16, kv_cache [P,64,576] bf16, idx [B,T,K] int32.
    Returns (out [B,T,H,512] bf16, lse [B,T,H] fp32 or None)."""
    B, T, H, D = q.shape
    K = idx.shape[-1]
    P = kv_cache.shape[0] if num_pages is None else num_pages
    layout = make_layout(block_table, seq_lens, P, max_seq_len)
    shape = AttnShape(T, H, D, DIM_V, K, float(sm_scale))
    if out is None:
        out = torch.empty((B, T, H, DIM_V), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    need = dsa_sparse_attn_workspace_size(layout, shape)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_sparse_attn(_ptr(q), _ptr(kv_cache), _ptr(idx), ctypes.byref(layout),
                                 ctypes.byref(shape), _ptr(out), _ptr(lse), _ptr(workspace), wsb,
                                 _stream(stream)))
    return out, lse


def dsa_sparse_attn_noalloc(q, kv_cache, idx, block_table, seq_lens, *, sm_scale: float,
                            max_seq_len: int, num_pages: int | None = None, out=None, lse=None,
                            want_lse: bool = True, stream=None):
    """dsa_sparse_attn without a workspace: the library's static per-GPU scratch is used instead
    (outputs are still allocated here when not given)."""
    B, T, H, D = q.shape
    K = idx.shape[-1]
    P = kv_cache.shape[0] if num_pages is None else num_pages
    layout = make_layout(block_table, seq_lens, P, max_seq_len)
    shape = AttnShape(T, H, D, DIM_V, K, float(sm_scale))
    if out is None:
        out = torch.empty((B, T, H, DIM_V), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    _check(lib().dsa_sparse_attn_noalloc(_ptr(q), _ptr(kv_cache), _ptr(idx), ctypes.byref(layout),
                                         ctypes.byref(shape), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def dsa_sparse_attn_fp8kv(q, kv_codes, kv_scale, idx, block_table, seq_lens, *, sm_scale: float,
                          max_seq_len: int, num_pages: int | None = None, out=None, lse=None,
                          want_lse: bool = True, workspace=None, stream=None):
    """Sparse attention over an FP8 latent cache: kv_codes [P,64,576] uint8 (E4M3), kv_scale
    [P,64,8] fp32 tile scales; otherwise as dsa_sparse_attn."""
    B, T, H, D = q.shape
    K = idx.shape[-1]
    P = kv_codes.shape[0] if num_pages is None else num_pages
    layout = make_layout(block_table, seq_lens, P, max_seq_len)
    shape = AttnShape(T, H, D, DIM_V, K, float(sm_scale))
    if out is None:
        out = torch.empty((B, T, H, DIM_V), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device)
    need = dsa_sparse_attn_workspace_size(layout, shape)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_sparse_attn_fp8kv(_ptr(q), _ptr(kv_codes), _ptr(kv_scale), _ptr(idx),
                                       ctypes.byref(layout), ctypes.byref(shape), _ptr(out), _ptr(lse),
                                       _ptr(workspace), wsb, _stream(stream)))
    return out, lse


def dsa_profile_start() -> None:
    _check(lib().dsa_profile_start())


def dsa_profile_stop() -> dict:
    """{kernel name: (launches, total GPU ms)} recorded since dsa_profile_start()."""
    buf = (KernelTime * 64)()
    n = lib().dsa_profile_stop(buf, 64)
    if n < 0:
        raise DsaError(6, "dsa_profile_stop: HIP error")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n, 64))}


def dsa_debug_status(stream=None) -> None:
    """Synchronises the stream and raises DsaError if a kernel met a violated device-side
    precondition since the last call (bad block-table entry, sequence length or attention
    index); the record is cleared by reading it."""
    _check(lib().dsa_debug_status(_stream(stream)))
