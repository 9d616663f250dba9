"""MI355X (gfx950) DSA hot path: Lightning Indexer with fused Top-K and Sparse Flash Attention.

The computation lives in hand-written HIP kernels behind the C ABI of include/dsa.h (libdsa.so,
built in-tree by sparse_attention_15_amd.build).  This package only marshals torch tensors into
that ABI; it has no fallback path.
"""
from ._lib import (DSA_BF16, DSA_FP8_E4M3, DSA_MXFP8_E4M3, AttnShape, DsaError,  # noqa: F401
                   IndexerShape, Layout, dsa_debug_status, dsa_indexer_cache_append, dsa_indexer_cache_append_fp8,
                   dsa_latent_cache_append_fp8,
                   dsa_fp8_quantize_heads,
                   dsa_indexer_topk, dsa_indexer_workspace_size, dsa_mxfp8_quantize,
                   dsa_profile_start, dsa_profile_stop, dsa_sparse_attn, dsa_sparse_attn_fp8kv,
                   dsa_sparse_attn_noalloc,
                   dsa_sparse_attn_workspace_size, lib, make_layout)

__all__ = ["dsa_indexer_topk", "dsa_sparse_attn", "dsa_sparse_attn_noalloc", "dsa_sparse_attn_fp8kv", "dsa_mxfp8_quantize", "dsa_indexer_cache_append", "dsa_indexer_cache_append_fp8", "dsa_latent_cache_append_fp8", "dsa_fp8_quantize_heads", "dsa_indexer_workspace_size", "dsa_debug_status",
           "dsa_sparse_attn_workspace_size", "dsa_profile_start", "dsa_profile_stop", "DsaError", "Layout", "IndexerShape", "AttnShape",
           "make_layout", "lib"]
