"""CPU oracle for the DSA Lightning-Indexer + Sparse-Flash-Attention path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously-correct definition that the
HIP kernels are checked against.  Only the tests, the package's smoke check and the benchmark's CPU
baseline leg may import it; the product path never does, and it shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing).  NumPy only, float64
arithmetic on the decoded bf16 / e4m3 inputs.

Pages cited (titles shortened after first use):
  [P1] "Inference Optimization for Kimi K3.1 Pro: Decoding Architecture Evolution and Systems
       Engineering Practices"
  [P2] "Optimizing Kimi K3.1 Pro Sparse Attention Inference: Day0 Adaptation and Performance Tuning
       on Ascend"
  [P3] "Day0 Inference Adaptation for Next-Gen LLMs: Deep Optimization Practices with CANN
       Heterogeneous Computing Architecture"

What the oracle computes (readings of the pages where they are silent are marked "reading"):
  * indexer_topk_ref  -- [P1] §1 (DSA steps 1-2: Lightning-Indexer relevance score with head
    weights, then Top-K positions), [P1] §2 (only indices leave the fused operator; indices address
    the paged cache), [P3] §3.1 (score, head-weight sum, Top-K; paged K cache read in place).
    Score (reading): I[t,s] = sum_h w[t,h] * ReLU(q[t,h,:] . k[s,:]) with one key vector per
    position shared by all indexer heads; ties go to the lower position; output is the selected
    logical positions in ascending order, padded with -1 to K.
  * sparse_attn_ref   -- [P1] §1 (DSA step 3: attention over the KV rows at the selected indices),
    [P2] "Inheritance and Extension of Core Operators" (blockwise attention whose cross-block
    reduction equals the global softmax).  Reading: exact softmax over the selected set, MLA latent
    rows of width 576 of which the first 512 columns are V, explicit softmax scale.
  * sparse_attn_fp8kv_ref / dequant_kv_fp8 -- [P1] §4 (FP8 SFA cache, per-token scales over
    128-wide tiles, BF16 products).  Reading: 5 fp32 scales per token (columns 0-127, ..., 384-511,
    512-575), element = bf16(float32(e4m3(code) * scale)), then sparse_attn_ref on those rows.
  * codecs            -- bf16, OCP E4M3FN and E8M0 (MX shared scale) decoding from the format
    definitions.  The MXFP8 indexer inputs ([P1] §4) are E4M3FN codes with one E8M0 scale per 32
    consecutive elements of each q row and each cached key row.

Pins: every function is pinned in tests/test_oracle_*.py against closed forms, invariants,
brute force on tiny inputs and library routines (torch casts, torch SDPA); see the test headers.
"""
from .codecs import bf16_bits_to_f64, e4m3_codes_to_f64, e4m3_table, e8m0_to_f64  # noqa: F401
from .indexer import indexer_scores_ref, indexer_topk_ref, visible_positions  # noqa: F401
from .sfa import dequant_kv_fp8, sparse_attn_fp8kv_ref, sparse_attn_ref  # noqa: F401
