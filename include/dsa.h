/* dsa.h -- C ABI of the MI355X (gfx950) DSA hot path: Lightning Indexer with fused Top-K, and
 * Sparse Flash Attention over the selected MLA latent rows.
 *
 * Pages cited:
 *   [P1] "Inference Optimization for Kimi K3.1 Pro: Decoding Architecture Evolution and Systems
 *        Engineering Practices"
 *   [P2] "Optimizing Kimi K3.1 Pro Sparse Attention Inference: Day0 Adaptation and Performance
 *        Tuning on Ascend"
 *   [P3] "Day0 Inference Adaptation for Next-Gen LLMs: Deep Optimization Practices with CANN
 *        Heterogeneous Computing Architecture"
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers into caller-owned memory, contiguous, row-major, with
 *     the alignment stated per argument.  The library never allocates, frees or retains device
 *     memory; scratch comes from the caller's `workspace` (size from the *_workspace_size call).
 *     The one exception is dsa_sparse_attn_noalloc, which uses a static per-GPU array instead.
 *   - Calls are asynchronous on `stream` (NULL = the null stream); nothing is synchronised and
 *     nothing is allocated, so a call may be captured into a hipGraph.  Buffers must stay alive
 *     until the stream has passed the call.  Calls are deterministic: identical inputs give
 *     bitwise-identical outputs.  Two calls that share a workspace must be ordered on one stream.
 *   - Argument errors (NULL pointer, misalignment, unsupported or inconsistent shape, workspace
 *     too small) are detected on the host before anything is launched; the call then returns a
 *     non-OK status, launches nothing and leaves outputs untouched.  A launch failure returns
 *     DSA_ERR_HIP.  dsa_last_error() gives a thread-local description of the last failure.
 *   - Workgroups of one launch meet through device memory in two places: a decode indexer
 *     workgroup waits for the workgroup that makes sure its row's histogram is clear, and an
 *     attention combine workgroup waits for the split workgroups of its row.  The workgroup waited
 *     for always has a lower index than the waiting one, so the waits end as long as the GPU
 *     dispatches the workgroups of a launch in index order (which AMD GPUs do).  Each wait is
 *     bounded (about 50 ms of polling): if it ever gives up, the affected outputs are not computed
 *     from partial data -- the indexer row is written as all -1, the attention outputs of the row
 *     (out and lse) as NaN -- and dsa_debug_status() reports the timeout.  Test hooks, read at
 *     each indexer call and unset in normal use: DSA_TEST_SYNC_SPIN_CAP=<n> bounds the indexer
 *     wait at n polls, and DSA_TEST_WITHHOLD_TAG=1 makes the clearing workgroups skip their
 *     signal, so every indexer row with more than top_k visible keys takes the timeout path.
 *   - Device-side preconditions (not checked on the host because the data lives on the device):
 *     T <= seq_lens[b] <= max_seq_len <= max_pages * page_size, block_table entries used by a
 *     sequence lie in [0, num_pages), fp8 scales are finite and > 0.  The kernels clamp page ids
 *     and lengths so that a violated precondition gives wrong numbers, never an out-of-bounds
 *     access.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_VERSION 4             /* 4: per-page fp8 indexer-K append; 3: FP8 latent cache, per-head fp8 q */
#define DSA_PAGE_SIZE 64          /* tokens per cache page */
#define DSA_DIM_QK 576            /* MLA latent row: 512 "nope" + 64 rope columns */
#define DSA_DIM_V 512             /* V = the first 512 columns of the latent row */
#define DSA_MAX_TOP_K 2048        /* largest supported K */

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,          /* a required pointer is NULL */
  DSA_ERR_SHAPE = 2,         /* inconsistent or out-of-range size */
  DSA_ERR_ALIGN = 3,         /* pointer not aligned as documented */
  DSA_ERR_UNSUPPORTED = 4,   /* valid request the library has no kernel for */
  DSA_ERR_WORKSPACE = 5,     /* workspace NULL or smaller than *_workspace_size */
  DSA_ERR_HIP = 6            /* the HIP runtime reported an error at launch */
} dsa_status;

typedef enum {
  DSA_BF16 = 0,              /* bfloat16 */
  DSA_FP8_E4M3 = 1,          /* OCP E4M3FN (max 448, no infinities), fp32 scale per q head and
                                per K page */
  DSA_MXFP8_E4M3 = 2         /* MXFP8 (OCP Microscaling): E4M3FN codes, one E8M0 scale byte
                                2^(e - 127) per 32 consecutive elements of each q head row and
                                each cached key row ([P1] §4, [P3] §3.3); indexer only, on
                                every query-row count (decode, verify, causal prefill) */
} dsa_dtype;

/* Geometry of the paged caches ([P1] §2: indices resolve to page slots on demand; [P3] §3.1: the
 * paged K cache is read in place).  Logical token s of sequence b lives in physical page
 * block_table[b * max_pages + s / page_size], slot s % page_size.  The indexer-K cache and the
 * latent-KV cache share this geometry. */
typedef struct {
  const int32_t *block_table;   /* device, [batch, max_pages] physical page ids, 4-byte aligned */
  const int32_t *seq_lens;      /* device, [batch] tokens in the cache INCLUDING the T query
                                   tokens of this call; 4-byte aligned */
  int32_t batch;                /* >= 1 */
  int32_t max_pages;            /* row length of block_table, >= ceil(max_seq_len / page_size) */
  int32_t page_size;            /* must be DSA_PAGE_SIZE */
  int32_t num_pages;            /* pages in each cache pool */
  int32_t max_seq_len;          /* host-side upper bound of seq_lens[] (sizes the launch grid) */
} dsa_paged_layout;

/* Query t (0 <= t < T) of sequence b sits at position pos = seq_lens[b] - T + t and sees keys
 * 0..pos (its own key included): T = 1 is decode, T = 4 speculative verify of 4 causal drafts,
 * T = seq_len a causal prefill chunk over its own context. */
typedef struct {
  int32_t T;                    /* query tokens per sequence, >= 1 */
  int32_t heads;                /* indexer heads H_I: 8, 16, 32 or 64 */
  int32_t dim;                  /* indexer head dim d_I: 64 or 128 */
  int32_t top_k;                /* K, 1..DSA_MAX_TOP_K */
  dsa_dtype dtype;              /* storage of q and the indexer-K cache (any T for all three) */
} dsa_indexer_shape;

typedef struct {
  int32_t T;                    /* query tokens per sequence, >= 1 */
  int32_t heads;                /* attention heads H: a multiple of 16, 16..128 */
  int32_t dim_qk;               /* must be DSA_DIM_QK */
  int32_t dim_v;                /* must be DSA_DIM_V */
  int32_t top_k;                /* row length of the index tensor, 1..DSA_MAX_TOP_K */
  float sm_scale;               /* softmax scale applied to q.k (e.g. 1/sqrt(576)) */
} dsa_attn_shape;

/* Bytes of workspace dsa_indexer_topk needs for this layout and shape (0 on invalid input). */
size_t dsa_indexer_workspace_size(const dsa_paged_layout *layout, const dsa_indexer_shape *shape);

/* Lightning Indexer with fused Top-K ([P1] §1 DSA steps 1-2; [P1] §2 "Single Fused Kernel":
 * score, head weighting and Top-K keep their intermediates on chip and only the selected indices
 * are output; [P3] §3.1, bf16 and quantised indexer paths in prefill and decode).
 *
 * For every query row (b, t) it computes, for each visible key s (0 <= s <= pos),
 *     I[s] = sum_h w[b,t,h] * max(0, q[b,t,h,:] . k[s,:])
 * (fp8: q = q_scale[b,t,h] * e4m3(q code), k = k_scale[page of s] * e4m3(k code); MXFP8:
 * q[d] = 2^(q_scale[b,t,h,d/32] - 127) * e4m3(q code[d]) and k[d] likewise with the key's own
 * scale bytes k_scale[page of s, slot of s, d/32]), keeps the
 * K' = min(top_k, pos + 1) largest scores with ties going to the lower position, and writes
 * those positions in ascending order followed by -1 up to top_k.  Scores are accumulated in fp32.
 *
 *   q        [batch, T, heads, dim]  bf16 or e4m3, 16-byte aligned
 *   q_scale  DSA_FP8_E4M3: [batch, T, heads] fp32 > 0, 4-byte aligned;
 *            DSA_MXFP8_E4M3: [batch, T, heads, dim / 32] uint8 E8M0 exponents (255 = NaN);
 *            bf16: must be NULL
 *   w        [batch, T, heads] fp32 head weights, 4-byte aligned
 *   k_cache  [num_pages, page_size, dim] bf16 or e4m3 (same dtype as q), 16-byte aligned
 *   k_scale  DSA_FP8_E4M3: [num_pages] fp32 > 0, one per page, 4-byte aligned;
 *            DSA_MXFP8_E4M3: [num_pages, page_size, dim / 32] uint8 E8M0 exponents, 16-byte
 *            aligned; bf16: must be NULL
 *   idx_out  [batch, T, top_k] int32 logical positions, ascending, -1 padded; 4-byte aligned
 *   workspace / workspace_bytes: device scratch, 256-byte aligned, at least
 *            dsa_indexer_workspace_size() bytes; contents on entry are ignored (a call leaves
 *            the rows' histograms it read zero, so the next call on the same workspace skips
 *            clearing them; any other contents are cleared first).
 */
dsa_status dsa_indexer_topk(const void *q, const void *q_scale, const float *w,
                            const void *k_cache, const void *k_scale,
                            const dsa_paged_layout *layout, const dsa_indexer_shape *shape,
                            int32_t *idx_out, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* MXFP8 quantisation of bf16 rows ([P1] §4: the Lightning Indexer's Q and K in MXFP8; [P1] §3,
 * [P3] §3.3: the indexer prolog quantises the indexer q and k).  Each run of 32 consecutive
 * elements of a row shares the E8M0 exponent s = floor(log2(max |v|)) - 8 (OCP Microscaling;
 * clamped to [-127, 127], -127 for a run of zeros); its elements are v * 2^-s rounded to E4M3
 * (nearest, ties to even) and clamped to +-448.  Finite inputs only.
 *
 *   x       [rows, dim] bf16, 16-byte aligned; dim a multiple of 32 (32..4096)
 *   codes   [rows, dim] E4M3 codes, 16-byte aligned
 *   scales  [rows, dim / 32] E8M0 bytes (value 2^(e - 127))
 * For the indexer queries: rows = batch * T * heads, the layout dsa_indexer_topk reads with
 * DSA_MXFP8_E4M3. */
dsa_status dsa_mxfp8_quantize(const void *x, int64_t rows, int32_t dim, void *codes, void *scales,
                              hipStream_t stream);

/* Appends the T newest keys of every sequence to the paged MXFP8 indexer-K cache ([P1] §3: the
 * prolog writes the new keys into the cache; §4: MXFP8 storage), quantising each key row exactly as
 * dsa_mxfp8_quantize does.  Key t of sequence b is logical position seq_lens[b] - T + t (the
 * lengths already count the new tokens, as in dsa_indexer_topk) and is written to page
 * block_table[b, pos / page_size], slot pos % page_size; nothing else in the cache changes.
 *
 *   k_new    [batch, T, dim] bf16, 16-byte aligned; dim a multiple of 32 (32..4096)
 *   k_cache  [num_pages, page_size, dim] E4M3 codes, 16-byte aligned
 *   k_scale  [num_pages, page_size, dim / 32] E8M0 bytes
 * Positions of one call must be distinct (true whenever the block tables of different sequences
 * do not share pages); seq_lens and block_table entries are device-side preconditions as for
 * dsa_indexer_topk. */
dsa_status dsa_indexer_cache_append(const void *k_new, const dsa_paged_layout *layout, int32_t T,
                                    int32_t dim, void *k_cache, void *k_scale, hipStream_t stream);

/* Appends the T newest keys of every sequence to the per-page fp8 indexer-K cache that
 * dsa_indexer_topk reads with DSA_FP8_E4M3 ([P1] §3: the prolog writes each step's new keys into
 * the cache; the fp8 indexer keys carry one fp32 scale per page).  Key t of sequence b is logical
 * position seq_lens[b] - T + t, stored at page block_table[b, pos / 64], slot pos % 64.
 *
 * A page's scale only grows: it is the largest |key| the page has received / 448 (fp32 division),
 * 1 while it has received only zeros.  For each page that receives new keys, with m = the largest
 * |element| of those keys and s_old = the page's stored scale if it already holds keys of the
 * sequence (positions before seq_lens[b] - T; otherwise the stored value is ignored):
 *     s = max(s_old, m / 448)  (1 if that is 0)
 *     if s > s_old, every held code c becomes E4M3((e4m3(c) * s_old) / s)   (a second rounding)
 *     new codes are E4M3(x / s);  k_scale[page] = s
 * with every product and quotient rounded to nearest even in fp32 and every E4M3 conversion
 * nearest even, clamped to +-448.  A page written by one call holds exactly the one-shot
 * quantisation (scale = amax / 448 of its keys).  Nothing else in the cache changes.
 *
 *   k_new    [batch, T, dim] bf16, finite, 16-byte aligned; dim 64 or 128
 *   k_cache  [num_pages, page_size, dim] E4M3FN codes, 16-byte aligned; held codes finite
 *   k_scale  [num_pages] fp32, 4-byte aligned; held pages' scales positive and finite
 * The block-table entries a call reaches must name distinct pages, within a sequence and across
 * sequences (each page is rewritten by one workgroup).  A sequence whose length lies outside [T, max_seq_len] is left untouched and sets
 * the length check that dsa_debug_status() reports; block_table entries are device-side
 * preconditions as for dsa_indexer_topk.  DSA_ERR_UNSUPPORTED for another dim, DSA_ERR_SHAPE for
 * T < 1 or batch * T beyond 2^31 - 1, DSA_ERR_NULL / DSA_ERR_ALIGN as named. */
dsa_status dsa_indexer_cache_append_fp8(const void *k_new, const dsa_paged_layout *layout, int32_t T,
                                        int32_t dim, void *k_cache, float *k_scale, hipStream_t stream);

/* Bytes of workspace dsa_sparse_attn needs for this layout and shape (0 on invalid input). */
size_t dsa_sparse_attn_workspace_size(const dsa_paged_layout *layout, const dsa_attn_shape *shape);

/* Sparse Flash Attention ([P1] §1 DSA step 3: read the KV cache at the selected indices and
 * attend over them; [P1] §2: indices resolve to pages in place; [P2] "Inheritance and Extension
 * of Core Operators": blockwise attention with a cross-block reduction that reproduces the
 * global softmax).
 *
 * For each query row (b, t) with selected set S = { idx[b,t,j] : idx[b,t,j] >= 0 } and each head h:
 *     z_j = sm_scale * q[b,t,h,:] . X[s_j,:]     (X = 576-wide latent row of token s_j)
 *     out[b,t,h,:] = sum_j softmax(z)_j * X[s_j, 0:512],   lse[b,t,h] = ln sum_j exp(z_j)
 * with fp32 accumulation; out is rounded to bf16 (round to nearest even).  An empty set gives
 * out = 0 and lse = -inf.  The softmax runs against a fixed per-head reference taken from the first
 * 32 selected keys of each split (their maximum logit + 64 in log2 units); a later logit more than
 * 100 log2 units above it raises the reference and restarts the split from its first key, so the
 * result is exact for any logits, and the extra cost is at most one more pass over the split per
 * raise: a split of t 32-key tiles whose largest logit climbs by more than 164 log2 units (about
 * 114 in natural units, after sm_scale) from each tile to the next restarts up to t - 1 times,
 * about t^2 / 2 tile passes in all; real attention logits stay within one reference.  An entry
 * outside [0, pos], pos = seq_lens[b] - T + t (the positions query t may attend to), is skipped
 * like -1 and sets the attention-index check that dsa_debug_status() reports.
 *
 *   q         [batch, T, heads, 576] bf16 (MLA-absorbed query), 16-byte aligned
 *   kv_cache  [num_pages, page_size, 576] bf16 latent rows, 16-byte aligned
 *   idx       [batch, T, top_k] int32, -1 = skip; entries of a row must be unique
 *   out       [batch, T, heads, 512] bf16, 16-byte aligned
 *   lse       [batch, T, heads] fp32 natural-log LSE, or NULL
 *   workspace / workspace_bytes: device scratch, 256-byte aligned, at least
 *             dsa_sparse_attn_workspace_size() bytes (may be 0 / NULL when that size is 0).
 */
dsa_status dsa_sparse_attn(const void *q, const void *kv_cache, const int32_t *idx,
                           const dsa_paged_layout *layout, const dsa_attn_shape *shape,
                           void *out, float *lse, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Sparse Flash Attention for callers that cannot allocate device memory or own a workspace (code
 * under hipGraph capture, tight serving loops, harnesses that forbid allocation).  Same operation,
 * arguments, output and errors as dsa_sparse_attn, minus the workspace: the scratch comes from a
 * static array of DSA_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy per GPU, held from
 * the first call on that GPU until the process ends.  The call allocates nothing (no hipMalloc,
 * no hipFree).  A shape whose scratch need (dsa_sparse_attn_workspace_size) exceeds
 * DSA_NOALLOC_SCRATCH_BYTES returns DSA_ERR_WORKSPACE and launches nothing; every shape the
 * library supports fits today.  All calls on one GPU share its array: calls that may overlap on
 * one GPU (different streams, no ordering between them) race and give wrong results; calls
 * ordered on one stream are safe and need no clearing between them. */
#define DSA_NOALLOC_SCRATCH_BYTES (72u << 20)
dsa_status dsa_sparse_attn_noalloc(const void *q, const void *kv_cache, const int32_t *idx,
                                   const dsa_paged_layout *layout, const dsa_attn_shape *shape,
                                   void *out, float *lse, hipStream_t stream);

/* Sparse Flash Attention over an FP8 latent cache ([P1] §4: the SFA cache stored in FP8 with
 * per-token scales over 128-wide tiles; the products stay BF16 and the dequantised BF16 tile feeds
 * the matrix unit directly).  Same operation, arguments, workspace and errors as dsa_sparse_attn,
 * with the cache given as
 *   kv_codes  [num_pages, page_size, 576] E4M3FN codes (uint8), 16-byte aligned
 *   kv_scale  [num_pages, page_size, 8] fp32, 16-byte aligned: per token the scales of columns
 *             0-127, 128-255, 256-383, 384-511 and 512-575 (entries 5-7 are not read)
 * Each selected row is dequantised as bf16(e4m3(code) * scale), the float32 product rounded to
 * nearest even and then to bf16 (nearest even), before the bf16 products of dsa_sparse_attn.
 * The workspace size is dsa_sparse_attn_workspace_size() of the same layout and shape. */
dsa_status dsa_sparse_attn_fp8kv(const void *q, const void *kv_codes, const float *kv_scale,
                                 const int32_t *idx, const dsa_paged_layout *layout,
                                 const dsa_attn_shape *shape, void *out, float *lse, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* Per-head fp8 quantisation of indexer queries for DSA_FP8_E4M3 ([P1] §3: the prolog quantises the
 * indexer q; dsa_indexer_topk folds each head's weight and scale together, w * sq, when it loads a
 * query row).  x [rows, dim] bf16 (rows = batch * T * heads, one head row each; dim 64 or 128;
 * 16-byte aligned) -> codes [rows, dim] E4M3FN (16-byte aligned) and scales [rows] fp32 (the
 * q_scale of dsa_indexer_topk): per row sq = amax / 448 (1 for an all-zero row), code = E4M3(x / sq),
 * both divisions fp32 nearest even, codes nearest even, clamped to +-448.  Finite inputs.  rows = 0
 * is a no-op.  DSA_ERR_UNSUPPORTED for another dim, DSA_ERR_NULL / DSA_ERR_ALIGN as named. */
dsa_status dsa_fp8_quantize_heads(const void *x, int64_t rows, int32_t dim, void *codes, float *scales,
                                  hipStream_t stream);

/* FP8 latent-cache append (the prolog step that writes a step's new latent rows into the cache
 * that dsa_sparse_attn_fp8kv reads; [P1] §4: FP8 SFA cache with per-token scales over tiles of
 * 128).  kv_new [batch, T, 576] bf16 (16-byte aligned): token t of sequence b is logical position
 * seq_lens[b] - T + t, written to page block_table[b, pos / 64], slot pos % 64 of kv_codes
 * [num_pages, 64, 576] E4M3 and kv_scale [num_pages, 64, 8] fp32 (both 16-byte aligned).  Per
 * token and per 128-column tile (0-127, ..., 384-511, 512-575): scale = amax / 448 (1 for an
 * all-zero tile), code = E4M3(x / scale), both divisions fp32 nearest even, codes nearest even and
 * clamped to +-448; scale entries 5-7 are set to 1.  Finite inputs.  seq_lens must already count
 * the T new tokens.  Errors as for dsa_indexer_cache_append. */
dsa_status dsa_latent_cache_append_fp8(const void *kv_new, const dsa_paged_layout *layout, int32_t T,
                                       void *kv_codes, float *kv_scale, hipStream_t stream);

/* Opt-in per-kernel timing (off by default).  dsa_profile_start() turns recording on for the
 * calling thread: each kernel the library then launches from this thread is bracketed by two
 * hipEvents on its stream (events come from a reusable host-side pool; no device memory).
 * dsa_profile_stop() turns recording off, waits for the recorded events, and writes up to
 * max_entries per-kernel totals (kernel name, launch count, summed GPU milliseconds) to `out`;
 * it returns the number of distinct kernels seen, or -1 if the HIP runtime reported an error.
 * The extra event records perturb back-to-back launches slightly, so time whole calls without
 * recording and use recording for the per-kernel split. */
typedef struct {
  char name[48];
  int32_t launches;
  double total_ms;
} dsa_kernel_time;

dsa_status dsa_profile_start(void);
int dsa_profile_stop(dsa_kernel_time *out, int max_entries);

/* Thread-local text describing the last non-OK status returned on this thread ("" if none). */
const char *dsa_last_error(void);

/* DSA_VERSION of the library. */
int dsa_version(void);

/* Synchronises `stream`, then reports the device-side precondition checks of every call made on
 * the current device since the last dsa_debug_status (the kernels clamp or skip what fails them,
 * see the conventions above, and record which kind failed).  Returns DSA_OK when none failed;
 * DSA_ERR_SHAPE when some did, with dsa_last_error() naming them (a block_table entry outside
 * [0, num_pages) for a visible position, a seq_lens entry outside [T, max_seq_len], an attention
 * index that is neither -1 nor a visible position, a timed-out wait between workgroups (see the
 * conventions above)); DSA_ERR_HIP if the synchronisation fails.
 * Reading clears the record.  The checks cost a compare per page or index in the kernels'
 * set-up code and run in every build. */
dsa_status dsa_debug_status(hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
