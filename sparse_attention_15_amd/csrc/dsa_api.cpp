// dsa_api.cpp -- the C ABI declared in include/dsa.h: host-side validation, workspace sizing and
// dispatch to the gfx950 kernels.  Nothing here allocates device memory or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <string>

#include "dsa.h"
#include "dsa_internal.h"

namespace dsa {

unsigned long long next_call_tag() {
  static std::atomic<unsigned long long> counter{
      (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count() ^
      (unsigned long long)(uintptr_t)&counter};
  unsigned long long z = counter.fetch_add(0x9E3779B97F4A7C15ull) + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z | 1ull;
}

}  // namespace dsa

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

dsa_status check_layout(const dsa_paged_layout* L, int T) {
  if (L == nullptr) return fail(DSA_ERR_NULL, "layout is NULL");
  if (L->block_table == nullptr || L->seq_lens == nullptr)
    return fail(DSA_ERR_NULL, "layout.block_table / layout.seq_lens is NULL");
  if (!aligned(L->block_table, 4) || !aligned(L->seq_lens, 4))
    return fail(DSA_ERR_ALIGN, "block_table / seq_lens must be 4-byte aligned");
  if (L->page_size != DSA_PAGE_SIZE)
    return fail(DSA_ERR_UNSUPPORTED, "page_size %d unsupported (only %d)", L->page_size, DSA_PAGE_SIZE);
  if (L->batch < 1) return fail(DSA_ERR_SHAPE, "batch %d < 1", L->batch);
  if (L->num_pages < 1) return fail(DSA_ERR_SHAPE, "num_pages %d < 1", L->num_pages);
  if (L->max_seq_len < T) return fail(DSA_ERR_SHAPE, "max_seq_len %d < T %d", L->max_seq_len, T);
  if (L->max_seq_len > (1 << 20)) return fail(DSA_ERR_UNSUPPORTED, "max_seq_len %d > 1048576", L->max_seq_len);
  if ((long long)L->max_pages * L->page_size < L->max_seq_len)
    return fail(DSA_ERR_SHAPE, "max_pages %d * page_size too small for max_seq_len %d", L->max_pages, L->max_seq_len);
  return DSA_OK;
}

dsa_status check_indexer_shape(const dsa_indexer_shape* S) {
  if (S == nullptr) return fail(DSA_ERR_NULL, "shape is NULL");
  if (S->T < 1) return fail(DSA_ERR_SHAPE, "T %d < 1", S->T);
  if (S->top_k < 1 || S->top_k > DSA_MAX_TOP_K)
    return fail(DSA_ERR_UNSUPPORTED, "top_k %d outside 1..%d", S->top_k, DSA_MAX_TOP_K);
  if (S->dtype != DSA_BF16 && S->dtype != DSA_FP8_E4M3 && S->dtype != DSA_MXFP8_E4M3)
    return fail(DSA_ERR_UNSUPPORTED, "unknown dtype %d", (int)S->dtype);
  if (!dsa::indexer_supported(S->heads, S->dim))
    return fail(DSA_ERR_UNSUPPORTED, "indexer heads %d x dim %d unsupported (heads 8/16/32/64, dim 64/128)", S->heads, S->dim);
  return DSA_OK;
}

dsa_status check_attn_shape(const dsa_attn_shape* S) {
  if (S == nullptr) return fail(DSA_ERR_NULL, "shape is NULL");
  if (S->T < 1) return fail(DSA_ERR_SHAPE, "T %d < 1", S->T);
  if (S->dim_qk != DSA_DIM_QK || S->dim_v != DSA_DIM_V)
    return fail(DSA_ERR_UNSUPPORTED, "dims %d/%d unsupported (only %d/%d)", S->dim_qk, S->dim_v, DSA_DIM_QK, DSA_DIM_V);
  if (S->heads < 16 || S->heads > 128 || S->heads % 16 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "attention heads %d unsupported (multiple of 16, 16..128)", S->heads);
  if (S->top_k < 1 || S->top_k > DSA_MAX_TOP_K)
    return fail(DSA_ERR_UNSUPPORTED, "top_k %d outside 1..%d", S->top_k, DSA_MAX_TOP_K);
  if (!(S->sm_scale == S->sm_scale) || S->sm_scale <= 0.f || S->sm_scale > 1e4f)
    return fail(DSA_ERR_SHAPE, "sm_scale must be finite and > 0");
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_version(void) { return DSA_VERSION; }

const char* dsa_last_error(void) { return g_last_error.c_str(); }

dsa_status dsa_debug_status(hipStream_t stream) {
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "stream synchronize: %s", hipGetErrorString(e));
  uint32_t fi = 0, fa = 0, fq = 0;
  e = dsa::indexer_take_input_flags(&fi);
  if (e == hipSuccess) e = dsa::attn_take_input_flags(&fa);
  if (e == hipSuccess) e = dsa::quant_take_input_flags(&fq);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "reading the input-check flags: %s", hipGetErrorString(e));
  const uint32_t f = fi | fa | fq;
  if (f == 0) return DSA_OK;
  return fail(DSA_ERR_SHAPE, "device-side input checks failed:%s%s%s%s",
              (f & 1u) ? " block_table entry outside [0, num_pages);" : "",
              (f & 2u) ? " seq_lens entry outside [T, max_seq_len];" : "",
              (f & 4u) ? " attention index neither -1 nor a visible position;" : "",
              (f & 8u) ? " decode histogram-clear handshake timed out, the rows concerned were written as -1 "
                         "(workspace shared by overlapping calls?);" : "");
}

size_t dsa_indexer_workspace_size(const dsa_paged_layout* layout, const dsa_indexer_shape* shape) {
  if (check_indexer_shape(shape) != DSA_OK || check_layout(layout, shape->T) != DSA_OK) return 0;
  return dsa::plan_indexer(*layout, *shape).total;
}

dsa_status dsa_indexer_topk(const void* q, const void* q_scale, const float* w, const void* k_cache,
                            const void* k_scale, const dsa_paged_layout* layout,
                            const dsa_indexer_shape* shape, int32_t* idx_out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  dsa_status st = check_indexer_shape(shape);
  if (st != DSA_OK) return st;
  if ((st = check_layout(layout, shape->T)) != DSA_OK) return st;
  const bool fp8 = shape->dtype == DSA_FP8_E4M3;
  const bool mx = shape->dtype == DSA_MXFP8_E4M3;
  if (q == nullptr || w == nullptr || k_cache == nullptr || idx_out == nullptr)
    return fail(DSA_ERR_NULL, "q / w / k_cache / idx_out is NULL");
  if ((fp8 || mx) && (q_scale == nullptr || k_scale == nullptr))
    return fail(DSA_ERR_NULL, "fp8 and MXFP8 indexers need q_scale and k_scale");
  if (!fp8 && !mx && (q_scale != nullptr || k_scale != nullptr))
    return fail(DSA_ERR_SHAPE, "q_scale / k_scale must be NULL for the bf16 indexer");
  if (mx && !dsa::indexer_mx_supported(layout->batch, shape->T))
    return fail(DSA_ERR_UNSUPPORTED, "no MXFP8 indexer path for T %d, batch %d", shape->T, layout->batch);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(w, 4) || !aligned(idx_out, 4) ||
      (fp8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4))) || (mx && !aligned(k_scale, 16)))
    return fail(DSA_ERR_ALIGN, "q / k_cache need 16-byte alignment, w / idx_out 4-byte, fp8 scales 4-byte, "
                "MXFP8 k_scale 16-byte");
  const dsa::IndexerPlan plan = dsa::plan_indexer(*layout, *shape);
  if (workspace == nullptr || workspace_bytes < plan.total)
    return fail(DSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, plan.total);
  if (!aligned(workspace, 256)) return fail(DSA_ERR_ALIGN, "workspace must be 256-byte aligned");

  dsa::IndexerArgs a;
  a.q = q; a.q_scale = q_scale; a.w = w; a.k_cache = k_cache; a.k_scale = k_scale;
  a.block_table = layout->block_table; a.seq_lens = layout->seq_lens;
  a.B = layout->batch; a.T = shape->T; a.max_pages = layout->max_pages; a.num_pages = layout->num_pages;
  a.max_seq_len = layout->max_seq_len;
  a.heads = shape->heads; a.dim = shape->dim; a.top_k = shape->top_k; a.fp8 = fp8; a.mx = mx;
  a.idx_out = idx_out; a.workspace = workspace;
  const hipError_t e = dsa::launch_indexer(a, plan, stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "indexer launch: %s", hipGetErrorString(e));
  return DSA_OK;
}

// One thread per 32-element group, 256 per block: the grid's block count must fit 31 bits.
static constexpr long long kMaxQuantGroups = 256LL * 0x7FFFFFFFLL;

dsa_status dsa_mxfp8_quantize(const void* x, int64_t rows, int32_t dim, void* codes, void* scales,
                              hipStream_t stream) {
  if (x == nullptr || codes == nullptr || scales == nullptr)
    return fail(DSA_ERR_NULL, "x / codes / scales is NULL");
  if (rows < 0) return fail(DSA_ERR_SHAPE, "rows %lld < 0", (long long)rows);
  if (dim < 32 || dim > 4096 || dim % 32 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "dim %d unsupported (a multiple of 32, 32..4096)", dim);
  if (!aligned(x, 16) || !aligned(codes, 16)) return fail(DSA_ERR_ALIGN, "x / codes need 16-byte alignment");
  if (rows > kMaxQuantGroups / (dim / 32)) return fail(DSA_ERR_SHAPE, "rows %lld too large", (long long)rows);
  dsa::QuantLaunch q;
  q.src = x; q.codes = codes; q.scales = scales; q.rows = rows; q.dim = dim;
  const hipError_t e = dsa::launch_mx_quant(q, stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "quantise launch: %s", hipGetErrorString(e));
  return DSA_OK;
}

dsa_status dsa_indexer_cache_append(const void* k_new, const dsa_paged_layout* layout, int32_t T,
                                    int32_t dim, void* k_cache, void* k_scale, hipStream_t stream) {
  if (T < 1) return fail(DSA_ERR_SHAPE, "T %d < 1", T);
  dsa_status st = check_layout(layout, T);
  if (st != DSA_OK) return st;
  if (k_new == nullptr || k_cache == nullptr || k_scale == nullptr)
    return fail(DSA_ERR_NULL, "k_new / k_cache / k_scale is NULL");
  if (dim < 32 || dim > 4096 || dim % 32 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "dim %d unsupported (a multiple of 32, 32..4096)", dim);
  if (!aligned(k_new, 16) || !aligned(k_cache, 16)) return fail(DSA_ERR_ALIGN, "k_new / k_cache need 16-byte alignment");
  if ((long long)layout->batch * T > kMaxQuantGroups / (dim / 32))
    return fail(DSA_ERR_SHAPE, "batch * T = %lld rows too large", (long long)layout->batch * T);
  dsa::QuantLaunch q;
  q.src = k_new; q.codes = k_cache; q.scales = k_scale;
  q.block_table = layout->block_table; q.seq_lens = layout->seq_lens;
  q.rows = (long long)layout->batch * T; q.dim = dim; q.T = T;
  q.max_pages = layout->max_pages; q.num_pages = layout->num_pages; q.max_seq_len = layout->max_seq_len;
  q.paged = true;
  const hipError_t e = dsa::launch_mx_quant(q, stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "cache append launch: %s", hipGetErrorString(e));
  return DSA_OK;
}

dsa_status dsa_indexer_cache_append_fp8(const void* k_new, const dsa_paged_layout* layout, int32_t T,
                                        int32_t dim, void* k_cache, float* k_scale, hipStream_t stream) {
  if (T < 1) return fail(DSA_ERR_SHAPE, "T %d < 1", T);
  dsa_status st = check_layout(layout, T);
  if (st != DSA_OK) return st;
  if (k_new == nullptr || k_cache == nullptr || k_scale == nullptr)
    return fail(DSA_ERR_NULL, "k_new / k_cache / k_scale is NULL");
  if (dim != 64 && dim != 128) return fail(DSA_ERR_UNSUPPORTED, "dim %d unsupported (64 or 128)", dim);
  if (!aligned(k_new, 16) || !aligned(k_cache, 16) || !aligned(k_scale, 4))
    return fail(DSA_ERR_ALIGN, "k_new / k_cache need 16-byte alignment, k_scale 4-byte");
  const long long span = (T + 62) / 64 + 1;           // pages one sequence's T keys can reach
  if ((long long)layout->batch * T > 0x7FFFFFFFLL || (long long)layout->batch * span > 0x7FFFFFFFLL)
    return fail(DSA_ERR_SHAPE, "batch * T exceeds 2^31 - 1");
  dsa::Fp8PageLaunch q;
  q.src = k_new; q.codes = k_cache; q.scales = k_scale;
  q.block_table = layout->block_table; q.seq_lens = layout->seq_lens;
  q.batch = layout->batch; q.T = T; q.dim = dim;
  q.max_pages = layout->max_pages; q.num_pages = layout->num_pages; q.max_seq_len = layout->max_seq_len;
  const hipError_t e = dsa::launch_fp8_page_append(q, stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "fp8 cache append launch: %s", hipGetErrorString(e));
  return DSA_OK;
}

dsa_status dsa_fp8_quantize_heads(const void* x, int64_t rows, int32_t dim, void* codes, float* scales,
                                  hipStream_t stream) {
  if (rows < 0) return fail(DSA_ERR_SHAPE, "rows %lld < 0", (long long)rows);
  if (rows > 0x7FFFFFFFLL) return fail(DSA_ERR_SHAPE, "rows %lld too large", (long long)rows);
  if (dim != 64 && dim != 128) return fail(DSA_ERR_UNSUPPORTED, "dim %d unsupported (64 or 128)", dim);
  if (rows == 0) return DSA_OK;
  if (x == nullptr || codes == nullptr || scales == nullptr) return fail(DSA_ERR_NULL, "x / codes / scales is NULL");
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return fail(DSA_ERR_ALIGN, "x / codes need 16-byte alignment, scales 4-byte");
  const hipError_t e = dsa::launch_fp8_heads(x, rows, dim, codes, scales, stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "fp8 head quantisation launch: %s", hipGetErrorString(e));
  return DSA_OK;
}

dsa_status dsa_latent_cache_append_fp8(const void* kv_new, const dsa_paged_layout* layout, int32_t T,
                                       void* kv_codes, float* kv_scale, hipStream_t stream) {
  if (T < 1) return fail(DSA_ERR_SHAPE, "T %d < 1", T);
  dsa_status st = check_layout(layout, T);
  if (st != DSA_OK) return st;
  if (kv_new == nullptr || kv_codes == nullptr || kv_scale == nullptr)
    return fail(DSA_ERR_NULL, "kv_new / kv_codes / kv_scale is NULL");
  if (!aligned(kv_new, 16) || !aligned(kv_codes, 16) || !aligned(kv_scale, 16))
    return fail(DSA_ERR_ALIGN, "kv_new / kv_codes / kv_scale need 16-byte alignment");
  if ((long long)layout->batch * T > 0x7FFFFFFFLL) return fail(DSA_ERR_SHAPE, "batch * T exceeds 2^31 - 1");
  dsa::Kv8Launch q;
  q.src = kv_new; q.codes = kv_codes; q.scales = kv_scale;
  q.block_table = layout->block_table; q.seq_lens = layout->seq_lens;
  q.rows = (long long)layout->batch * T; q.T = T;
  q.max_pages = layout->max_pages; q.num_pages = layout->num_pages; q.max_seq_len = layout->max_seq_len;
  const hipError_t e = dsa::launch_kv8_append(q, stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "latent cache append launch: %s", hipGetErrorString(e));
  return DSA_OK;
}

size_t dsa_sparse_attn_workspace_size(const dsa_paged_layout* layout, const dsa_attn_shape* shape) {
  if (check_attn_shape(shape) != DSA_OK || check_layout(layout, shape->T) != DSA_OK) return 0;
  return dsa::plan_attn(*layout, *shape).total;
}

static dsa_status sparse_attn_impl(const void* q, const void* kv_cache, const float* kv_scale, bool kv8,
                                   const int32_t* idx, const dsa_paged_layout* layout,
                                   const dsa_attn_shape* shape, void* out, float* lse, void* workspace,
                                   size_t workspace_bytes, bool own_scratch, hipStream_t stream) {
  dsa_status st = check_attn_shape(shape);
  if (st != DSA_OK) return st;
  if ((st = check_layout(layout, shape->T)) != DSA_OK) return st;
  if (q == nullptr || kv_cache == nullptr || idx == nullptr || out == nullptr)
    return fail(DSA_ERR_NULL, "q / kv_cache / idx / out is NULL");
  if (kv8 && kv_scale == nullptr) return fail(DSA_ERR_NULL, "kv_scale is NULL");
  if (!aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(out, 16) || !aligned(idx, 4) ||
      (lse != nullptr && !aligned(lse, 4)) || (kv8 && !aligned(kv_scale, 16)))
    return fail(DSA_ERR_ALIGN, "q / kv_cache / out / kv_scale need 16-byte alignment, idx / lse 4-byte");
  const dsa::AttnPlan plan = dsa::plan_attn(*layout, *shape);
  if (own_scratch) {
    // the library's static per-device scratch stands in for the caller's workspace
    if (plan.total > dsa::attn_scratch_bytes())
      return fail(DSA_ERR_WORKSPACE, "this shape needs %zu bytes of scratch; the library holds %zu",
                  plan.total, dsa::attn_scratch_bytes());
    workspace = nullptr;
    if (plan.total > 0) {
      const hipError_t e = dsa::attn_scratch(&workspace);
      if (e != hipSuccess) return fail(DSA_ERR_HIP, "resolving the scratch address: %s", hipGetErrorString(e));
    }
  } else if (plan.total > 0) {
    if (workspace == nullptr || workspace_bytes < plan.total)
      return fail(DSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, plan.total);
    if (!aligned(workspace, 256)) return fail(DSA_ERR_ALIGN, "workspace must be 256-byte aligned");
  }
  dsa::AttnArgs a;
  a.q = q; a.kv_cache = kv_cache; a.kv_scale = kv8 ? kv_scale : nullptr; a.idx = idx;
  a.block_table = layout->block_table; a.seq_lens = layout->seq_lens;
  a.B = layout->batch; a.T = shape->T; a.max_pages = layout->max_pages; a.num_pages = layout->num_pages;
  a.max_seq_len = layout->max_seq_len;
  a.heads = shape->heads; a.top_k = shape->top_k; a.sm_scale = shape->sm_scale;
  a.out = out; a.lse = lse; a.workspace = workspace;
  const hipError_t e = dsa::launch_attn(a, plan, stream);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  return DSA_OK;
}

dsa_status dsa_sparse_attn(const void* q, const void* kv_cache, const int32_t* idx,
                           const dsa_paged_layout* layout, const dsa_attn_shape* shape, void* out,
                           float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return sparse_attn_impl(q, kv_cache, nullptr, false, idx, layout, shape, out, lse, workspace,
                          workspace_bytes, false, stream);
}

dsa_status dsa_sparse_attn_noalloc(const void* q, const void* kv_cache, const int32_t* idx,
                                   const dsa_paged_layout* layout, const dsa_attn_shape* shape,
                                   void* out, float* lse, hipStream_t stream) {
  return sparse_attn_impl(q, kv_cache, nullptr, false, idx, layout, shape, out, lse, nullptr, 0, true,
                          stream);
}

dsa_status dsa_sparse_attn_fp8kv(const void* q, const void* kv_codes, const float* kv_scale,
                                 const int32_t* idx, const dsa_paged_layout* layout,
                                 const dsa_attn_shape* shape, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return sparse_attn_impl(q, kv_codes, kv_scale, true, idx, layout, shape, out, lse, workspace,
                          workspace_bytes, false, stream);
}

}  // extern "C"
