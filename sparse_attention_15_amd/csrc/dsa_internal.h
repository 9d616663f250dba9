// dsa_internal.h -- host-side interface between the C ABI (dsa_api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

// Brackets one kernel launch with profiling events when dsa_profile_start() is active.
class LaunchScope {
 public:
  LaunchScope(const char* name, hipStream_t s);
  ~LaunchScope();
  LaunchScope(const LaunchScope&) = delete;
  LaunchScope& operator=(const LaunchScope&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t stop_;
};

// A fresh 64-bit tag per call (never 0): a random start mixed with a call counter (SplitMix64
// finaliser), so a tag that an earlier call left in a workspace cannot match by accident.  Kernels
// that hand work between workgroups mark a handshake word with it.
unsigned long long next_call_tag();

// Workspace carving and grid sizes of one dsa_indexer_topk call.
struct IndexerPlan {
  int rows = 0;          // batch * T query rows
  int row_stride = 0;    // u32 keys per row in the score scratch
  int n_chunks = 0;      // key chunks per sequence in the chunked (prefill) score grid
  int tq = 1;            // query rows sharing one pass over the keys (1, 2 or 4)
  int n_qtiles = 0;      // ceil(T / tq)
  int n_seg = 1;         // select workgroups per row (grid y)
  size_t off_hist = 0, off_keys = 0, off_gt = 0, off_cand = 0, total = 0;
};

struct IndexerArgs {
  const void* q;
  const void* q_scale;    // fp32 per head (fp8) or E8M0 bytes per 32 elements (MXFP8)
  const float* w;
  const void* k_cache;
  const void* k_scale;    // fp32 per page (fp8) or E8M0 bytes per 32 elements (MXFP8)
  const int32_t* block_table;
  const int32_t* seq_lens;
  int B, T, max_pages, num_pages, max_seq_len, heads, dim, top_k;
  bool fp8;              // E4M3 with fp32 per-head / per-page scales
  bool mx;               // MXFP8: E4M3 with E8M0 scales per 32 elements
  int32_t* idx_out;
  void* workspace;
};

// Read and clear the device-side input-check flags of each translation unit (current device).
hipError_t indexer_take_input_flags(uint32_t* flags);
hipError_t attn_take_input_flags(uint32_t* flags);
hipError_t quant_take_input_flags(uint32_t* flags);

// MXFP8 quantisation of bf16 rows (quant.hip): to contiguous rows, or appended to the paged cache.
struct Kv8Launch {
  const void* src;          // [B * T, 576] bf16
  void* codes;              // [P, 64, 576] E4M3
  float* scales;            // [P, 64, 8] fp32
  const int32_t* block_table;
  const int32_t* seq_lens;
  long long rows;
  int T, max_pages, num_pages, max_seq_len;
};
hipError_t launch_kv8_append(const Kv8Launch& q, hipStream_t stream);
struct Fp8PageLaunch {
  const void* src;          // [B, T, dim] bf16
  void* codes;              // [P, 64, dim] E4M3
  float* scales;            // [P] fp32
  const int32_t* block_table;
  const int32_t* seq_lens;
  int batch, T, dim, max_pages, num_pages, max_seq_len;
};
hipError_t launch_fp8_page_append(const Fp8PageLaunch& q, hipStream_t stream);
hipError_t launch_fp8_heads(const void* src, long long rows, int dim, void* codes, float* scales,
                            hipStream_t stream);

struct QuantLaunch {
  const void* src;            // bf16 [rows, dim]
  void* codes;                // E4M3 destination
  void* scales;               // E8M0 destination
  const int32_t* block_table = nullptr;
  const int32_t* seq_lens = nullptr;
  long long rows = 0;
  int dim = 0, T = 1, max_pages = 0, num_pages = 0, max_seq_len = 0;
  bool paged = false;
};
hipError_t launch_mx_quant(const QuantLaunch& q, hipStream_t stream);

IndexerPlan plan_indexer(const dsa_paged_layout& L, const dsa_indexer_shape& S);
bool indexer_supported(int heads, int dim);
bool indexer_mx_supported(int batch, int T);   // the MXFP8 indexer runs the decode path only
hipError_t launch_indexer(const IndexerArgs& a, const IndexerPlan& p, hipStream_t stream);

struct AttnPlan {
  int waves = 1;         // 32-head groups of the row (each handled by a pair of waves)
  int groups_per_wg = 1; // head groups per workgroup
  int head_chunks = 1;   // workgroups per (row, split) along the heads
  int n_splits = 1;      // workgroups per query row along the selected set
  int comb_parts = 1;    // combine workgroups per (row, head group) of a split row
  int keys_per_split = 0;
  size_t off_ml = 0, off_part = 0, off_sync = 0, total = 0;
};

struct AttnArgs {
  const void* q;
  const void* kv_cache;
  const void* kv_scale = nullptr;   // fp8 latent cache: [P, 64, 8] fp32 tile scales; null for bf16
  const int32_t* idx;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int B, T, max_pages, num_pages, max_seq_len, heads, top_k;
  float sm_scale;
  void* out;
  float* lse;
  void* workspace;
};

AttnPlan plan_attn(const dsa_paged_layout& L, const dsa_attn_shape& S);
hipError_t launch_attn(const AttnArgs& a, const AttnPlan& p, hipStream_t stream);

// The attention library's own scratch for callers that cannot allocate: its size, and its device
// address on the current device (resolved on the first call per device, then cached).
constexpr int kMaxDevices = 64;
size_t attn_scratch_bytes();
hipError_t attn_scratch(void** ptr);

}  // namespace dsa
