// quant.hip -- MXFP8 quantisation of indexer rows for gfx950: the step that writes the new keys of
// a decode or prefill step into the paged MXFP8 indexer-K cache, and the same quantiser for the
// indexer queries.
//
// Pages: "Inference Optimization for Kimi K3.1 Pro: Decoding Architecture Evolution and Systems
// Engineering Practices" §3 (the indexer prolog produces the indexer q and k and writes k into the
// cache) and §4 (the Lightning Indexer's Q and K in MXFP8); "Day0 Inference Adaptation for
// Next-Gen LLMs" §3.3 (quantised indexer storage).
//
// MXFP8 (OCP Microscaling): each run of 32 consecutive elements of a row shares the E8M0 exponent
// s = floor(log2(max |v|)) - 8 (8 = the largest E4M3 exponent), clamped to [-127, 127], -127 for a
// run of zeros; its elements are v * 2^-s rounded to E4M3 (nearest, ties to even), clamped to
// +-448.  The rescale is exact (a power of two applied to a bf16 value inside the fp32 range) and
// the rounding is the hardware conversion's, in the default round-to-nearest-even mode.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

struct QuantArgs {
  const uint16_t* src;        // bf16 rows [rows, D]
  unsigned char* codes;       // rows: [rows, D]; paged: the K cache [P, 64, D]
  unsigned char* scales;      // rows: [rows, D/32]; paged: [P, 64, D/32]
  const int32_t* block_table; // paged only: [B, max_pages]
  const int32_t* seq_lens;    // paged only: [B], tokens including the T new ones
  long long rows;             // rows of src (paged: B * T)
  int D, T, max_pages, num_pages, max_seq_len;
  bool paged;
};

// Four E4M3 codes of four floats (already within +-448), byte i = element i.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return (uint32_t)v;
}

// One thread per 32-element group.
__global__ __launch_bounds__(256) void mx_quant_rows(QuantArgs a) {
  const int G = a.D / 32;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= a.rows * G) return;
  const long long r = gid / G;
  const int g = (int)(gid % G);
  const u32x4* src = reinterpret_cast<const u32x4*>(a.src + r * a.D + 32 * g);
  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = src[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = __uint_as_float(v[j] << 16);
      x[8 * i + 2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  int s = amax > 0.f ? ilogbf(amax) - 8 : -127;
  s = s < -127 ? -127 : (s > 127 ? 127 : s);
  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = fminf(fmaxf(ldexpf(x[4 * i + j], -s), -448.f), 448.f);
    out[i / 4][i % 4] = e4m3x4(y[0], y[1], y[2], y[3]);
  }
  long long row = r;
  if (a.paged) {
    // token t of sequence b is logical position seq_len - T + t
    const int b = (int)(r / a.T), t = (int)(r % a.T);
    const int n = row_visible(a.seq_lens, b, a.T, t, a.max_seq_len);
    const int pos = n > 0 ? n - 1 : 0;
    const int page = clamp_page(a.block_table[(size_t)b * a.max_pages + pos / kPage], a.num_pages);
    row = (long long)page * kPage + pos % kPage;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(a.codes + row * a.D + 32 * g);
  dst[0] = out[0];
  dst[1] = out[1];
  a.scales[row * G + g] = (unsigned char)(s + 127);
}

hipError_t quant_take_input_flags(uint32_t* flags) {
  uint32_t z = 0;
  hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_input_flags), sizeof(uint32_t), 0, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(g_input_flags), &z, sizeof z, 0, hipMemcpyHostToDevice);
  return e;
}

hipError_t launch_mx_quant(const QuantLaunch& q, hipStream_t st) {
  QuantArgs a;
  a.src = static_cast<const uint16_t*>(q.src);
  a.codes = static_cast<unsigned char*>(q.codes);
  a.scales = static_cast<unsigned char*>(q.scales);
  a.block_table = q.block_table;
  a.seq_lens = q.seq_lens;
  a.rows = q.rows;
  a.D = q.dim; a.T = q.T; a.max_pages = q.max_pages; a.num_pages = q.num_pages;
  a.max_seq_len = q.max_seq_len;
  a.paged = q.paged;
  const long long groups = q.rows * (q.dim / 32);
  if (groups == 0) return hipSuccess;
  const long long blocks = (groups + 255) / 256;
  {
    LaunchScope ls(q.paged ? "mx_cache_append" : "mx_quant_rows", st);
    hipLaunchKernelGGL(mx_quant_rows, dim3((unsigned)blocks), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace dsa
