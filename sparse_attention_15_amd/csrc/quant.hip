// quant.hip -- quantisation kernels of the prolog for gfx950: MXFP8 indexer rows (the step that
// writes the new keys of a decode or prefill step into the paged MXFP8 indexer-K cache, and the
// same quantiser for the indexer queries), the per-page fp8 indexer-K append, the per-head fp8
// query quantiser, and the FP8 latent-row append for the SFA cache.
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
    // a length below T (flagged by row_visible) leaves this token without a slot: store nothing
    // rather than overwrite a valid cached row
    if (n <= 0) return;
    const int pos = n - 1;
    const int page = clamp_page(a.block_table[(size_t)b * a.max_pages + pos / kPage], a.num_pages);
    row = (long long)page * kPage + pos % kPage;
  }
  u32x4* dst = reinterpret_cast<u32x4*>(a.codes + row * a.D + 32 * g);
  dst[0] = out[0];
  dst[1] = out[1];
  a.scales[row * G + g] = (unsigned char)(s + 127);
}

// FP8 latent rows ("Inference Optimization for Kimi K3.1 Pro" §4: the SFA cache in FP8 with
// per-token scales over 128-wide tiles).  Per token and per 128-column tile of the 576-wide row
// (columns 0-127, ..., 384-511 and the rope remainder 512-575): scale = amax / 448 (1 for an
// all-zero tile), codes = E4M3 of x / scale (both divisions rounded to nearest even, the
// conversion nearest even, clamped to +-448).  One wave per 8 rows: for each row lane l holds
// columns 8l..8l+7 of the value part (a value tile's amax is a max over 16 lanes), and lane l also
// holds columns 512 + 8(l % 8).. of row l / 8 (a rope tile's amax is a max over 8 lanes).
struct Kv8Args {
  const uint16_t* src;        // [rows, 576] bf16, row = b * T + t
  unsigned char* codes;       // [P, 64, 576]
  float* scales;              // [P, 64, 8]
  const int32_t* block_table;
  const int32_t* seq_lens;
  long long rows;
  int T, max_pages, num_pages, max_seq_len;
};

__device__ __forceinline__ void bf16x8_to_f32(const u32x4 v, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(v[j] << 16);
    x[2 * j + 1] = __uint_as_float(v[j] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint2 e4m3x8_scaled(const float (&x)[8], float sc) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = fminf(fmaxf(__fdiv_rn(x[i], sc), -448.f), 448.f);
  return make_uint2(e4m3x4(y[0], y[1], y[2], y[3]), e4m3x4(y[4], y[5], y[6], y[7]));
}

constexpr int kKv8RowsPerWave = 8;   // rows per wave: lane l also holds rope chunk l % 8 of row l / 8

// Max over each row of 16 lanes, left in every lane of the row (DPP: swap neighbours, swap pairs,
// rotate the row by 4 and by 8).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true)));
  return v;
}

// Max over each group of 8 lanes (swap neighbours, swap pairs, mirror the half row).
__device__ __forceinline__ float row8_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true)));
  return v;
}

__global__ __launch_bounds__(256) void kv8_append_rows(Kv8Args a) {
  constexpr int RPW = kKv8RowsPerWave;
  const long long r0 = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
  const int lane = threadIdx.x & 63;
  if (r0 >= a.rows) return;                                  // whole waves
  auto row_of = [&](int i) { return (int)(r0 + i < a.rows ? r0 + i : r0); };   // past the end: row r0
  // The table lookups of all rows go out together with the row loads, so a wave waits for memory
  // twice (lengths, then pages and rows), not twice per row.  Rows < 2^31: checked by the host.
  int sl[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) sl[i] = a.seq_lens[row_of(i) / a.T];
  u32x4 v[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) v[i] = *reinterpret_cast<const u32x4*>(a.src + (size_t)row_of(i) * kDimQK + 8 * lane);
  const int ri = lane >> 3;                                  // this lane's rope row and chunk
  const u32x4 vr = *reinterpret_cast<const u32x4*>(a.src + (size_t)row_of(ri) * kDimQK + kDimV + 8 * (lane & 7));
  // token t of sequence b is logical position seq_len - T + t; a length outside [T, cap] is
  // flagged and clamped, as everywhere in the library
  int pg[RPW], slot[RPW];
  bool has_slot[RPW];                 // false for a token whose flagged length leaves it no slot
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int r = row_of(i);
    const int b = r / a.T, t = r % a.T;
    int L = sl[i];
    if (L < a.T || L > a.max_seq_len) {
      flag_input(kFlagLen);
      L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
    }
    const int n = max(L - a.T + t + 1, 0);
    const int pos = n > 0 ? n - 1 : 0;
    has_slot[i] = n > 0;
    pg[i] = a.block_table[(size_t)b * a.max_pages + pos / kPage];
    slot[i] = pos % kPage;
  }
  long long dst_row[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) dst_row[i] = (long long)clamp_page(pg[i], a.num_pages) * kPage + slot[i];

  // rope tiles of the wave's 8 rows, one chunk per lane
  float xr[8];
  bf16x8_to_f32(vr, xr);
  float amr = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amr = fmaxf(amr, fabsf(xr[j]));
  amr = row8_max(amr);
  const float scr = amr > 0.f ? __fdiv_rn(amr, 448.f) : 1.f;
  bool rope_ok = has_slot[0];
#pragma unroll
  for (int i = 1; i < RPW; ++i) rope_ok = ri == i ? has_slot[i] : rope_ok;
  if (r0 + ri < a.rows && rope_ok) {
    long long dr = dst_row[0];
#pragma unroll
    for (int i = 1; i < RPW; ++i) dr = ri == i ? dst_row[i] : dr;
    *reinterpret_cast<uint2*>(a.codes + dr * kDimQK + kDimV + 8 * (lane & 7)) = e4m3x8_scaled(xr, scr);
  }

#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    if (r0 + i >= a.rows) break;                             // wave-uniform
    float x[8];
    bf16x8_to_f32(v[i], x);
    float am = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[j]));
    am = row16_max(am);                                      // lanes 16k..16k+15: value tile k
    const float sc = am > 0.f ? __fdiv_rn(am, 448.f) : 1.f;
    // scale row: value tiles 0-3 (from lanes 0, 16, 32, 48), the rope tile (lane 8i), then 1
    float s_out = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(scr), 8 * i));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float sk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), 16 * k));
      s_out = lane == k ? sk : s_out;
    }
    s_out = lane > 4 ? 1.f : s_out;
    if (!has_slot[i]) continue;                              // wave-uniform
    *reinterpret_cast<uint2*>(a.codes + dst_row[i] * kDimQK + 8 * lane) = e4m3x8_scaled(x, sc);
    if (lane < 8) a.scales[dst_row[i] * 8 + lane] = s_out;
  }
}

// Per-head fp8 queries ("Inference Optimization for Kimi K3.1 Pro" §3: the prolog quantises the
// indexer q; the indexer folds the head weights and these scales together, w * sq, when it loads a
// query row): per head row sq = amax / 448 (1 for an all-zero row), codes = E4M3 of q / sq (both
// divisions nearest even, codes nearest even, clamped to +-448).  D / 8 lanes per head row (a DPP
// max over 8 or 16 lanes), 64 / (D / 8) rows per wave.
struct HeadArgs {
  const uint16_t* src;        // [rows, D] bf16
  unsigned char* codes;       // [rows, D] E4M3
  float* scales;              // [rows]
  long long rows;
};

template <int D>
__global__ __launch_bounds__(256) void fp8_quant_heads(HeadArgs a) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;
  static_assert(LPR == 8 || LPR == 16, "head dims 64 and 128");
  const int lane = threadIdx.x & 63;
  const long long r = ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int c = lane % LPR;
  const bool valid = r < a.rows;
  const long long rr = valid ? r : 0;                        // lanes past the end read row 0
  float x[8];
  bf16x8_to_f32(*reinterpret_cast<const u32x4*>(a.src + rr * D + 8 * c), x);
  float am = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) am = fmaxf(am, fabsf(x[j]));
  am = LPR == 16 ? row16_max(am) : row8_max(am);
  const float sq = am > 0.f ? __fdiv_rn(am, 448.f) : 1.f;
  if (valid) {
    *reinterpret_cast<uint2*>(a.codes + rr * D + 8 * c) = e4m3x8_scaled(x, sq);
    if (c == 0) a.scales[rr] = sq;
  }
}

// Per-page fp8 indexer-K append ("Inference Optimization for Kimi K3.1 Pro" §3: the prolog writes
// each step's new keys into the cache; the fp8 indexer keeps one fp32 scale per 64-token page).
// A page's scale only grows: it is the largest |key| the page has received / 448 (fp32 division),
// 1 while the page has received only zeros.  For a page that receives new keys:
//   s = max(s_old, m / 448), m = max |new key element| in the page, s_old = the stored scale if
//   the page already holds keys of the sequence (else 0); s = 1 if that is 0;
//   if s > s_old the held codes are re-encoded as E4M3((e4m3(c) * s_old) / s), each operation
//   rounded to nearest even in fp32; new codes are E4M3(x / s); the page's scale becomes s.
// One 256-thread workgroup per page the append reaches (the span of T keys touches at most
// (T + 62) / 64 + 1 pages of a sequence): a page row of D bf16 is D / 8 16-byte chunks, so thread i
// handles chunks i, i + 256, ... of the page (2 for D = 64, 4 for D = 128), all loads issued
// before the block maximum is taken.
typedef float f32x2_t __attribute__((ext_vector_type(2)));

struct Fp8PageArgs {
  const uint16_t* src;        // [B, T, D] bf16
  unsigned char* codes;       // [P, 64, D] E4M3
  float* scales;              // [P]
  const int32_t* block_table;
  const int32_t* seq_lens;
  int T, span, max_pages, num_pages, max_seq_len;
};

template <int D>
__global__ __launch_bounds__(256) void fp8_page_append(Fp8PageArgs a) {
  constexpr int CPR = D / 8;                   // 16-byte chunks per key row
  constexpr int PER = kPage * CPR / 256;       // chunks per thread
  static_assert(PER * 256 == kPage * CPR, "D = 64 or 128");
  __shared__ float red[4];
  const int b = blockIdx.x / a.span, jj = blockIdx.x % a.span;
  const int L = a.seq_lens[b];
  if (L < a.T || L > a.max_seq_len) {          // no position is certain: write nothing
    if (jj == 0 && threadIdx.x == 0) flag_input(kFlagLen);
    return;
  }
  const int first = L - a.T;                   // logical position of the first new key
  const int j = first / kPage + jj;            // the sequence's page this workgroup writes
  if (j * kPage >= L) return;                  // whole workgroup: the span ends before this page
  const int page = clamp_page(a.block_table[(size_t)b * a.max_pages + j], a.num_pages);
  const int held = max(first - j * kPage, 0);  // slots 0 .. held-1 hold earlier keys
  const int end = min(L - j * kPage, kPage);   // new keys fill slots held .. end-1
  const long long src_row0 = (long long)b * a.T + (j * kPage - first);   // row of slot 0

  u32x4 v[PER];
  float am = 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int c = threadIdx.x + 256 * k, slot = c / CPR, col = c % CPR;
    if (slot >= held && slot < end)
      v[k] = *reinterpret_cast<const u32x4*>(a.src + (size_t)(src_row0 + slot) * D + 8 * col);
  }
  const float s_old = held > 0 ? a.scales[page] : 0.f;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int slot = (threadIdx.x + 256 * k) / CPR;
    if (slot >= held && slot < end) {
      float x[8];
      bf16x8_to_f32(v[k], x);
#pragma unroll
      for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(x[i]));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = fmaxf(s_old, __fdiv_rn(m, 448.f));
  if (s == 0.f) s = 1.f;

  unsigned char* pg = a.codes + (size_t)page * kPage * D;
  if (held > 0 && s > s_old) {                 // workgroup-uniform
    // each chunk of a held slot is read and written by the same thread
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int c = threadIdx.x + 256 * k, slot = c / CPR, col = c % CPR;
      if (slot < held) {
        uint2* q = reinterpret_cast<uint2*>(pg + (size_t)slot * D + 8 * col);
        const uint2 w = *q;
        float x[8];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t word = h ? w.y : w.x;
          const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
          const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
          x[4 * h] = __fmul_rn(lo[0], s_old);
          x[4 * h + 1] = __fmul_rn(lo[1], s_old);
          x[4 * h + 2] = __fmul_rn(hi[0], s_old);
          x[4 * h + 3] = __fmul_rn(hi[1], s_old);
        }
        *q = e4m3x8_scaled(x, s);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int c = threadIdx.x + 256 * k, slot = c / CPR, col = c % CPR;
    if (slot >= held && slot < end) {
      float x[8];
      bf16x8_to_f32(v[k], x);
      *reinterpret_cast<uint2*>(pg + (size_t)slot * D + 8 * col) = e4m3x8_scaled(x, s);
    }
  }
  if (threadIdx.x == 0) a.scales[page] = s;
}

hipError_t launch_fp8_page_append(const Fp8PageLaunch& q, hipStream_t st) {
  if (q.batch == 0) return hipSuccess;
  Fp8PageArgs a;
  a.src = static_cast<const uint16_t*>(q.src);
  a.codes = static_cast<unsigned char*>(q.codes);
  a.scales = q.scales;
  a.block_table = q.block_table;
  a.seq_lens = q.seq_lens;
  a.T = q.T; a.max_pages = q.max_pages; a.num_pages = q.num_pages; a.max_seq_len = q.max_seq_len;
  a.span = (q.T + kPage - 2) / kPage + 1;
  const long long blocks = (long long)q.batch * a.span;
  LaunchScope ls("fp8_page_append", st);
  if (q.dim == 128) hipLaunchKernelGGL(fp8_page_append<128>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(fp8_page_append<64>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fp8_heads(const void* src, long long rows, int dim, void* codes, float* scales,
                            hipStream_t st) {
  if (rows == 0) return hipSuccess;
  HeadArgs a;
  a.src = static_cast<const uint16_t*>(src);
  a.codes = static_cast<unsigned char*>(codes);
  a.scales = scales;
  a.rows = rows;
  const long long per_block = 4LL * (64 / (dim / 8));
  const long long blocks = (rows + per_block - 1) / per_block;
  LaunchScope ls("fp8_quant_heads", st);
  if (dim == 128) hipLaunchKernelGGL(fp8_quant_heads<128>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(fp8_quant_heads<64>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_kv8_append(const Kv8Launch& q, hipStream_t st) {
  Kv8Args a;
  a.src = static_cast<const uint16_t*>(q.src);
  a.codes = static_cast<unsigned char*>(q.codes);
  a.scales = q.scales;
  a.block_table = q.block_table;
  a.seq_lens = q.seq_lens;
  a.rows = q.rows;
  a.T = q.T; a.max_pages = q.max_pages; a.num_pages = q.num_pages; a.max_seq_len = q.max_seq_len;
  if (q.rows == 0) return hipSuccess;
  const long long blocks = (q.rows + 4 * kKv8RowsPerWave - 1) / (4 * kKv8RowsPerWave);
  {
    LaunchScope ls("kv8_cache_append", st);
    hipLaunchKernelGGL(kv8_append_rows, dim3((unsigned)blocks), dim3(256), 0, st, a);
  }
  return hipGetLastError();
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
