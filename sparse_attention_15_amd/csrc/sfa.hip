// sfa.hip -- Sparse Flash Attention over the selected MLA latent rows, for gfx950.
//
// Pages: "Inference Optimization for Kimi K3.1 Pro" §1 (DSA step 3: attend over the KV rows at
// the indexer's selected positions) and §2 (indices resolve to pages in place); "Optimizing Kimi
// K3.1 Pro Sparse Attention Inference", "Inheritance and Extension of Core Operators" (blockwise
// attention over fixed-size KV blocks, reduced across blocks without a global softmax).
//
// One workgroup handles one query row, up to 128 heads (32 per wave) and a contiguous range of
// the row's selected indices (a "split").  Per 32-index tile it gathers the 1152-byte latent rows
// (page-table resolved) into LDS twice: row-major for the score product and transposed (first
// 512 columns) for the value product.  With the key tile as MFMA operand A and the wave's query
// rows (held in registers) as operand B it computes S^T = X q^T, so each lane ends up owning one
// head and 16 keys: the online-softmax row max and sum need one cross-half exchange, and the
// probabilities feed the value product O^T += V^T P^T as operand B without leaving the lane.  The
// accumulator O^T (512 x 32 per wave) stays in registers; the running max is kept in the log2
// domain (exp2 with log2(e) folded into the scale).  With one split the workgroup normalises and
// writes bf16 output and the natural-log LSE; with several, each writes (m, l, O) partials and
// sfa_combine merges them: M = max m_i, O = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i.
#include <algorithm>
#include <cmath>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kBK = 32;                 // selected rows per tile
constexpr int kRowBytes = kDimQK * 2;   // 1152
constexpr int kKvStride = kRowBytes + 16;   // LDS row stride (bank spread)
constexpr int kVtStride = kBK * 2 + 16;     // LDS bytes per transposed V row (one latent column)
constexpr int kQSteps = kDimQK / 16;        // 36 MFMA K steps for the score product
constexpr int kVBlocks = kDimV / 32;        // 16 M blocks of the value product
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleLog2 = 8.f;        // lazy-rescale threshold (log2 units)

struct SfaArgs {
  const unsigned char* q;       // [rows, H, 576] bf16
  const unsigned char* kv;      // [P, 64, 576] bf16
  const int32_t* idx;           // [rows, K]
  const int32_t* block_table;
  const int32_t* seq_lens;
  __bf16* out;                  // [rows, H, 512]
  float* lse;                   // [rows, H] or null
  float* part_ml;               // [rows, splits, H, 2]
  float* part_o;                // [rows, splits, waves, 16, 16, 64]
  int T, H, K, max_pages, num_pages, n_splits, keys_per_split, max_seq_len;
  float scale_log2;             // sm_scale * log2(e)
};

// key j of a 32-key tile -> column of the transposed V tile, chosen so that the probabilities a
// lane holds after the score product are exactly the B-operand values the value product needs
// (swap bits 2 and 3 of j).
__device__ __forceinline__ int vt_col(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int NG>
__global__ __launch_bounds__(NG * 128) void sfa_main(SfaArgs a) {
  constexpr int NT = NG * 128;              // two waves per 32-head group
  __shared__ __attribute__((aligned(16))) unsigned char lds_kv[kBK * kKvStride];
  __shared__ __attribute__((aligned(16))) unsigned char lds_vt[kDimV * kVtStride];
  __shared__ __attribute__((aligned(16))) float lds_sx[NG * 2 * 16 * 64];   // partial-score exchange
  __shared__ long long lds_off[kBK];
  __shared__ uint32_t lds_valid;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 31, hh = lane >> 5;
  const int g = wave % NG, hf = wave / NG;  // head group, half (of the contraction / of V)
  const int row = blockIdx.x, split = blockIdx.y;
  const int b = row / a.T, t = row % a.T;
  const int n = row_visible(a.seq_lens, b, a.T, t, a.max_seq_len);
  const int k_begin = split * a.keys_per_split;
  const int k_end = min(a.K, k_begin + a.keys_per_split);
  const int head = g * 32 + nl;
  const bool hvalid = head < a.H;

  // B operand of the score product: this lane's head row of q over this wave's half of the
  // 576 latent columns (18 K steps of 16)
  bf16x8 qf[kQSteps / 2];
  {
    const unsigned char* src = a.q + ((size_t)row * a.H + (hvalid ? head : 0)) * kRowBytes +
                               hf * (kRowBytes / 2) + 16 * hh;
    const uint32_t keep = hvalid ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int ks = 0; ks < kQSteps / 2; ++ks) {
      u32x4 v = *reinterpret_cast<const u32x4*>(src + 32 * ks);
      v[0] &= keep; v[1] &= keep; v[2] &= keep; v[3] &= keep;
      qf[ks] = as_bf16x8(v);
    }
  }
  // O^T for this wave's 256 latent columns (8 blocks of 32) x 32 heads
  f32x16 o[kVBlocks / 2];
#pragma unroll
  for (int mb = 0; mb < kVBlocks / 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int32_t* idx = a.idx + (size_t)row * a.K;
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
  float* sx_mine = lds_sx + ((g * 2 + hf) * 16) * 64 + lane;
  const float* sx_0 = lds_sx + ((g * 2 + 0) * 16) * 64 + lane;
  const float* sx_1 = lds_sx + ((g * 2 + 1) * 16) * 64 + lane;

  for (int kb = k_begin; kb < k_end; kb += kBK) {
    if (tid < 64) {
      const int j = kb + tid;
      const int s = (tid < kBK && j < k_end) ? idx[j] : -1;
      long long off = -1;
      if (s >= 0 && s < n)
        off = ((long long)clamp_page(bt[s / kPage], a.num_pages) * kPage + (s % kPage)) * kRowBytes;
      if (tid < kBK) lds_off[tid] = off;
      const unsigned long long vm = __ballot(off >= 0);
      if (tid == 0) lds_valid = (uint32_t)vm;
    }
    __syncthreads();
    // gather: 32 rows x 72 chunks of 16 bytes; consecutive lanes take the same chunk of
    // consecutive rows so the transposed stores spread over the LDS banks
#pragma unroll 1
    for (int i = tid; i < kBK * (kRowBytes / 16); i += NT) {
      const int r = i % kBK, c = i / kBK;
      const long long off = lds_off[r];
      u32x4 v = off >= 0 ? *reinterpret_cast<const u32x4*>(a.kv + off + 16 * c) : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(lds_kv + r * kKvStride + 16 * c) = v;
      if (c < kDimV / 8) {
        const int col = vt_col(r);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t wv = v[e];
          *reinterpret_cast<uint16_t*>(lds_vt + (8 * c + 2 * e) * kVtStride + 2 * col) = (uint16_t)(wv & 0xFFFFu);
          *reinterpret_cast<uint16_t*>(lds_vt + (8 * c + 2 * e + 1) * kVtStride + 2 * col) = (uint16_t)(wv >> 16);
        }
      }
    }
    __syncthreads();

    // partial S^T = X q^T over this wave's 288 columns: rows = the tile's 32 keys, cols = heads
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kQSteps / 2; ++ks) {
      const bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4*>(
          lds_kv + nl * kKvStride + hf * (kRowBytes / 2) + 32 * ks + 16 * hh));
      s = mfma_bf16(af, qf[ks], s);
      if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);   // bound the LDS reads in flight
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sx_mine[r * 64] = s[r];
    __syncthreads();
    // both waves of the pair form the same full score, summing the halves in a fixed order
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = sx_0[r * 64] + sx_1[r * 64];

    // online softmax over the 16 keys this lane holds (+ the other half-wave's 16)
    const uint32_t valid = lds_valid >> (4 * hh);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + (r & 3);          // + 4*hh, folded into `valid`
      s[r] = ((valid >> key) & 1u) ? s[r] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazy rescale: the reference max moves only when a logit exceeds it by more than 2^8, so
    // probabilities stay <= 256 and the accumulator is rescaled rarely (exact either way, the
    // final normalisation uses the same reference).
    const bool grow = mx > m_run + kRescaleLog2;
    if (__any(grow)) {
      const float alpha = grow ? exp2f(m_run - mx) : 1.f;   // m_run = -inf gives 0
      m_run = grow ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < kVBlocks / 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = (m_run == -INFINITY) ? 0.f : exp2f(s[r] - m_run);
      psum += s[r];
    }
    psum += __shfl_xor(psum, 32, 64);
    l_run += psum;
    // P^T as the B operand of the value product: two K steps of 16 keys
    bf16x8 pf[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = (uint32_t)bf16_bits_rne(s[8 * k2 + 2 * e]) | ((uint32_t)bf16_bits_rne(s[8 * k2 + 2 * e + 1]) << 16);
      pf[k2] = as_bf16x8(v);
    }
    // O^T += V^T P^T over this wave's 256 latent columns
#pragma unroll
    for (int mb = 0; mb < kVBlocks / 2; ++mb) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const bf16x8 vf = as_bf16x8(*reinterpret_cast<const u32x4*>(
            lds_vt + (hf * (kDimV / 2) + 32 * mb + nl) * kVtStride + 2 * (16 * k2 + 8 * hh)));
        o[mb] = mfma_bf16(vf, pf[k2], o[mb]);
      }
      if ((mb & 1) == 1) __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }

  if (a.n_splits == 1) {
    if (hvalid) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + ((size_t)row * a.H + head) * kDimV + hf * (kDimV / 2);
#pragma unroll
      for (int mb = 0; mb < kVBlocks / 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * mb + 8 * j + 4 * hh;
          uint2 v;
          v.x = (uint32_t)bf16_bits_rne(o[mb][4 * j] * inv) | ((uint32_t)bf16_bits_rne(o[mb][4 * j + 1] * inv) << 16);
          v.y = (uint32_t)bf16_bits_rne(o[mb][4 * j + 2] * inv) | ((uint32_t)bf16_bits_rne(o[mb][4 * j + 3] * inv) << 16);
          *reinterpret_cast<uint2*>(dst + d) = v;
        }
      if (a.lse != nullptr && hh == 0 && hf == 0)
        a.lse[(size_t)row * a.H + head] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    }
  } else {
    const size_t ps = (size_t)row * a.n_splits + split;
    if (hvalid && hh == 0 && hf == 0) {
      a.part_ml[(ps * a.H + head) * 2] = m_run;
      a.part_ml[(ps * a.H + head) * 2 + 1] = l_run;
    }
    // partial O in the accumulator's own lane order: [wave][block][register][lane]
    float* dst = a.part_o + ((ps * (2 * NG) + wave) * (kVBlocks / 2)) * 16 * 64;
#pragma unroll
    for (int mb = 0; mb < kVBlocks / 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(mb * 16 + r) * 64 + lane] = o[mb][r];
  }
}

// One workgroup per (query row, 32-head group): merges the split partials.
struct CombineArgs {
  const float* part_ml;
  const float* part_o;
  __bf16* out;
  float* lse;
  int H, n_splits, waves;
};

__global__ __launch_bounds__(256) void sfa_combine(CombineArgs a) {
  constexpr int kMaxSplits = 64;
  __shared__ float wgt[kMaxSplits][32];
  __shared__ float inv_l[32];
  const int tid = threadIdx.x;
  const int row = blockIdx.x, wave = blockIdx.y;
  const int S = a.n_splits;
  if (tid < 32) {
    const int head = wave * 32 + tid;
    float M = -INFINITY;
    if (head < a.H)
      for (int i = 0; i < S; ++i) M = fmaxf(M, a.part_ml[(((size_t)row * S + i) * a.H + head) * 2]);
    float L = 0.f;
    for (int i = 0; i < S; ++i) {
      float w = 0.f;
      if (head < a.H && M != -INFINITY) {
        const size_t e = (((size_t)row * S + i) * a.H + head) * 2;
        w = exp2f(a.part_ml[e] - M);
        L += w * a.part_ml[e + 1];
      }
      wgt[i][tid] = w;
    }
    inv_l[tid] = L > 0.f ? 1.f / L : 0.f;
    if (a.lse != nullptr && head < a.H) a.lse[(size_t)row * a.H + head] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  const int NG = a.waves;   // head groups; partials come from 2 waves per group
  for (int i = tid; i < kVBlocks * 16 * 64; i += 256) {
    const int lane = i & 63, r = (i >> 6) & 15, mbg = i >> 10;   // mbg: 0..15 over 512 columns
    const int hf = mbg >> 3, mb = mbg & 7;
    const int nl = lane & 31, hh = lane >> 5;
    const int head = wave * 32 + nl;
    if (head >= a.H) continue;
    float acc = 0.f;
    for (int s = 0; s < S; ++s)
      acc += wgt[s][nl] * a.part_o[((((size_t)row * S + s) * (2 * NG) + hf * NG + wave) * (kVBlocks / 2) * 16 + mb * 16 + r) * 64 + lane];
    const int d = 256 * hf + 32 * mb + 8 * (r >> 2) + 4 * hh + (r & 3);
    out[((size_t)row * a.H + head) * kDimV + d] = bf16_bits_rne(acc * inv_l[nl]);
  }
}

// ------------------------------------------------------------------------------------------------
static size_t align_up(size_t x, size_t al) { return (x + al - 1) / al * al; }

AttnPlan plan_attn(const dsa_paged_layout& L, const dsa_attn_shape& S) {
  AttnPlan p;
  p.waves = (S.heads + 31) / 32;
  const int rows = L.batch * S.T;
  // splits: enough workgroups to cover the GPU's 256 compute units, at most 64, each split
  // holding a whole number of 32-row tiles
  const int tiles = (S.top_k + kBK - 1) / kBK;
  int splits = (256 + rows - 1) / std::max(rows, 1);
  splits = std::max(1, std::min(splits, std::min(64, tiles)));
  const int tiles_per = (tiles + splits - 1) / splits;
  p.keys_per_split = tiles_per * kBK;
  p.n_splits = (tiles + tiles_per - 1) / tiles_per;
  size_t off = 0;
  if (p.n_splits > 1) {
    p.off_ml = off; off = align_up(off + (size_t)rows * p.n_splits * S.heads * 2 * 4, 256);
    p.off_part = off; off = align_up(off + (size_t)rows * p.n_splits * p.waves * kVBlocks * 16 * 64 * 4, 256);  // 2 waves x 8 blocks per group
  }
  p.total = off;
  return p;
}

hipError_t launch_attn(const AttnArgs& a, const AttnPlan& p, hipStream_t st) {
  SfaArgs s;
  s.q = static_cast<const unsigned char*>(a.q);
  s.kv = static_cast<const unsigned char*>(a.kv_cache);
  s.idx = a.idx;
  s.block_table = a.block_table;
  s.seq_lens = a.seq_lens;
  s.out = static_cast<__bf16*>(a.out);
  s.lse = a.lse;
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  s.part_ml = p.n_splits > 1 ? reinterpret_cast<float*>(ws + p.off_ml) : nullptr;
  s.part_o = p.n_splits > 1 ? reinterpret_cast<float*>(ws + p.off_part) : nullptr;
  s.T = a.T; s.H = a.heads; s.K = a.top_k; s.max_pages = a.max_pages; s.num_pages = a.num_pages;
  s.n_splits = p.n_splits; s.keys_per_split = p.keys_per_split; s.max_seq_len = a.max_seq_len;
  s.scale_log2 = a.sm_scale * kLog2e;
  const int rows = a.B * a.T;
  const dim3 grid(rows, p.n_splits);
  {
  LaunchScope ls("sfa_main", st);
  switch (p.waves) {
    case 1: hipLaunchKernelGGL(sfa_main<1>, grid, dim3(128), 0, st, s); break;
    case 2: hipLaunchKernelGGL(sfa_main<2>, grid, dim3(256), 0, st, s); break;
    case 3: hipLaunchKernelGGL(sfa_main<3>, grid, dim3(384), 0, st, s); break;
    case 4: hipLaunchKernelGGL(sfa_main<4>, grid, dim3(512), 0, st, s); break;
    default: return hipErrorInvalidValue;
  }
  }
  if (p.n_splits > 1) {
    LaunchScope ls("sfa_combine", st);
    CombineArgs c;
    c.part_ml = s.part_ml; c.part_o = s.part_o; c.out = s.out; c.lse = a.lse;
    c.H = a.heads; c.n_splits = p.n_splits; c.waves = p.waves;
    hipLaunchKernelGGL(sfa_combine, dim3(rows, p.waves), dim3(256), 0, st, c);
  }
  return hipGetLastError();
}

}  // namespace dsa
