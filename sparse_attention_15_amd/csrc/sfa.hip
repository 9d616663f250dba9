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
#include <type_traits>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kBK = 32;                 // selected rows per tile
constexpr int kRowBytes = kDimQK * 2;   // 1152
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

// LDS layout of a gathered tile: 32 rows of 1152 bytes (72 chunks of 16 bytes), no padding; the
// 16-byte chunk c of row r is stored at chunk c ^ swz(r).  swz keeps both read patterns free of
// bank conflicts: 16 rows reading the same chunk (the score product's A operand) land on 16
// distinct 16-byte bank slots, and the transposed 8-byte reads of the value product (8 rows x 64
// bytes) put at most two requests on a slot.  XOR on the low three bits keeps a chunk inside its
// aligned group of eight, so every swizzled chunk stays inside the 72-chunk row.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 3) | ((((r >> 2) ^ (r >> 3)) & 1) << 2); }

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two floats to packed bf16 (round to nearest even) with gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

constexpr int kTileBytes = kBK * kRowBytes;          // 36864
constexpr int kDmaPerTile = kTileBytes / 1024;       // 36 wave-wide 16-byte-per-lane loads
constexpr int kStages = 3;                           // gather ring depth (the main loop is unrolled by it)
constexpr int kMaxSplitKeys = DSA_MAX_TOP_K;

template <int NW, int W>
__device__ __forceinline__ void wait_tile_dma(bool next_pending) {
  // loads this wave issues per tile; the ring keeps at most one later tile in flight
  constexpr int n = (kDmaPerTile - W + NW - 1) / NW;
  if (next_pending) wait_vmcnt<n>(); else wait_vmcnt<0>();
}

template <int NW>
__device__ __forceinline__ void wait_tile(int wave, bool next_pending) {
  // dispatch the per-wave count to an immediate
  if constexpr (NW == 8) {
    if (wave < kDmaPerTile % 8) wait_tile_dma<8, 0>(next_pending); else wait_tile_dma<8, 7>(next_pending);
  } else if constexpr (NW == 6) {
    wait_tile_dma<6, 0>(next_pending);
  } else if constexpr (NW == 4) {
    wait_tile_dma<4, 0>(next_pending);
  } else {
    wait_tile_dma<2, 0>(next_pending);
  }
}

template <int NG>
__global__ __launch_bounds__(NG * 128) void sfa_main(SfaArgs a) {
  constexpr int NT = NG * 128;              // two waves per 32-head group
  constexpr int NW = NG * 2;
  static_assert(kDmaPerTile % NW == 0 || NW == 8, "per-wave load count must be uniform or split 2-way");
  __shared__ __attribute__((aligned(1024))) unsigned char lds_kv[kStages][kTileBytes];
  __shared__ __attribute__((aligned(16))) float lds_sx[NG * 2 * 16 * 64];   // partial-score exchange
  __shared__ int lds_rows[kMaxSplitKeys];   // physical row of each selected index, -1 = skip

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 31, hh = lane >> 5;
  const int g = wave % NG, hf = wave / NG;  // head group, half (of the contraction / of V)
  const int row = blockIdx.x, split = blockIdx.y;
  const int NGT = (a.H + 31) / 32;          // 32-head groups over all workgroups of a row
  const int gg = blockIdx.z * NG + g;       // this wave's global head group
  const int b = row / a.T, t = row % a.T;
  const int n = row_visible(a.seq_lens, b, a.T, t, a.max_seq_len);
  const int k_begin = split * a.keys_per_split;
  const int k_end = min(a.K, k_begin + a.keys_per_split);
  const int nkeys = k_end - k_begin;
  const int ntiles = (nkeys + kBK - 1) / kBK;
  const int head = gg * 32 + nl;
  const bool hvalid = head < a.H;

  // row table for this split (one round of idx + block-table loads for the whole split)
  {
    const int32_t* idx = a.idx + (size_t)row * a.K + k_begin;
    const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
    for (int j = tid; j < ntiles * kBK; j += NT) {
      int r = -1;
      if (j < nkeys) {
        const int s = idx[j];
        if (s >= 0 && s < n) r = clamp_page(bt[s / kPage], a.num_pages) * kPage + (s % kPage);
      }
      lds_rows[j] = r;
    }
  }
  __syncthreads();

  // gather tile `tile` into ring slot `buf`: this wave's loads are chunks 64*q + lane of the tile,
  // q = wave, wave + NW, ...; slot position p holds row p / 72, chunk (p % 72) ^ swz(row)
  constexpr int kDmaMax = (kDmaPerTile + NW - 1) / NW;
  auto issue = [&](int tile, int buf) {
#pragma unroll
    for (int u = 0; u < kDmaMax; ++u) {
      const int q = wave + u * NW;
      if (q < kDmaPerTile) {
        const int p = 64 * q + lane;
        const int r = p / 72;
        const int c = (p % 72) ^ swz(r);
        const int prow = lds_rows[tile * kBK + r];
        const unsigned char* src = a.kv + (size_t)(prow < 0 ? 0 : prow) * kRowBytes + 16 * c;
        __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_kv[buf] + 1024 * q), 16, 0, 0);
      }
    }
  };

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
  // running max in log2 units; a finite floor keeps masked (-inf) logits at probability 0
  // without special cases (the first valid tile always moves the reference)
  float m_run = -1e30f, l_run = 0.f;

  float* sx_mine = lds_sx + ((g * 2 + hf) * 16) * 64 + lane;
  const float* sx_other = lds_sx + ((g * 2 + (hf ^ 1)) * 16) * 64 + lane;

  // Per-lane LDS byte offsets.  XOR with swz() only touches the low three bits of a chunk index,
  // so offsets repeat every 8 chunks: four bases per operand plus immediate strides cover a tile.
  // Score A operand: row nl, chunk c = 36*hf + 2*ks + hh; ks = 4u + v -> base[v] + 128*u.
  int qk_off[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int c = 36 * hf + 2 * v + hh;
    qk_off[v] = nl * kRowBytes + 16 * ((c & ~7) | ((c & 7) ^ swz(nl)));
  }
  // Value A operand (transposed reads): key = 16*k2 + 8*q + kq, column = dim0 + 32*mb with
  // mb = 2u + v; swz(key) = swz(kq) ^ 4q, so the offset is base[q][v] + 16*8*u + 16*kRowBytes*k2.
  const int kq = 4 * hh + ((lane & 15) >> 2);
  const int dim0 = hf * (kDimV / 2) + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  int pv_off[2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int key = 8 * q + kq;
      const int c = (dim0 >> 3) + 4 * v;
      pv_off[q][v] = key * kRowBytes + 16 * ((c & ~7) | ((c & 7) ^ swz(key))) + 2 * (dim0 & 7);
    }

  // One tile of the main loop.  The ring slot is a compile-time constant (the loop is unrolled by
  // the ring depth), so every LDS address below is a per-lane base plus an immediate offset.
  auto step = [&](int it, auto slot) {
    constexpr int buf = decltype(slot)::value;
    wait_tile<NW>(wave, it + 1 < ntiles);
    lds_barrier();                          // tile `it` landed for every wave; slot it+2 is free
    if (it + 2 < ntiles) issue(it + 2, (buf + 2) % kStages);
    const unsigned char* tile = lds_kv[buf];
    const uint32_t valid = (uint32_t)__ballot(lane < kBK && lds_rows[it * kBK + (lane & 31)] >= 0);

    // partial S^T = X q^T over this wave's 288 columns: rows = the tile's 32 keys, cols = heads
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kQSteps / 2; ++ks) {
      const bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4*>(tile + qk_off[ks & 3] + 128 * (ks >> 2)));
      s = mfma_bf16(af, qf[ks], s);
      if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);   // bound the LDS reads in flight
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sx_mine[r * 64] = s[r];
    lds_barrier();
    // both waves of the pair form the same full score (one addition of the two halves, which is
    // commutative, so both waves get the same bits)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] += sx_other[r * 64];

    // online softmax over the 16 keys this lane holds (+ the other half-wave's 16)
    float mx = -INFINITY;
    if (valid == 0xFFFFFFFFu) {             // wave-uniform: every key of the tile is selected
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] *= a.scale_log2;
        mx = fmaxf(mx, s[r]);
      }
    } else {
      const uint32_t vmask = valid >> (4 * hh);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + (r & 3);        // + 4*hh, folded into `vmask`
        s[r] = ((vmask >> key) & 1u) ? s[r] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazy rescale: the reference max moves only when a logit exceeds it by more than 2^8, so
    // probabilities stay <= 256 and the accumulator is rescaled rarely (exact either way, the
    // final normalisation uses the same reference).
    const bool grow = mx > m_run + kRescaleLog2;
    if (__any(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;   // first tile: 0
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
      s[r] = __builtin_amdgcn_exp2f(s[r] - m_run);
      psum += s[r];
    }
    psum += __shfl_xor(psum, 32, 64);
    l_run += psum;
    // P^T as the B operand of the value product: K step k2 covers keys 16*k2 .. 16*k2 + 15; this
    // lane's 8 values are keys 16*k2 + {0..3, 8..11} + 4*hh (accumulator rows of the score tile)
    bf16x8 pf[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = pack_bf16(s[8 * k2 + 2 * e], s[8 * k2 + 2 * e + 1]);
      pf[k2] = as_bf16x8(v);
    }
    // O^T += V^T P^T over this wave's 256 latent columns.  The A operand (latent column m, the
    // same 8 keys) comes from two transposed reads of the row-major tile: a 16-lane group reading
    // 8 bytes (4 columns) of 4 consecutive keys hands lane i the 4 keys of column i.
    // consecutive MFMAs go to different accumulators (block-major inner loop)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
      for (int mb = 0; mb < kVBlocks / 2; ++mb) {
        s16x4 part[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          part[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(
              tile + pv_off[q][mb & 1] + 128 * (mb >> 1) + 16 * kRowBytes * k2));
        }
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
        o[mb] = mfma_bf16(vf, pf[k2], o[mb]);
        if ((mb & 1) == 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  if (ntiles > 0) issue(0, 0);
  if (ntiles > 1) issue(1, 1);
  for (int it = 0; it < ntiles; it += kStages) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntiles) step(it + 1, std::integral_constant<int, 1>{});
    if (it + 2 < ntiles) step(it + 2, std::integral_constant<int, 2>{});
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
          v.x = pack_bf16(o[mb][4 * j] * inv, o[mb][4 * j + 1] * inv);
          v.y = pack_bf16(o[mb][4 * j + 2] * inv, o[mb][4 * j + 3] * inv);
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
    // partial O in the accumulator's own lane order: [half][head group][block][register][lane]
    if (gg >= NGT) return;
    float* dst = a.part_o + (((ps * 2 + hf) * NGT + gg) * (kVBlocks / 2)) * 16 * 64;
#pragma unroll
    for (int mb = 0; mb < kVBlocks / 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(mb * 16 + r) * 64 + lane] = o[mb][r];
  }
}

// Merges the split partials.  Grid (query row, 32-head group, chunk): each of the 16 chunks of a
// (row, group) handles 1024 of its 16384 partial-O floats, 4 consecutive accumulator lanes per
// thread; every workgroup first rebuilds the per-head merge weights of its group.
constexpr int kCombineChunks = 16;

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
  const int row = blockIdx.x, g = blockIdx.y, chunk = blockIdx.z;
  const int S = a.n_splits, NG = a.waves;
  if (tid < 32) {
    const int head = g * 32 + tid;
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
    if (a.lse != nullptr && head < a.H && chunk == 0)
      a.lse[(size_t)row * a.H + head] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  // this thread's 4 floats: e = index into the group's [hf][mb][r][lane] block of 16384 floats
  const int e = (chunk * 256 + tid) * 4;
  const int lane0 = e & 63, r = (e >> 6) & 15, mb = (e >> 10) & 7, hf = e >> 13;
  const size_t blk = (size_t)(hf * NG + g) * (kVBlocks / 2) * 16 * 64 + (size_t)(mb * 16 + r) * 64 + lane0;
  const size_t per_split = (size_t)2 * NG * (kVBlocks / 2) * 16 * 64;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* src = a.part_o + (size_t)row * S * per_split + blk;
  const int nl0 = lane0 & 31, hh = lane0 >> 5;
  for (int sp = 0; sp < S; ++sp) {
    const float4 v = *reinterpret_cast<const float4*>(src + sp * per_split);
    acc.x += wgt[sp][nl0] * v.x;
    acc.y += wgt[sp][nl0 + 1] * v.y;
    acc.z += wgt[sp][nl0 + 2] * v.z;
    acc.w += wgt[sp][nl0 + 3] * v.w;
  }
  const int d = 256 * hf + 32 * mb + 8 * (r >> 2) + 4 * hh + (r & 3);
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
  const float vals[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int head = g * 32 + nl0 + q;
    if (head < a.H) out[((size_t)row * a.H + head) * kDimV + d] = bf16_bits_rne(vals[q] * inv_l[nl0 + q]);
  }
}

// ------------------------------------------------------------------------------------------------
static size_t align_up(size_t x, size_t al) { return (x + al - 1) / al * al; }

AttnPlan plan_attn(const dsa_paged_layout& L, const dsa_attn_shape& S) {
  AttnPlan p;
  p.waves = (S.heads + 31) / 32;                       // 32-head groups
  p.groups_per_wg = p.waves >= 2 ? 2 : 1;
  p.head_chunks = (p.waves + p.groups_per_wg - 1) / p.groups_per_wg;
  const int rows = L.batch * S.T;
  // splits: enough workgroups (rows x head chunks x splits) to cover the GPU's 256 compute units,
  // at most 64 splits, each holding a whole number of 32-row tiles
  const int tiles = (S.top_k + kBK - 1) / kBK;
  const int per_split = std::max(rows * p.head_chunks, 1);
  int splits = (256 + per_split - 1) / per_split;
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
  const dim3 grid(rows, p.n_splits, p.head_chunks);
  {
    LaunchScope ls("sfa_main", st);
    if (p.groups_per_wg == 2) hipLaunchKernelGGL(sfa_main<2>, grid, dim3(256), 0, st, s);
    else hipLaunchKernelGGL(sfa_main<1>, grid, dim3(128), 0, st, s);
  }
  if (p.n_splits > 1) {
    LaunchScope ls("sfa_combine", st);
    CombineArgs c;
    c.part_ml = s.part_ml; c.part_o = s.part_o; c.out = s.out; c.lse = a.lse;
    c.H = a.heads; c.n_splits = p.n_splits; c.waves = p.waves;
    hipLaunchKernelGGL(sfa_combine, dim3(rows, p.waves, kCombineChunks), dim3(256), 0, st, c);
  }
  return hipGetLastError();
}

}  // namespace dsa
