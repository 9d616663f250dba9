// indexer.hip -- Lightning Indexer with exact Top-K for gfx950.
//
// Pages: "Inference Optimization for Kimi K3.1 Pro: Decoding Architecture Evolution and Systems
// Engineering Practices" §1 (DSA steps 1-2) and §2 (score, head weighting and Top-K fused, only
// indices leave, the paged K cache is addressed in place); "Day0 Inference Adaptation for
// Next-Gen LLMs" §3.1 (bf16 and quantised indexer, prefill and decode).
//
// Score: I[s] = sum_h w[h] * max(0, q[h,:] . k[s,:]) accumulated in fp32 (fp8: the per-head q
// scale folds into w, the per-page k scale multiplies the weighted sum; both are > 0).  Top-K
// keeps the K' = min(K, n) largest scores, ties to the lower position, and writes the positions
// in ascending order, -1 padded.
//
// Kernels, in launch order:
//   li_zero_hist    clears the per-row 2048-bin histograms of the score keys' top 11 bits (prefill
//                   and verify; the decode score kernel clears its rows itself, see there).
//   li_score        one workgroup per (sequence, tile of query rows, chunk of 1024 keys): streams
//                   the chunk's pages (page-table resolved) through LDS, MFMA score GEMM
//                   [heads x dim] x [dim x keys], ReLU and head-weight reduction in registers,
//                   order-preserving u32 keys to the row scratch, LDS histogram -> global.
//   li_select       one workgroup per row: resolves the K'-th key digit by digit (first digit from
//                   the row histogram), stages the positions above the threshold range and the
//                   (key, position) candidates inside it in LDS with one ordered pass over the
//                   row, finishes the threshold in LDS, keeps candidates above it plus the
//                   lowest-position ties up to the quota, and merges both lists into idx_out.
// A row with n <= K selects every visible position and skips the score scratch.
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kTileKeys = 128;    // keys staged in LDS per step (two pages)
constexpr int kChunkKeys = 1024;  // keys per score workgroup
constexpr int kBins = 2048;       // first radix digit: key bits 31..21
// Control words per row, after the histograms: [0..2] the select's counters (segments done, list
// cursors), [4..5] the 64-bit tag that marks the row's histogram cleared for this call (decode),
// [6..7] the poison words: the call's tag when a decode workgroup gave up waiting for that clear.
constexpr int kCtl = 8;
constexpr int kTagWord = 4;
constexpr int kPoisonWord = 6;
constexpr unsigned kSyncSpinCap = 1u << 20;   // waits for a tag end after ~50 ms at most
constexpr int kThreads = 256;

// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void li_zero_hist(uint32_t* __restrict__ hist, size_t n_words) {
  u32x4* p = reinterpret_cast<u32x4*>(hist);
  const size_t n4 = n_words / 4;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

// max(x, 0) as one integer max on the bits: a non-negative float compares as a non-negative
// integer, a negative one as a negative integer (avoids the NaN-quieting fmaxf expansion).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// MXFP8 operands (OCP Microscaling: E4M3 elements, one E8M0 scale 2^(e - 127) per 32 consecutive
// elements) go straight to gfx950's block-scaled MFMA, 32x32x64 with E4M3 A and B.  Its operand
// lanes (checked on the device): for a 64-element chunk of the dot product, lane r + 32h of A
// (row r) or B (column r) holds 32 codes, bytes 0-15 in the chunk's first 32-element block and
// bytes 16-31 in its second; the block's scale comes from byte 0 of the scale operand of lane
// r + 32 * block.  So lane (r, h) takes elements 16h..16h+15 of each 32-element group of the
// chunk and the scale of group h: one E8M0 scale per MX group, no dequantisation.
typedef int mx_i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma_mx(mx_i32x8 a, mx_i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
__device__ __forceinline__ mx_i32x8 mx_join(u32x4 lo, u32x4 hi) {
  return mx_i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// ------------------------------------------------------------------------------------------------
struct ScoreArgs {
  const unsigned char* q;       // [B,T,HI,DI] bf16 | e4m3
  const float* q_scale;         // [B,T,HI] (fp8)
  const float* w;               // [B,T,HI]
  const unsigned char* kc;      // [P,64,DI]
  const float* k_scale;         // [P] (fp8)
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint32_t* keys;               // [rows, row_stride]
  uint32_t* hist;               // [rows, kBins]
  uint32_t* ctl;                // [rows, kCtl] control words
  unsigned long long tag;       // decode: this call's histogram-cleared tag (never 0)
  unsigned spin_cap;            // decode: sleeps before a tag wait gives up
  int withhold_tag;             // decode, test hook: the clearing workgroups publish no tag
  const unsigned char* q_e8;    // MXFP8: [B,T,HI,DI/32] E8M0 scale bytes of q
  const unsigned char* k_e8;    // MXFP8: [P,64,DI/32] E8M0 scale bytes of the K cache
  int B, T, max_pages, num_pages, K, n_chunks, n_qtiles, row_stride, max_seq_len;
};

template <int HI, int DI, bool FP8, int TQ>
struct ScoreCfg {
  static constexpr int MB = (HI + 31) / 32;       // 32-head M blocks
  static constexpr int KS = DI / 16;              // MFMA K steps
  static constexpr int ELT = FP8 ? 1 : 2;         // bytes per element
  static constexpr int ROWB = DI * ELT;           // bytes per key row
  static constexpr int CPK = ROWB / 16;           // 16-byte chunks per key row
  static constexpr int TILEB = kTileKeys * ROWB;  // LDS bytes per tile
  static constexpr int LPT = TILEB / 16 / kThreads;  // 16-byte loads per thread per tile
  static constexpr int WPQ = 4 / TQ;              // waves per query row
  static_assert(CPK >= 4 && (CPK & (CPK - 1)) == 0, "row must be 4..16 chunks");
  static_assert(LPT >= 1, "tile too small");
};

template <bool FP8>
struct AFrag;
template <>
struct AFrag<false> { typedef bf16x8 T; };
template <>
struct AFrag<true> { typedef long T; };

// MX: MXFP8 operands (E4M3 codes, one E8M0 scale per 32 elements) on the 32x32x64 block-scaled MFMA.
template <int HI, int DI, bool FP8, int TQ, bool MX = false>
__global__ __launch_bounds__(256) void li_score(ScoreArgs a) {
  static_assert(!MX || (FP8 && DI % 64 == 0), "MXFP8 keeps E4M3 codes, 64-element MFMA chunks");
  using C = ScoreCfg<HI, DI, FP8, TQ>;
  typedef typename AFrag<FP8>::T frag_t;
  constexpr int NG = DI / 32;                     // MX: scale bytes per key row
  constexpr int NC = DI / 64;                     // MX: 64-element chunks of the dot product
  constexpr int SBT = kTileKeys * NG;             // MX: scale bytes per tile (two pages)
  static_assert(!MX || (SBT % 32 == 0 && SBT / 16 <= kThreads), "tile scale bytes");
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[C::TILEB];
  __shared__ uint32_t lds_hist[TQ * kBins];
  __shared__ float lds_ksc[kTileKeys / kPage];
  __shared__ __attribute__((aligned(16))) unsigned char lds_kx[MX ? SBT : 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 31, hh = lane >> 5;

  int id = blockIdx.x;
  const int chunk = id % a.n_chunks;
  id /= a.n_chunks;
  const int b = id % a.B;
  id /= a.B;
  const int qt = a.n_qtiles - 1 - id;  // longest causal rows first
  const int t0 = qt * TQ;
  const int cap = a.max_seq_len;

  int nmax = 0;
  bool any = false;
#pragma unroll
  for (int i = 0; i < TQ; ++i) {
    const int t = t0 + i;
    const int n = (t < a.T) ? row_visible(a.seq_lens, b, a.T, t, cap) : 0;
    any |= n > a.K;
    nmax = n > nmax ? n : nmax;
  }
  const int s_begin = chunk * kChunkKeys;
  if (!any || s_begin >= nmax) return;
  const int s_end = min(s_begin + kChunkKeys, nmax);

  for (int i = tid; i < TQ * kBins; i += kThreads) lds_hist[i] = 0u;

  // this wave's query row and share of the tile's four 32-key column blocks
  const int qi = wave / C::WPQ, nsub = wave % C::WPQ;
  const int t = t0 + qi;
  const bool qvalid = t < a.T;
  const int tq = qvalid ? t : a.T - 1;
  const int n_me = qvalid ? row_visible(a.seq_lens, b, a.T, t, cap) : 0;
  const bool emit = qvalid && n_me > a.K;
  const size_t row = (size_t)b * a.T + tq;

  // A operand: q rows of this query, held for the whole chunk
  frag_t afrag[MX ? 1 : C::MB][MX ? 1 : C::KS];
  mx_i32x8 amx[MX ? C::MB : 1][MX ? NC : 1];      // MX: q codes of lane (head, h) per chunk
  int asc[MX ? C::MB : 1][MX ? NC : 1];           // MX: their group scales
#pragma unroll
  for (int m = 0; m < C::MB; ++m) {
    const int head = 32 * m + nl;
    if constexpr (MX) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (head < HI) {
          const unsigned char* src = a.q + (row * HI + head) * DI + 64 * c + 16 * hh;
          amx[m][c] = mx_join(*reinterpret_cast<const u32x4*>(src), *reinterpret_cast<const u32x4*>(src + 32));
          asc[m][c] = a.q_e8[(row * HI + head) * NG + 2 * c + hh];
        } else {
          amx[m][c] = mx_i32x8{0, 0, 0, 0, 0, 0, 0, 0};
          asc[m][c] = 127;
        }
      }
      continue;
    }
#pragma unroll
    for (int kk = 0; kk < C::KS; ++kk) {
      if (head < HI) {
        const unsigned char* src = a.q + ((row * HI + head) * DI + 16 * kk + 8 * hh) * C::ELT;
        if constexpr (FP8) afrag[m][kk] = *reinterpret_cast<const long*>(src);
        else afrag[m][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(src));
      } else {
        if constexpr (FP8) afrag[m][kk] = 0;
        else afrag[m][kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      }
    }
  }
  // head weights in accumulator-row order (fp8: times the per-head q scale)
  float wreg[C::MB][16];
#pragma unroll
  for (int m = 0; m < C::MB; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int head = 32 * m + 8 * (r >> 2) + 4 * hh + (r & 3);
      float wv = 0.f;
      if (head < HI) {
        wv = a.w[row * HI + head];
        if constexpr (FP8 && !MX) wv *= a.q_scale[row * HI + head];
      }
      wreg[m][r] = wv;
    }

  const int ntiles = (s_end - s_begin + kTileKeys - 1) / kTileKeys;
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
  u32x4 pre[C::LPT];
  u32x4 pre_sc;   // MX: 16 of the tile's scale bytes (threads < SBT / 16)

  auto issue = [&](int tile) {
    const int ts = s_begin + tile * kTileKeys;
#pragma unroll
    for (int j = 0; j < C::LPT; ++j) {
      const int i = tid + kThreads * j;
      const int key = i / C::CPK, c = i % C::CPK;
      const int lp = ts / kPage + key / kPage;
      if (lp * kPage < s_end) {
        const int phys = clamp_page(bt[lp], a.num_pages);
        pre[j] = *reinterpret_cast<const u32x4*>(a.kc + ((size_t)phys * kPage + (key % kPage)) * C::ROWB + 16 * c);
      }
    }
    if constexpr (MX) {
      // a page's 64 keys hold kPage * NG contiguous scale bytes
      if (tid < SBT / 16) {
        const int half = tid / (SBT / 32), off = 16 * (tid % (SBT / 32));
        const int lp = ts / kPage + half;
        if (lp * kPage < s_end)
          pre_sc = *reinterpret_cast<const u32x4*>(a.k_e8 + (size_t)clamp_page(bt[lp], a.num_pages) * kPage * NG + off);
      }
    }
  };
  auto commit = [&](int tile) {
    const int ts = s_begin + tile * kTileKeys;
#pragma unroll
    for (int j = 0; j < C::LPT; ++j) {
      const int i = tid + kThreads * j;
      const int key = i / C::CPK, c = i % C::CPK;
      *reinterpret_cast<u32x4*>(lds_k + key * C::ROWB + 16 * (c ^ (key & (C::CPK - 1)))) = pre[j];
    }
    if constexpr (MX) {
      if (tid < SBT / 16) *reinterpret_cast<u32x4*>(lds_kx + 16 * tid) = pre_sc;
    } else if constexpr (FP8) {
      if (tid < kTileKeys / kPage) {
        const int lp = ts / kPage + tid;
        lds_ksc[tid] = (lp * kPage < s_end) ? a.k_scale[clamp_page(bt[lp], a.num_pages)] : 0.f;
      }
    }
  };

  issue(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    lds_barrier();
    commit(tile);
    lds_barrier();
    if (tile + 1 < ntiles) issue(tile + 1);
    const int ts = s_begin + tile * kTileKeys;
    if (qvalid) {
#pragma unroll
      for (int j = 0; j < TQ; ++j) {
        const int kt = (nsub + j * C::WPQ) * 32 + nl;   // key (B column) within the tile
        f32x16 acc[C::MB];
#pragma unroll
        for (int m = 0; m < C::MB; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
        if constexpr (MX) {
          // key kt: chunks 4c + h and 4c + 2 + h of its row, and its group scales
          const unsigned char* krow = lds_k + kt * C::ROWB;
          mx_i32x8 bmx[NC];
          int bsc[NC];
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            bmx[c] = mx_join(*reinterpret_cast<const u32x4*>(krow + 16 * ((4 * c + hh) ^ (kt & (C::CPK - 1)))),
                             *reinterpret_cast<const u32x4*>(krow + 16 * ((4 * c + 2 + hh) ^ (kt & (C::CPK - 1)))));
            bsc[c] = lds_kx[kt * NG + 2 * c + hh];
          }
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int m = 0; m < C::MB; ++m) acc[m] = mfma_mx(amx[m][c], bmx[c], acc[m], asc[m][c], bsc[c]);
        } else {
          // all B fragments of the key column are read before the first MFMA
          frag_t bfr[C::KS];
#pragma unroll
          for (int kk = 0; kk < C::KS; ++kk) {
            if constexpr (FP8)
              bfr[kk] = *reinterpret_cast<const long*>(lds_k + kt * C::ROWB + 16 * (kk ^ (kt & (C::CPK - 1))) + 8 * hh);
            else
              bfr[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(
                  lds_k + kt * C::ROWB + 16 * ((2 * kk + hh) ^ (kt & (C::CPK - 1)))));
          }
#pragma unroll
          for (int kk = 0; kk < C::KS; ++kk)
#pragma unroll
            for (int m = 0; m < C::MB; ++m) {
              if constexpr (FP8) acc[m] = mfma_fp8(afrag[m][kk], bfr[kk], acc[m]);
              else acc[m] = mfma_bf16(afrag[m][kk], bfr[kk], acc[m]);
            }
        }
        float part = 0.f;
#pragma unroll
        for (int m = 0; m < C::MB; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) part = fmaf(wreg[m][r], relu(acc[m][r]), part);
        part = xor32_sum(part);
        if constexpr (FP8 && !MX) part *= lds_ksc[kt / kPage];
        const int s = ts + kt;
        if (emit && hh == 0 && s < n_me) {
          const uint32_t key = float_key(part);
          a.keys[row * a.row_stride + s] = key;
          atomicAdd(&lds_hist[qi * kBins + (key >> 21)], 1u);
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < TQ * kBins; i += kThreads) {
    const int q2 = i / kBins, t2 = t0 + q2;
    const uint32_t v = lds_hist[i];
    if (v != 0u && t2 < a.T)
      atomicAdd(&a.hist[((size_t)b * a.T + t2) * kBins + (i % kBins)], v);
  }
}

// ------------------------------------------------------------------------------------------------
// Decode / verify (T <= 4 query rows per sequence): a persistent, load-balanced grid.  The work is
// the flattened list of (sequence, KT-key tile) pairs over sequences that have more than K keys;
// workgroup g takes the contiguous share [g*N/G, (g+1)*N/G).  Each workgroup rebuilds the per-
// sequence tile offsets from seq_lens (no host round trip).  Loads run two tiles ahead in
// registers and the LDS tile is double-buffered, so one barrier per tile suffices.
constexpr int kMaxSeqPersist = 512;
constexpr int kMaxPagesPersist = 512;

template <int TQ>
struct PTile { static constexpr int KT = TQ == 1 ? 128 : 64; };

template <int HI, int DI, bool FP8, int TQ>
struct PCfg {
  static constexpr int KT = PTile<TQ>::KT;         // keys per tile
  static constexpr int MB = (HI + 31) / 32;
  static constexpr int KS = DI / 16;
  static constexpr int ELT = FP8 ? 1 : 2;
  static constexpr int ROWB = DI * ELT;
  static constexpr int CPK = ROWB / 16;
  static constexpr int TILEB = KT * ROWB;
  static constexpr int LPT = TILEB / 16 / kThreads;
  static constexpr int WPQ = 4 / TQ;                // waves per query row
  static constexpr int NBW = (KT / 32) / WPQ;       // 32-key column blocks per wave per tile
  static_assert(LPT >= 1 && NBW >= 1, "tile shape");
};

// MX: MXFP8 operands (E4M3 codes, one E8M0 scale per 32 elements) on the 32x32x64 block-scaled MFMA.
template <int HI, int DI, bool FP8, int TQ, bool MX = false>
__global__ __launch_bounds__(256, 2) void li_score_persist(ScoreArgs a) {
  static_assert(!MX || (FP8 && DI % 64 == 0), "MXFP8 keeps E4M3 codes, 64-element MFMA chunks");
  using C = PCfg<HI, DI, FP8, TQ>;
  typedef typename AFrag<FP8>::T frag_t;
  constexpr int NG = DI / 32;                     // MX: scale bytes per key row
  constexpr int NC = DI / 64;                     // MX: 64-element chunks of the dot product
  constexpr int SBT = C::KT * NG;                 // MX: scale bytes per tile
  static_assert(!MX || (SBT % 16 == 0 && SBT / 16 <= kThreads && C::KT == kPage), "tile scale bytes");
  __shared__ __attribute__((aligned(16))) unsigned char lds_kx[2][MX ? SBT : 16];
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][C::TILEB];
  __shared__ uint32_t lds_hist[TQ * kBins];
  __shared__ float lds_ksc[2][C::KT / kPage > 0 ? C::KT / kPage : 1];
  __shared__ int lds_tstart[kMaxSeqPersist + 1];
  __shared__ int lds_len[kMaxSeqPersist];       // clamped sequence length (= visible keys of the last query row)
  // per tile of this workgroup: sequence | tile index << 9, the physical pages of its (one or two)
  // pages (-1 past the sequence end), and the sequence's clamped length
  __shared__ int4 lds_rec[kMaxPagesPersist];
  __shared__ uint32_t sh[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nl = lane & 31, hh = lane >> 5;
  const int cap = a.max_seq_len;

  // flattened work list: tiles per sequence, exclusive prefix in LDS
  int carry = 0;
  for (int base = 0; base < a.B; base += kThreads) {
    const int b = base + tid;
    int v = 0;
    if (b < a.B) {
      const int nmax = row_visible(a.seq_lens, b, a.T, a.T - 1, cap);
      lds_len[b] = nmax;
      v = nmax > a.K ? (nmax + C::KT - 1) / C::KT : 0;
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<kThreads>((uint32_t)v, sh, tot);
    if (b < a.B) lds_tstart[b] = carry + (int)ex;
    carry += (int)tot;
  }
  if (tid == 0) lds_tstart[a.B] = carry;
  __syncthreads();
  const int total = carry;
  const int lo = (int)((long long)blockIdx.x * total / gridDim.x);
  const int hi = (int)((long long)(blockIdx.x + 1) * total / gridDim.x);
  // the grid keeps every range within the page table (n_items * PPT <= kMaxPagesPersist)
  constexpr int PPT = C::KT / kPage > 0 ? C::KT / kPage : 1;   // pages per tile
  const int n_items = min(hi - lo, kMaxPagesPersist / PPT);
  if (n_items <= 0) return;

  auto locate = [&](int f) -> int {   // sequence holding flat tile f
    int l = 0, h = a.B;
    while (h - l > 1) {
      const int m = (l + h) >> 1;
      if (lds_tstart[m] <= f) l = m; else h = m;
    }
    return l;
  };
  // Tile records of this workgroup's range: one round of block-table loads, off the per-tile
  // path.  A tile's loads then depend on one LDS read, and the compiler sees exactly the tile
  // loads between two tiles, so it can wait for the oldest while the others stay in flight.
  static_assert(PPT <= 2, "two pages per record");
  for (int i = tid; i < n_items; i += kThreads) {
    const int f = lo + i;
    const int b = locate(f);
    const int j = f - lds_tstart[b];
    const int n = lds_len[b];
    int pg[2] = {-1, -1};
#pragma unroll
    for (int h = 0; h < PPT; ++h) {
      const int lp = j * PPT + h;
      if (lp * kPage < n) pg[h] = clamp_page(a.block_table[(size_t)b * a.max_pages + lp], a.num_pages);
    }
    lds_rec[i] = make_int4(b | (j << 9), pg[0], pg[1], n);
  }
  __syncthreads();

  const int qi = wave / C::WPQ, nsub = wave % C::WPQ;
  const bool qvalid = qi < a.T;
  frag_t afrag[MX ? 1 : C::MB][MX ? 1 : C::KS];
  mx_i32x8 amx[MX ? C::MB : 1][MX ? NC : 1];      // MX: q codes of lane (head, h) per chunk
  int asc[MX ? C::MB : 1][MX ? NC : 1];           // MX: their group scales
  float wreg[C::MB][16];
  auto load_q = [&](int b) {
    const size_t row = (size_t)b * a.T + (qvalid ? qi : 0);
#pragma unroll
    for (int m = 0; m < C::MB; ++m) {
      const int head = 32 * m + nl;
      if constexpr (MX) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if (head < HI) {
            const unsigned char* src = a.q + (row * HI + head) * DI + 64 * c + 16 * hh;
            amx[m][c] = mx_join(*reinterpret_cast<const u32x4*>(src), *reinterpret_cast<const u32x4*>(src + 32));
            asc[m][c] = a.q_e8[(row * HI + head) * NG + 2 * c + hh];
          } else {
            amx[m][c] = mx_i32x8{0, 0, 0, 0, 0, 0, 0, 0};
            asc[m][c] = 127;
          }
        }
      }
#pragma unroll
      for (int kk = 0; kk < (MX ? 0 : C::KS); ++kk) {
        if (head < HI) {
          const unsigned char* src = a.q + ((row * HI + head) * DI + 16 * kk + 8 * hh) * C::ELT;
          if constexpr (FP8) afrag[m][kk] = *reinterpret_cast<const long*>(src);
          else afrag[m][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(src));
        } else {
          if constexpr (FP8) afrag[m][kk] = 0;
          else afrag[m][kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hd = 32 * m + 8 * (r >> 2) + 4 * hh + (r & 3);
        float wv = 0.f;
        if (hd < HI) {
          wv = a.w[row * HI + hd];
          if constexpr (FP8 && !MX) wv *= a.q_scale[row * HI + hd];
        }
        wreg[m][r] = wv;
      }
    }
  };
  auto flush = [&](int b) {
    for (int i = tid; i < TQ * kBins; i += kThreads) {
      const int t2 = i / kBins;
      const uint32_t v = lds_hist[i];
      if (v != 0u && t2 < a.T) atomicAdd(&a.hist[((size_t)b * a.T + t2) * kBins + (i % kBins)], v);
      lds_hist[i] = 0u;
    }
  };

  // Tile prefetch into registers.  Every call issues exactly LPT loads per thread (pages past the
  // sequence end and tiles past the range read page 0 instead), so the compiler can wait for one
  // tile while the next stays in flight: a load that is skipped on some path would make it wait
  // for all of them.
  // kPre tiles are in flight while one is computed; the two LDS buffers alternate by step parity.
  constexpr int kPre = TQ == 1 ? 2 : 3;
  u32x4 pre[kPre][C::LPT];
  int pb[kPre], pj[kPre];
  float psc[kPre];                    // fp8: this thread's page scale of the tile (thread < PPT)
  u32x4 psx[kPre];                    // MX: 16 of the tile's scale bytes (threads < SBT / 16 keep theirs)
  int b_iss = lds_rec[0].x & 511;     // sequence of the last tile issued (dummies reuse it)
  // A dummy call (live == false, past the end of the range) reads page 0 only and leaves the
  // sequence cursor alone; its buffer is never committed.
  auto issue = [&](int f, bool live, u32x4 (&pre)[C::LPT], int& pb, int& pj, float& psc, u32x4& psx) {
    int b = b_iss, j = 0, pg0 = -1, pg1 = -1;
    if (live) {
      const int4 r = lds_rec[f - lo];
      b = r.x & 511; j = r.x >> 9; pg0 = r.y; pg1 = r.z;
      b_iss = b;
    }
    pb = b; pj = j;
#pragma unroll
    for (int q = 0; q < C::LPT; ++q) {
      const int i = tid + kThreads * q;
      const int key = i / C::CPK, c = i % C::CPK;
      const int pg = PPT == 1 || key < kPage ? pg0 : pg1;   // -1 past the end (and for dummies)
      const int phys = pg < 0 ? 0 : pg;
      pre[q] = *reinterpret_cast<const u32x4*>(a.kc + ((size_t)phys * kPage + (key % kPage)) * C::ROWB + 16 * c);
    }
    if constexpr (MX) {               // every thread loads 16 scale bytes of the tile's page
      const int phys = pg0 < 0 ? 0 : pg0;
      psx = *reinterpret_cast<const u32x4*>(a.k_e8 + (size_t)phys * kPage * NG + 16 * (tid % (SBT / 16)));
    } else if constexpr (FP8) {       // one scale load per thread; pages past the end read page 0
      const int pg = PPT == 2 && tid == 1 ? pg1 : pg0;
      psc = a.k_scale[pg < 0 ? 0 : pg];
    }
  };
  auto commit = [&](const u32x4 (&pre)[C::LPT], float psc, const u32x4& psx, int buf, int b, int j) {
#pragma unroll
    for (int q = 0; q < C::LPT; ++q) {
      const int i = tid + kThreads * q;
      const int key = i / C::CPK, c = i % C::CPK;
      *reinterpret_cast<u32x4*>(lds_k[buf] + key * C::ROWB + 16 * (c ^ (key & (C::CPK - 1)))) = pre[q];
    }
    if constexpr (MX) {
      if (tid < SBT / 16) *reinterpret_cast<u32x4*>(lds_kx[buf] + 16 * tid) = psx;
    } else if constexpr (FP8) {
      if (tid < PPT) {
        const int lp = j * C::KT / kPage + tid;
        lds_ksc[buf][tid] = (lp * kPage < lds_len[b]) ? psc : 0.f;
      }
    }
  };
  auto compute = [&](int buf, int b, int j) {
    if (!qvalid) return;
    const int n_me = lds_len[b] - (a.T - 1 - qi);     // visible keys of query row qi
    if (n_me <= a.K) return;
    const size_t row = (size_t)b * a.T + qi;
#pragma unroll
    for (int jb = 0; jb < C::NBW; ++jb) {
      const int kt = (nsub + jb * C::WPQ) * 32 + nl;
      f32x16 acc[C::MB];
#pragma unroll
      for (int m = 0; m < C::MB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[m][r] = 0.f;
      if constexpr (MX) {
        // key kt: chunks 4c + h and 4c + 2 + h of its row, and its group scales
        const unsigned char* krow = lds_k[buf] + kt * C::ROWB;
        mx_i32x8 bmx[NC];
        int bsc[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          bmx[c] = mx_join(*reinterpret_cast<const u32x4*>(krow + 16 * ((4 * c + hh) ^ (kt & (C::CPK - 1)))),
                           *reinterpret_cast<const u32x4*>(krow + 16 * ((4 * c + 2 + hh) ^ (kt & (C::CPK - 1)))));
          bsc[c] = lds_kx[buf][kt * NG + 2 * c + hh];
        }
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int m = 0; m < C::MB; ++m) acc[m] = mfma_mx(amx[m][c], bmx[c], acc[m], asc[m][c], bsc[c]);
      } else {
        // all B fragments of the key column are read before the first MFMA
        frag_t bfr[C::KS];
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
          if constexpr (FP8)
            bfr[kk] = *reinterpret_cast<const long*>(lds_k[buf] + kt * C::ROWB + 16 * (kk ^ (kt & (C::CPK - 1))) + 8 * hh);
          else
            bfr[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(
                lds_k[buf] + kt * C::ROWB + 16 * ((2 * kk + hh) ^ (kt & (C::CPK - 1)))));
        }
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk)
#pragma unroll
          for (int m = 0; m < C::MB; ++m) {
            if constexpr (FP8) acc[m] = mfma_fp8(afrag[m][kk], bfr[kk], acc[m]);
            else acc[m] = mfma_bf16(afrag[m][kk], bfr[kk], acc[m]);
          }
      }
      float part = 0.f;
#pragma unroll
      for (int m = 0; m < C::MB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) part = fmaf(wreg[m][r], relu(acc[m][r]), part);
      part = xor32_sum(part);
      if constexpr (FP8 && !MX) part *= lds_ksc[buf][kt / kPage];
      const int s = j * C::KT + kt;
      if (hh == 0 && s < n_me) {
        const uint32_t key = float_key(part);
        a.keys[row * a.row_stride + s] = key;
        atomicAdd(&lds_hist[qi * kBins + (key >> 21)], 1u);
      }
    }
  };

  for (int i = tid; i < TQ * kBins; i += kThreads) lds_hist[i] = 0u;
#pragma unroll
  for (int u = 0; u < kPre; ++u) issue(u < n_items ? lo + u : lo, u < n_items, pre[u], pb[u], pj[u], psc[u], psx[u]);
  int b_cur = -1;
  // Every step commits, meets the barrier and issues its loads, including the up to kPre - 1
  // dead steps past the range (dummy loads, no compute): the same kPre - 1 tiles of loads then
  // follow each buffer's on every path, so the compiler waits for that buffer alone.
  auto step = [&](int i, u32x4 (&pre)[C::LPT], int& pb, int& pj, float& psc, u32x4& psx) {
    const int buf = i & 1;
    const bool alive = i < n_items;
    commit(pre, psc, psx, buf, pb, pj);
    const int b = pb, j = pj;
    // the buffer is free: the next loads go out before the barrier, their set-up overlapping it
    const bool live = i + kPre < n_items;
    issue(live ? lo + i + kPre : lo, live, pre, pb, pj, psc, psx);
    lds_barrier();                    // keeps the next tiles' loads in flight
    if (alive && b != b_cur) {        // new sequence: publish the old histogram, load new q
      if (b_cur >= 0) flush(b_cur);
      load_q(b);
      b_cur = b;
      // compiler-visible wait for q and w (vmcnt 0): without it the compiler keeps them pending
      // on every path and waits for them inside compute, behind the tiles in flight
      __builtin_amdgcn_s_waitcnt(0x0F70);
      lds_barrier();
    }
    if (alive) compute(buf, b, j);
  };
  for (int i = 0; i < n_items; i += kPre) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) step(i + u, pre[u], pb[u], pj[u], psc[u], psx[u]);
  }
  __syncthreads();
  flush(b_cur);
}

// ------------------------------------------------------------------------------------------------
// Decode (one query row per sequence) and verify (up to four).  The persistent grid walks the same
// flattened (sequence, 128-key tile) list as li_score_persist, but each wave streams its own 32-key
// blocks of every tile through a private LDS ring (two 8 KiB slots for bf16 keys, four 4 KiB slots
// for fp8) filled with direct-to-LDS loads (a block lies in one page, so its address is a scalar
// base plus a per-lane offset).  Nothing in the main loop waits for another wave: the waves meet
// only when the sequence changes, to publish the shared row histograms and load the next queries.
//   TQ = 1 (decode): 4 waves, wave w scores block w of each tile for the sequence's query row;
//                    two workgroups per CU.
//   TQ = 4 (verify): 8 waves, wave w scores query row w % 4 on blocks w / 4 and w / 4 + 2 of each
//                    tile, so every query row sees every key while the keys cross HBM once per
//                    workgroup; one workgroup per CU, histogram counters packed two per word.
constexpr int kDecodeMaxItems = 256;   // tiles per decode workgroup (the grid is sized for it)
constexpr int kMaxGroupsPersist = 4096; // query groups in a verify / prefill work list
constexpr int kGroupBits = 13;          // tile records: group | tile index << kGroupBits
static_assert(kMaxGroupsPersist <= (1 << kGroupBits) && kMaxSeqPersist <= (1 << kGroupBits), "group ids");

// MX: MXFP8 operands (FP8 storage, one E8M0 scale per 32 elements, block-scaled MFMA).
template <int HI, int DI, bool FP8, bool MX, int TQ, bool NTK = true>
__global__ __launch_bounds__(TQ == 1 ? 256 : 512, TQ == 1 ? 2 : 1) void li_score_decode(ScoreArgs a) {
  static_assert(!MX || FP8, "MXFP8 keeps E4M3 codes");
  static_assert(!FP8 || DI % 64 == 0, "E4M3 products run in 64-element MFMA chunks");
  static_assert(TQ == 1 || TQ == 4, "decode or verify");
  static_assert(HI % 4 == 0, "weights load four heads at a time");
  using C = PCfg<HI, DI, FP8, 1>;                  // 128-key tiles of four 32-key blocks
  typedef typename AFrag<FP8>::T frag_t;
  constexpr int NW = TQ == 1 ? 4 : 8;              // waves
  constexpr int NT = 64 * NW;
  constexpr int WPQ = NW / TQ;                     // waves per query row
  constexpr int NBW = 4 / WPQ;                     // blocks per wave and tile
  // E4M3 operands (fp8 and MXFP8) run on the 32x32x64 block-scaled MFMA, fp8 with unit scales
  // (its per-head and per-page scales apply outside the product)
  constexpr int NC = FP8 ? DI / 64 : 1;            // 64-element chunks of the dot product
  constexpr int BLK = 32 * C::ROWB;                // one block (bytes)
  constexpr int NG = DI / 32;                      // MX: scale bytes per key row
  constexpr int SB = 32 * NG;                      // MX: scale bytes per block
  // wave-wide loads per block: the code rows, plus (MX) one for the block's scale bytes
  constexpr int NLD = BLK / 1024 + (MX ? 1 : 0);
  constexpr int KPL = 1024 / C::ROWB;              // keys per load
  static_assert(NLD >= 1 && KPL * C::CPK == 64 && C::KT / kPage == 2, "block shape");
  static_assert(SB % 16 == 0 && SB / 16 <= 64, "scale bytes of a block: one 16-byte load per lane");
  // Decode: a private ring per wave, NSLOT slots of one block (16 KiB per wave either way).
  // Verify: one ring of RS whole tiles shared by the waves; each wave loads its share of every
  // tile, and a barrier per tile hands the tile to all of them (the four query rows read the same
  // keys, which then cross the memory system once per workgroup).
  constexpr bool SHARED = TQ != 1;
  constexpr int NSLOT = FP8 ? 4 : 2;
  constexpr int RS = 4;                            // shared ring: tiles
  constexpr int LPW = 4 * (BLK / 1024) / NW;       // shared ring: code loads per wave and tile
  constexpr int NLDT = LPW + (MX ? 1 : 0);         // shared ring: all loads per wave and tile
  static_assert(!SHARED || (4 * (BLK / 1024)) % NW == 0, "tile loads split evenly over the waves");
  static_assert(!SHARED || !MX || SB % 32 == 0, "tile scale bytes split over eight waves");
  constexpr int RING = SHARED ? RS * 4 * BLK : NW * NSLOT * BLK;
  // histogram words per query row: two 16-bit counters per word (a workgroup holds at most
  // kDecodeMaxItems * 128 = 32768 keys of a row).  Decode keeps two histograms: at a sequence
  // change the finished sequence's counts stay in LDS and go out at the end, so no device atomics
  // are in flight when the wave next waits for its loads (their acknowledgements are slow while
  // the key streams load the memory system, and the counter waits are in order).
  constexpr int HW = kBins / 2;
  constexpr int HB = TQ == 1 ? 2 : 1;
  static_assert(kDecodeMaxItems * 128 < 65536, "16-bit counters");
  // the work list lives in the key ring until the first gather
  constexpr int MAXG = TQ == 1 ? kMaxSeqPersist : kMaxGroupsPersist;   // query groups in the work list
  constexpr int WLB = ((2 * MAXG + 1) * 4 + 1023) / 1024 * 1024;
  __shared__ __attribute__((aligned(1024))) unsigned char lds_k[RING > WLB ? RING : WLB];
  __shared__ uint32_t lds_hist[HB][TQ][HW];
  // per tile of this workgroup: query group | tile index << kGroupBits, the physical pages of its
  // two halves (-1 past the sequence end), and the visible length of the group's last query row
  __shared__ int4 lds_rec[kDecodeMaxItems];
  __shared__ float2 lds_rsc[FP8 && !MX ? kDecodeMaxItems : 1];   // fp8: the two pages' scales (0 past the end)
  __shared__ __attribute__((aligned(16))) unsigned char lds_kx[MX ? (SHARED ? RS * 4 : NW * NSLOT) : 1][MX ? SB : 16];
  __shared__ int lds_starts[kDecodeMaxItems];      // query groups whose first tile is in this range
  __shared__ int lds_nstarts, lds_ok;
  __shared__ int lds_dirty[2];              // started groups whose rows need a clear
  __shared__ uint32_t sh[8];
  static_assert(sizeof(lds_k) >= (2 * MAXG + 1) * sizeof(int), "work list in the ring");
  static_assert(kDecodeMaxItems <= NT, "one tile record per thread");
  int* const lds_tstart = reinterpret_cast<int*>(&lds_k[0]);
  int* const lds_len = lds_tstart + MAXG + 1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 31, hh = lane >> 5;
  const int qi = wave % TQ, sub = wave / TQ;       // this wave's query row and first block
  const int cap = a.max_seq_len;
  DSA_STAMP(0);
  // Query group g = rows TQ*k .. TQ*k + TQ - 1 (those below T) of sequence g / GPS, k = g % GPS:
  // the sequence's one row (decode), its T <= 4 rows (verify), or four consecutive rows of a causal
  // prefill chunk.  The group's tiles cover the keys its last row sees; each row masks the rest.
  const int GPS = (a.T + TQ - 1) / TQ;             // query groups per sequence
  const int NGR = a.B * GPS;                       // query groups (the host keeps it <= MAXG)
  auto seq_of = [&](int g) { return g / GPS; };
  auto row0_of = [&](int g) { return (size_t)(g / GPS) * a.T + TQ * (g % GPS); };   // first row
  auto rows_of = [&](int g) { return min(TQ, a.T - TQ * (g % GPS)); };              // rows < T
  auto last_t_of = [&](int g) { return TQ * (g % GPS) + rows_of(g) - 1; };

  int carry = 0;
  for (int base = 0; base < NGR; base += NT) {
    const int g = base + tid;
    int v = 0;
    if (g < NGR) {
      const int nmax = row_visible(a.seq_lens, seq_of(g), a.T, last_t_of(g), cap);
      lds_len[g] = nmax;
      v = nmax > a.K ? (nmax + C::KT - 1) / C::KT : 0;
    }
    uint32_t tot;
    const uint32_t ex = block_exclusive_scan<NT>((uint32_t)v, sh, tot);
    if (g < NGR) lds_tstart[g] = carry + (int)ex;
    carry += (int)tot;
  }
  if (tid == 0) {
    lds_tstart[NGR] = carry;
    lds_nstarts = 0;
  }
  for (int i = tid; i < HB * TQ * HW; i += NT) (&lds_hist[0][0][0])[i] = 0u;
  __syncthreads();
  const int total = carry;
  const int lo = (int)((long long)blockIdx.x * total / gridDim.x);
  const int hi = (int)((long long)(blockIdx.x + 1) * total / gridDim.x);
  const int n_items = min(hi - lo, kDecodeMaxItems);   // the grid keeps hi - lo within the table
  if (n_items <= 0) {
    DSA_STAMP(1); DSA_STAMP(2);
    return;
  }

  auto locate = [&](int f) -> int {
    int l = 0, h = NGR;
    while (h - l > 1) {
      const int m = (l + h) >> 1;
      if (lds_tstart[m] <= f) l = m; else h = m;
    }
    return l;
  };

  frag_t afrag[FP8 ? 1 : C::MB][FP8 ? 1 : C::KS];
  mx_i32x8 amx[FP8 ? C::MB : 1][NC];             // E4M3: q codes of lane (head, h) per chunk
  int asc[FP8 ? C::MB : 1][NC];                  // their group scales (127 = 1 for fp8)
  float wreg[C::MB][16];
  auto load_q = [&](int g) {
    const size_t row = row0_of(g) + (qi < rows_of(g) ? qi : 0);
#pragma unroll
    for (int m = 0; m < C::MB; ++m) {
      const int head = 32 * m + nl;
      if constexpr (FP8) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          if (head < HI) {
            const unsigned char* src = a.q + (row * HI + head) * DI + 64 * c + 16 * hh;
            amx[m][c] = mx_join(*reinterpret_cast<const u32x4*>(src), *reinterpret_cast<const u32x4*>(src + 32));
            asc[m][c] = MX ? (int)a.q_e8[(row * HI + head) * NG + 2 * c + hh] : 127;
          } else {
            amx[m][c] = mx_i32x8{0, 0, 0, 0, 0, 0, 0, 0};
            asc[m][c] = 127;
          }
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
          if (head < HI) {
            const unsigned char* src = a.q + ((row * HI + head) * DI + 16 * kk + 8 * hh) * C::ELT;
            afrag[m][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(src));
          } else {
            afrag[m][kk] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
          }
        }
      }
      // weights of heads 32m + 8j + 4hh .. + 3 (register r = 4j + i): one 16-byte load per j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int hd0 = 32 * m + 8 * j + 4 * hh;
        float4 wv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (hd0 + 4 <= HI) {
          wv = *reinterpret_cast<const float4*>(a.w + row * HI + hd0);
          if constexpr (FP8 && !MX) {
            const float4 qs = *reinterpret_cast<const float4*>(a.q_scale + row * HI + hd0);
            wv.x *= qs.x; wv.y *= qs.y; wv.z *= qs.z; wv.w *= qs.w;
          }
        } else {
          float* wp = &wv.x;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (hd0 + i < HI) wp[i] = FP8 && !MX ? a.w[row * HI + hd0 + i] * a.q_scale[row * HI + hd0 + i] : a.w[row * HI + hd0 + i];
        }
        wreg[m][4 * j] = wv.x;
        wreg[m][4 * j + 1] = wv.y;
        wreg[m][4 * j + 2] = wv.z;
        wreg[m][4 * j + 3] = wv.w;
      }
    }
  };
  // Adds the LDS histograms into group g's rows once the workgroup that clears them (the one
  // holding the group's first tile) has published this call's tag in the control words of the
  // group's first row.  That workgroup has a lower index, so with workgroups dispatched in
  // index order the wait always ends.  The wait is still bounded (a.spin_cap sleeps): past it this
  // workgroup adds nothing, sets the debug flag and marks the rows with this call's tag in their
  // poison words, which li_select answers with rows of -1 (never a selection from a histogram that
  // may not have been cleared or lacks these counts).
  auto flush = [&](int g, int hb) {
    const size_t r0 = row0_of(g);
    const int nrows = rows_of(g);
    if (tid == 0) {
      const unsigned long long* tagp =
          reinterpret_cast<const unsigned long long*>(a.ctl + r0 * kCtl + kTagWord);
      unsigned spins = 0;
      int ok = 1;
      while (__hip_atomic_load(tagp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != a.tag) {
        if (++spins > a.spin_cap) {
          flag_input(kFlagSync);
          for (int t = 0; t < nrows; ++t)
            __hip_atomic_store(reinterpret_cast<unsigned long long*>(a.ctl + (r0 + t) * kCtl + kPoisonWord),
                               a.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      lds_ok = ok;
    }
    __syncthreads();
    const bool ok = lds_ok != 0;
    for (int i = tid; i < TQ * HW; i += NT) {
      const int t = i / HW, w = i % HW;
      const uint32_t v = lds_hist[hb][t][w];
      if (ok && v != 0u && t < nrows) {
        uint32_t* row_hist = a.hist + (r0 + t) * kBins;
        if (v & 0xFFFFu) atomicAdd(&row_hist[2 * w], v & 0xFFFFu);
        if (v >> 16) atomicAdd(&row_hist[2 * w + 1], v >> 16);
      }
      lds_hist[hb][t][w] = 0u;
    }
  };

  // The first group's queries load after the first key blocks are requested: the block-table loads
  // of the tile records, and then those blocks, are the longer dependent chain.
  float2 my_sc = make_float2(0.f, 0.f);   // fp8: scales of this thread's record (n_items <= threads)
  int g_cur = locate(lo);
  size_t cur_row0 = row0_of(g_cur);          // the current group's first row and row count
  int cur_rows = rows_of(g_cur);
  int hb = 0;                                // histogram the current group counts into
  int pend = -1;                             // decode: group parked in the other histogram
  for (int i = tid; i < n_items; i += NT) {
    const int f = lo + i;
    const int g = locate(f);
    const int j = f - lds_tstart[g];
    const int n = lds_len[g];
    const int b = seq_of(g);
    int pg[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int lp = 2 * j + h;
      pg[h] = lp * kPage < n ? clamp_page(a.block_table[(size_t)b * a.max_pages + lp], a.num_pages) : -1;
    }
    lds_rec[i] = make_int4(g | (j << kGroupBits), pg[0], pg[1], n);
    if (j == 0) lds_starts[atomicAdd(&lds_nstarts, 1)] = g;
    // fp8 page scales: loaded now, stored to LDS once the first gathers are in flight
    if constexpr (FP8 && !MX) my_sc = make_float2(pg[0] < 0 ? 0.f : a.k_scale[pg[0]], pg[1] < 0 ? 0.f : a.k_scale[pg[1]]);
  }
  __syncthreads();
  // This workgroup makes sure the histograms and control words of every group it starts are clear
  // (no other workgroup has flushed into them: they all wait for the tag), then publishes this
  // call's tag for each.  The select of the previous call leaves the rows it read clear, so the
  // rows are first read (every wave its share, up to kCheckStarts groups) and cleared only if any
  // word is not zero: the first call on a workspace, or one after a call that left them dirty.
  // The reads go out before the first key blocks and the wait for those blocks below covers them.
  // A clear (wave 0) goes through device-coherent (agent-scope) stores, which go past the per-XCD
  // L2s, as the histogram adds are device-coherent atomics, so finished stores are visible to every
  // workgroup; wave 0 waits for them (vmcnt 0) before the tag, which only a dirty row costs: the
  // acknowledgements of such stores take microseconds while the key streams load the memory
  // system.  A release/acquire fence pair would write back and invalidate whole L2s instead.
  const int n_starts = lds_nstarts;
  constexpr int kCheckStarts = 2;
  constexpr int kChkWords = TQ * kBins / NT;               // histogram words per thread and group
  static_assert(kChkWords % 4 == 0 && kChkWords >= 4, "16-byte check loads");
  const bool check = n_starts <= kCheckStarts;
  u32x4 chk[kCheckStarts][kChkWords / 4 + 1];
  if (check) {
#pragma unroll
    for (int k = 0; k < kCheckStarts; ++k) {
      if (k < n_starts) {
        const size_t r0 = row0_of(lds_starts[k]);
        const int nrows = rows_of(lds_starts[k]);
#pragma unroll
        for (int v = 0; v < kChkWords / 4; ++v) {
          const int w0 = 4 * (tid + NT * v);               // word of the group's rows
          chk[k][v] = w0 < nrows * kBins ? *reinterpret_cast<const u32x4*>(a.hist + r0 * kBins + w0)
                                         : u32x4{0u, 0u, 0u, 0u};
        }
        // control words 0..3 (the select's counters) of row tid
        chk[k][kChkWords / 4] = tid < nrows ? *reinterpret_cast<const u32x4*>(a.ctl + (r0 + tid) * kCtl)
                                            : u32x4{0u, 0u, 0u, 0u};
      } else {
#pragma unroll
        for (int v = 0; v <= kChkWords / 4; ++v) chk[k][v] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  DSA_STAMP(1);

  // Block blk of tile item i holds keys 32 * blk .. 32 * blk + 31 of the tile (page half
  // blk / 2).  Lane l of load u fetches key KPL*u + l / CPK, chunk (l % CPK) ^ (key % CPK), so a
  // block holds key rows of ROWB bytes with chunks XOR-swizzled by the key.  A block past the
  // sequence end reads page 0; its keys are never stored.  The loop issues no other global load
  // (the fp8 page scales come from the tile records), so the counter waits below see only these.
  // Decode: block number k of this wave is block sub + WPQ * (k % NBW) of item k / NBW, in its
  // private ring slot k % NSLOT.  Verify and prefill: item i sits in shared ring slot i % RS; this
  // wave issues loads LPW * wave .. LPW * wave + LPW - 1 of the tile's 4 * BLK / 1024 (and, MXFP8,
  // half a block's scale bytes).
  auto block_ptr = [&](int slot, int blk) -> unsigned char* {
    return SHARED ? &lds_k[(slot * 4 + blk) * BLK] : &lds_k[(wave * NSLOT + slot) * BLK];
  };
  auto block_sx = [&](int slot, int blk) -> unsigned char* {
    return SHARED ? lds_kx[slot * 4 + blk] : lds_kx[wave * NSLOT + slot];
  };
  auto load_rows = [&](const int4& r, int blk, int u, unsigned char* dst) {
    const int pg = __builtin_amdgcn_readfirstlane(blk < 2 ? r.y : r.z);
    const int phys = pg < 0 ? 0 : pg;
    const unsigned char* base = a.kc + ((size_t)phys * kPage + 32 * (blk & 1)) * C::ROWB;
    const int key = KPL * u + lane / C::CPK;
    const int c = (lane % C::CPK) ^ (key & (C::CPK - 1));
    if constexpr (NTK) lds_dma16_rows_nt(base, (uint32_t)(key * C::ROWB + 16 * c), dst + 1024 * u);
    else lds_dma16_rows(base, (uint32_t)(key * C::ROWB + 16 * c), dst + 1024 * u);
  };
  const int n_blocks = n_items;                            // ring steps (decode: NBW = 1)
  auto issue = [&](int k) {
    if constexpr (SHARED) {
      const int4 r = lds_rec[k];
      const int slot = k % RS;
#pragma unroll
      for (int v = 0; v < LPW; ++v) {
        const int g = LPW * wave + v, blk = g / (BLK / 1024), u = g % (BLK / 1024);
        load_rows(r, blk, u, block_ptr(slot, blk));
      }
      if constexpr (MX) {
        // wave w: bytes (w % 2) * SB / 2 .. of block w / 2's scales (key-major, NG per key)
        const int blk = wave / 2;
        const int pg = __builtin_amdgcn_readfirstlane(blk < 2 ? r.y : r.z);
        const int phys = pg < 0 ? 0 : pg;
        if (lane < SB / 32)
          lds_dma16(a.k_e8 + ((size_t)phys * kPage + 32 * (blk & 1)) * NG + (wave % 2) * (SB / 2) + 16 * lane,
                    block_sx(slot, blk) + (wave % 2) * (SB / 2));
      }
    } else {
      const int4 r = lds_rec[k / NBW];
      const int blk = sub + WPQ * (k % NBW);
      const int slot = k % NSLOT;
#pragma unroll
      for (int u = 0; u < BLK / 1024; ++u) load_rows(r, blk, u, block_ptr(slot, 0));
      if constexpr (MX) {
        // the block's scale bytes (key-major, NG per key) are contiguous in the scale pool
        const int pg = __builtin_amdgcn_readfirstlane(blk < 2 ? r.y : r.z);
        const int phys = pg < 0 ? 0 : pg;
        if (lane < SB / 16)
          lds_dma16(a.k_e8 + ((size_t)phys * kPage + 32 * (blk & 1)) * NG + 16 * lane, block_sx(slot, 0));
      }
    }
  };
  constexpr int kAhead = SHARED ? RS - 1 : NSLOT;        // ring steps issued before the loop
#pragma unroll
  for (int u = 0; u < kAhead; ++u)
    if (u < n_blocks) issue(u);
  load_q(g_cur);
  // compiler-visible wait (vmcnt 0) for q, w, the tile records' block-table and scale loads and
  // the check reads, so no wait for them lands in the main loop (it also covers the first blocks)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if (n_starts > 0) {                        // workgroup-uniform
    if (tid < kCheckStarts) lds_dirty[tid] = check ? 0 : 1;
    __syncthreads();
    if (check) {
#pragma unroll
      for (int k = 0; k < kCheckStarts; ++k) {
        uint32_t any = 0u;
#pragma unroll
        for (int v = 0; v <= kChkWords / 4; ++v) any |= chk[k][v][0] | chk[k][v][1] | chk[k][v][2] | chk[k][v][3];
        if (k < n_starts && __ballot(any != 0u) != 0ull && lane == 0) lds_dirty[k] = 1;
      }
    }
    __syncthreads();
    if (wave == 0) {
      bool cleared = false;
      for (int k = 0; k < n_starts; ++k) {
        if (check && lds_dirty[k] == 0) continue;
        const size_t r0 = row0_of(lds_starts[k]);
        const int nrows = rows_of(lds_starts[k]);
        for (int i = lane; i < nrows * kBins; i += 64)
          __hip_atomic_store(&a.hist[r0 * kBins + i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int i = lane; i < nrows * kTagWord; i += 64)
          __hip_atomic_store(&a.ctl[(r0 + i / kTagWord) * kCtl + i % kTagWord], 0u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        cleared = true;
      }
      if (cleared) __builtin_amdgcn_s_waitcnt(0x0F70);
      if (!a.withhold_tag)
        for (int k = lane; k < n_starts; k += 64)
          __hip_atomic_store(reinterpret_cast<unsigned long long*>(a.ctl + row0_of(lds_starts[k]) * kCtl + kTagWord),
                             a.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if constexpr (FP8 && !MX) {
    if (tid < n_items) lds_rsc[tid] = my_sc;
    lds_barrier();
  }

  // A ring step is one block of this wave (decode) or one shared tile (verify, prefill), whose
  // NB blocks of this wave are scored together: their MFMA chains interleave, and one block's
  // reduction overlaps the other's products.
  constexpr int NB = SHARED ? NBW : 1;
  for (int k = 0; k < n_blocks; ++k) {
    const int i = k;                                  // tile record (decode: NBW = 1)
    const int slot = SHARED ? i % RS : k % NSLOT;
    if constexpr (SHARED) {
      // tile i has landed for this wave (up to RS - 2 later tiles stay in flight), then for all
      // waves; every wave is past tile i - 1, whose slot takes tile i + RS - 1
      const int later = min(RS - 2, n_items - 1 - i);
      if (later >= 2) wait_vmcnt<2 * NLDT>();
      else if (later == 1) wait_vmcnt<NLDT>();
      else wait_vmcnt<0>();
      lds_barrier();
      if (i + RS - 1 < n_items) issue(i + RS - 1);
    } else {
      // this wave's block k has landed; up to NSLOT - 1 later blocks stay in flight
      const int later = min(NSLOT - 1, n_blocks - 1 - k);
      if (later >= 3) wait_vmcnt<3 * NLD>();
      else if (later == 2) wait_vmcnt<2 * NLD>();
      else if (later == 1) wait_vmcnt<NLD>();
      else wait_vmcnt<0>();
    }
    const int4 rec = lds_rec[i];
    const int g = __builtin_amdgcn_readfirstlane(rec.x & ((1 << kGroupBits) - 1));
    const int j = __builtin_amdgcn_readfirstlane(rec.x >> kGroupBits);
    if (g != g_cur) {                 // new group: publish or park the histograms, load the queries
      if constexpr (HB == 2) {
        if (pend >= 0) {              // both histograms hold groups: publish the older one
          __syncthreads();
          flush(pend, hb ^ 1);
          __syncthreads();            // cleared before the new group counts into it
        }
        pend = g_cur;
        hb ^= 1;
        load_q(g);
        __builtin_amdgcn_s_waitcnt(0x0F70);
      } else {
        __syncthreads();
        flush(g_cur, 0);
        load_q(g);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
      }
      g_cur = g;
      cur_row0 = row0_of(g);
      cur_rows = rows_of(g);
    }
    // this wave's query row (valid below T) and its visible keys (rec.w is the group's last row's)
    const bool row_ok = qi < cur_rows;
    const int n_me = __builtin_amdgcn_readfirstlane(rec.w) - (cur_rows - 1 - qi);
    f32x16 acc[NB][C::MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int m = 0; m < C::MB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[nb][m][r] = 0.f;
    if constexpr (FP8) {
      // key nl: chunks 4c + h and 4c + 2 + h of its row (16 bytes each, XOR-swizzled by the key)
      mx_i32x8 bmx[NB][NC];
      int bsc[NB][NC];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int blk = sub + WPQ * nb;
        const unsigned char* row = block_ptr(slot, SHARED ? blk : 0) + nl * C::ROWB;
        const unsigned char* blkx = block_sx(slot, SHARED ? blk : 0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          bmx[nb][c] = mx_join(*reinterpret_cast<const u32x4*>(row + 16 * ((4 * c + hh) ^ (nl & (C::CPK - 1)))),
                               *reinterpret_cast<const u32x4*>(row + 16 * ((4 * c + 2 + hh) ^ (nl & (C::CPK - 1)))));
          bsc[nb][c] = MX ? (int)blkx[nl * NG + 2 * c + hh] : 127;
        }
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int m = 0; m < C::MB; ++m) acc[nb][m] = mfma_mx(amx[m][c], bmx[nb][c], acc[nb][m], asc[m][c], bsc[nb][c]);
    } else {
      bf16x8 bfr[NB][C::KS];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const unsigned char* row = block_ptr(slot, SHARED ? sub + WPQ * nb : 0) + nl * C::ROWB;
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk)
          bfr[nb][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(row + 16 * ((2 * kk + hh) ^ (nl & (C::CPK - 1)))));
      }
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int m = 0; m < C::MB; ++m) acc[nb][m] = mfma_bf16(afrag[m][kk], bfr[nb][kk], acc[nb][m]);
    }
    // decode: the slot's reads are complete (the MFMAs consumed them): refill it
    if (!SHARED && k + NSLOT < n_blocks) issue(k + NSLOT);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int blk = sub + WPQ * nb;
      float part = 0.f;
#pragma unroll
      for (int m = 0; m < C::MB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) part = fmaf(wreg[m][r], relu(acc[nb][m][r]), part);
      part = xor32_sum(part);
      if constexpr (FP8 && !MX) {
        const float2 sc = lds_rsc[i];
        part *= blk < 2 ? sc.x : sc.y;
      }
      const int s = j * C::KT + 32 * blk + nl;
      // rows with n_me <= K select every visible key without scores (li_select)
      if (hh == 0 && s < n_me && n_me > a.K && row_ok) {
        const uint32_t key = float_key(part);
        a.keys[(cur_row0 + qi) * a.row_stride + s] = key;
        atomicAdd(&lds_hist[hb][qi][key >> 22], 1u << (16 * ((key >> 21) & 1u)));
      }
    }
  }
  __syncthreads();
  flush(g_cur, hb);
  if (HB == 2 && pend >= 0) flush(pend, hb ^ 1);
  DSA_STAMP(2);
}

// ------------------------------------------------------------------------------------------------
// Top-K selection.  Workgroups of 1024 threads (256 when every row of the launch is short, see
// SelShape); a row of n keys is cut into segments of seg_len(n) keys, one workgroup each.
struct SelectArgs {
  const uint32_t* keys;     // [rows, row_stride] order-preserving score keys
  uint32_t* hist;           // [rows, kBins] histogram of key bits 31..21 (left zero once read)
  uint32_t* ctl;            // [rows, kCtl]: segments done, gt cursor, candidate cursor (zeroed per
                            // call), then the histogram-cleared tag, which the select resets
  int32_t* g_gt;            // [rows, DSA_MAX_TOP_K] positions above the threshold range
  uint2* g_cand;            // [rows, kCandCap] (key, position) inside the threshold range
  const int32_t* seq_lens;
  int32_t* idx_out;         // [rows, K]
  unsigned long long tag;   // decode: the score launch's tag (a row whose poison words hold it is
                            // emitted as -1); 0 otherwise
  int T, K, row_stride, max_seq_len;
};

constexpr int kSelThreads = 1024;
constexpr int kSelThreadsShort = 256;                // launches whose rows are all <= kShortRow keys
constexpr int kCandCap = 8192;                       // candidates per row in the global lists
constexpr int kSelVec = 4;                           // 16-byte loads per thread per scan step
constexpr int kSelPer = 4 * kSelVec;                 // consecutive keys per thread per step (16)
constexpr int kMaxSeg = 32;                          // workgroups per row at most

// Workgroup shape of the select: NT threads, kCand candidates staged in LDS, scan steps of 16 NT
// keys, bitmap chunks of 64 NT positions.  1024 threads for long rows (steps of 16384 keys,
// chunks of 65536 positions); 256 threads when every row of the launch has at most kShortRow
// keys: 40 KiB of LDS, so four rows share a CU.
template <int NT>
struct SelShape {
  // 2040 (not 2048) candidates keep the short shape's LDS within a quarter of the CU's 160 KiB
  static constexpr int kCand = NT == kSelThreads ? 8192 : 2040;
  static constexpr int kChunk = NT * kSelPer;        // keys per scan step
  static constexpr int kMapW = 2 * NT;               // bitmap words per emit chunk
  static constexpr int kMapB = 32 * kMapW;           // positions per emit chunk
};
constexpr int kShortRow = 2 * SelShape<kSelThreadsShort>::kChunk;   // 8192 keys: two steps, one segment

// Keys per segment: whole scan steps, at most kMaxSeg segments.  A row of up to two steps stays in
// one workgroup (its second, prefetched step costs less than the publish-and-reload round trip
// between the workgroups of a split row); longer rows take one step per segment.
template <int NT = kSelThreads>
__host__ __device__ __forceinline__ int seg_len_of(int n) {
  constexpr int kChunk = SelShape<NT>::kChunk;
  const int steps = (n + kChunk - 1) / kChunk;
  if (steps <= 2) return 2 * kChunk;
  return kChunk * ((steps + kMaxSeg - 1) / kMaxSeg);
}

template <int NT>
struct SelScratch {
  uint32_t wave_tot[2][NT / 64];     // per-wave totals, alternating halves between scans
  uint32_t res[3];                   // bin search result: bin, count above it, count in it
  uint32_t cursor;                   // LDS list fill: gt count | candidate count << 16
  uint32_t pub[3];                   // global list offsets of this segment, segments done before
};

// Exclusive prefix sum over the workgroup with a single barrier: wave totals go to alternating
// halves of `wave_tot`, so the next scan never overwrites totals still being read.
template <int NT>
__device__ __forceinline__ uint32_t sel_scan(uint32_t v, SelScratch<NT>& S, uint32_t& phase, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) S.wave_tot[phase][wid] = x;
  lds_barrier();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const uint32_t t = S.wave_tot[phase][i];
    pre += i < wid ? t : 0u;
    tot += t;
  }
  phase ^= 1u;
  total = tot;
  return pre + x - v;
}

// Bin holding the need-th largest element of a histogram of NB bins (higher bin = larger keys);
// returns it with the count in higher bins (`above`) and in the bin itself (`count`).  1 <= need
// <= total is required.  Thread 0 owns the highest bins.
// sel_find_bin_pre takes this thread's PER bins already loaded (h[i] = bin hi - 1 - i).
template <int NB, int NT>
__device__ __forceinline__ uint32_t sel_find_bin_pre(const uint32_t (&h)[NB / NT], uint32_t need,
                                                     SelScratch<NT>& S, uint32_t& phase, uint32_t& above,
                                                     uint32_t& count) {
  constexpr int PER = NB / NT;
  static_assert(PER >= 1 && NB % NT == 0, "bins per thread");
  const int hi = NB - PER * (int)threadIdx.x;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += h[i];
  uint32_t tot;
  const uint32_t pre = sel_scan<NT>(mine, S, phase, tot);
  if (pre < need && pre + mine >= need) {
    uint32_t run = pre;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (run < need && run + h[i] >= need) { S.res[0] = hi - 1 - i; S.res[1] = run; S.res[2] = h[i]; }
      run += h[i];
    }
  }
  lds_barrier();
  above = S.res[1];
  count = S.res[2];
  return S.res[0];
}
template <int NB, int NT>
__device__ __forceinline__ uint32_t sel_find_bin(const uint32_t* hist, uint32_t need, SelScratch<NT>& S,
                                                 uint32_t& phase, uint32_t& above, uint32_t& count) {
  constexpr int PER = NB / NT;
  const int hi = NB - PER * (int)threadIdx.x;
  uint32_t h[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) h[i] = hist[hi - 1 - i];
  return sel_find_bin_pre<NB, NT>(h, need, S, phase, above, count);
}

// Radix digits of a key: digit 0 = bits 31..21 (histogrammed by the score kernel), digit 1 =
// bits 20..10, digit 2 = bits 9..0.  With `resolved` digits known, the unresolved low bits number:
__device__ __forceinline__ int unresolved_bits(int resolved) {
  return resolved == 1 ? 21 : (resolved == 2 ? 10 : 0);
}

// Emits, in ascending order, the positions of one chunk whose bits are set in `sel` (taken) or in
// `tie` (taken while fewer than `need` ties of the row were seen before).  Thread t holds the two
// bitmap words of positions base + 64t .. base + 64t + 63.  run_out / run_tie carry the row's
// emitted count and tie count across chunks.
template <int NT>
__device__ __forceinline__ void emit_words(const uint32_t (&sel)[2], const uint32_t (&tie)[2], int base,
                                           uint32_t need, int K, int32_t* out, SelScratch<NT>& S,
                                           uint32_t& phase, uint32_t& run_out, uint32_t& run_tie) {
  const uint32_t cs = __popc(sel[0]) + __popc(sel[1]);
  const uint32_t ct = __popc(tie[0]) + __popc(tie[1]);
  uint32_t tot;
  // taken positions per chunk < K <= 2048 fit 12 bits; ties per chunk <= 65536 fit the other 20
  const uint32_t pre = sel_scan<NT>(cs | (ct << 12), S, phase, tot);
  uint32_t rank = run_tie + (pre >> 12);
  uint32_t o = run_out + (pre & 0xFFFu) + (min(rank, need) - min(run_tie, need));
  const int p0 = base + 64 * (int)threadIdx.x;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    uint32_t m = sel[w] | tie[w];
    while (m) {
      const int j = __ffs(m) - 1;
      m &= m - 1u;
      bool take = true;
      if (!((sel[w] >> j) & 1u)) { take = rank < need; ++rank; }
      if (take) {
        if (o < (uint32_t)K) out[o] = p0 + 32 * w + j;
        ++o;
      }
    }
  }
  run_out += (tot & 0xFFFu) + (min(run_tie + (tot >> 12), need) - min(run_tie, need));
  run_tie += tot >> 12;
}

// Leaves a row's histogram and the select's counters (control words 0..3) zero for the next call,
// whose score kernel then finds them clear and skips its own clearing stores.  Called once every
// reader of this call is done with them.  Plain stores: the next call's kernels run after this
// launch has ended, when they are visible to every workgroup.
template <int NT>
__device__ __forceinline__ void sel_leave_clear(const SelectArgs& a, int row) {
  u32x4* h = reinterpret_cast<u32x4*>(a.hist + (size_t)row * kBins);
  for (int i = threadIdx.x; i < kBins / 4; i += NT) h[i] = u32x4{0u, 0u, 0u, 0u};
  if (threadIdx.x == 0) *reinterpret_cast<u32x4*>(a.ctl + (size_t)row * kCtl) = u32x4{0u, 0u, 0u, 0u};
}

// The threshold key theta (the K-th largest of the row's n > K keys) is resolved digit by digit,
// digit 0 from the row histogram.  When the keys sharing the resolved prefix (the "candidates")
// fit in LDS, each segment's workgroup collects, from its keys, the positions above the prefix
// range and the (key, position) candidates; with several segments the lists go to global memory
// and the workgroup that finishes last gathers them.  It resolves the remaining digits over the
// candidates, then emits every key > theta plus the first `need` keys == theta in position order
// through per-chunk bitmaps.  A prefix range too big for LDS falls back to one workgroup for the
// row, which resolves more digits with histogram passes over the row, and, if even the exact key
// theta has too many ties, emits straight from the keys.
template <int NT>
__global__ __launch_bounds__(NT) void li_select(SelectArgs a) {
  using Sh = SelShape<NT>;
  constexpr int kCand = Sh::kCand, kChunk = Sh::kChunk, kMapW = Sh::kMapW, kMapB = Sh::kMapB;
  __shared__ uint32_t h1[kBins];           // digit-1 histogram
  __shared__ uint32_t h2[1024];            // digit-2 histogram
  __shared__ int32_t gt_list[DSA_MAX_TOP_K];
  __shared__ uint32_t c_key[kCand];
  __shared__ int32_t c_pos[kCand];
  __shared__ uint32_t bm_sel[kMapW], bm_tie[kMapW];
  __shared__ SelScratch<NT> S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int row = blockIdx.x, seg = blockIdx.y;
  const int b = row / a.T, t = row % a.T;
  // timeline points 3 and 4 from the row's first segment, 5..7 from the segment that finishes the
  // row (the score kernel uses 0..2)
#define SEL_STAMP(point) do { if (seg == 0 || (point) >= 5) DSA_STAMP(point); } while (0)
  SEL_STAMP(3);
  // The row histogram's bins of this thread go out first, beside the sequence length and poison
  // loads they would otherwise wait behind.
  constexpr int kHistPer = kBins / NT;
  uint32_t hist0[kHistPer];
#pragma unroll
  for (int i = 0; i < kHistPer; ++i)
    hist0[i] = a.hist[(size_t)row * kBins + kBins - kHistPer * tid - 1 - i];
  // the score kernel of this call is done with the row's histogram-cleared tag: reset it, so a
  // replay of the same launches (same tag) waits for its own clear again
  if (seg == 0 && tid == 0)
    *reinterpret_cast<unsigned long long*>(a.ctl + (size_t)row * kCtl + kTagWord) = 0ull;
  const int n = row_visible(a.seq_lens, b, a.T, t, a.max_seq_len);
  int32_t* out = a.idx_out + (size_t)row * a.K;
  if (n <= a.K) {
    if (seg == 0)
      for (int j = tid; j < a.K; j += NT) out[j] = j < n ? j : -1;
    return;
  }
  if (a.tag != 0ull &&
      *reinterpret_cast<const unsigned long long*>(a.ctl + (size_t)row * kCtl + kPoisonWord) == a.tag) {
    // a score workgroup of this call gave up waiting for the row's histogram clear
    if (seg == 0)
      for (int j = tid; j < a.K; j += NT) out[j] = -1;
    return;
  }
  const int seg_len = seg_len_of<NT>(n);
  int nseg = (n + seg_len - 1) / seg_len;
  if (seg >= nseg) return;
  int lo = seg * seg_len, hi = min(n, lo + seg_len);
  const uint32_t* keys = a.keys + (size_t)row * a.row_stride;
  uint32_t phase = 0;

  // Pass over [lo, hi) in steps of kChunk keys: per_step(v, s0) gets this thread's kSelPer
  // consecutive keys from position s0 on (entries at positions >= hi are zero or stale and must
  // be masked).  The next step loads while the current one is processed.  A 16-byte load is
  // issued only if it starts below hi <= n; the row stride is a multiple of 4, so none leaves the
  // row.
  auto load_step = [&](u32x4 (&v)[kSelVec], int s0) {
#pragma unroll
    for (int u = 0; u < kSelVec; ++u)
      if (s0 + 4 * u < hi) v[u] = *reinterpret_cast<const u32x4*>(keys + s0 + 4 * u);
  };
  u32x4 cur[kSelVec];
#pragma unroll
  for (int u = 0; u < kSelVec; ++u) cur[u] = u32x4{0u, 0u, 0u, 0u};
  load_step(cur, lo + tid * kSelPer);      // the first step is requested before anything else
  auto scan_keys = [&](auto&& per_step) {   // runs once per workgroup
    u32x4 nxt[kSelVec];
#pragma unroll
    for (int u = 0; u < kSelVec; ++u) nxt[u] = u32x4{0u, 0u, 0u, 0u};
    for (int base = lo; base < hi; base += kChunk) {
      const int s0 = base + tid * kSelPer;
      if (base + kChunk < hi) load_step(nxt, s0 + kChunk);
      per_step(cur, s0);
#pragma unroll
      for (int u = 0; u < kSelVec; ++u) cur[u] = nxt[u];
    }
  };
  auto key_of = [](const u32x4 (&v)[kSelVec], int j) -> uint32_t { return v[j >> 2][j & 3]; };

  for (int i = tid; i < kBins; i += NT) h1[i] = 0u;
  for (int i = tid; i < 1024; i += NT) h2[i] = 0u;
  if (tid == 0) S.cursor = 0u;
  uint32_t above, C;
  uint32_t prefix = sel_find_bin_pre<kBins, NT>(hist0, (uint32_t)a.K, S, phase, above, C);
  SEL_STAMP(4);
  if (nseg == 1) sel_leave_clear<NT>(a, row);   // the only reader has read it (the scan's barrier)
  uint32_t need = (uint32_t)a.K - above;  // keys still to take from the current prefix range
  const uint32_t G = above;               // keys above the digit-0 range
  int resolved = 1;
  uint32_t G2 = G;                        // keys above the final prefix range (fallback only)

  if (C > (uint32_t)kCand) {
    // one workgroup takes the whole row; more digits from histogram passes over it
    if (seg != 0) return;
    nseg = 1; lo = 0; hi = n;
    while (C > (uint32_t)kCand && resolved < 3) {
      const int sh = unresolved_bits(resolved);
      uint32_t* hh = resolved == 1 ? h1 : h2;
      for (int s = tid * 4; s < n; s += NT * 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(keys + s);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (s + j < n && (v[j] >> sh) == prefix)
            atomicAdd(&hh[resolved == 1 ? ((v[j] >> 10) & 2047u) : (v[j] & 1023u)], 1u);
      }
      lds_barrier();
      const uint32_t d = resolved == 1 ? sel_find_bin<kBins, NT>(hh, need, S, phase, above, C)
                                       : sel_find_bin<1024, NT>(hh, need, S, phase, above, C);
      need -= above;
      G2 += above;
      prefix = (prefix << (resolved == 1 ? 11 : 10)) | d;
      ++resolved;
    }
  }

  uint32_t run_out = 0, run_tie = 0;
  if (C <= (uint32_t)kCand) {
    const int shift = unresolved_bits(resolved);
    const uint32_t hi_key = shift ? ((prefix << shift) | ((1u << shift) - 1u)) : prefix;
    // collect positions above the prefix range and candidates inside it (any order); each wave
    // reserves its slots with one LDS atomic
    scan_keys([&](const u32x4 (&v)[kSelVec], int s0) {
      uint32_t gm = 0, cm = 0;
#pragma unroll
      for (int j = 0; j < kSelPer; ++j) {
        const uint32_t k = key_of(v, j);
        const bool ok = s0 + j < hi;
        gm |= (ok && k > hi_key) ? (1u << j) : 0u;
        cm |= (ok && (k >> shift) == prefix) ? (1u << j) : 0u;
      }
      const uint32_t mine = __popc(gm) | ((uint32_t)__popc(cm) << 16);
      const uint32_t incl = wave_inclusive_scan(mine);
      uint32_t wbase = 0;
      if (lane == 63) wbase = atomicAdd(&S.cursor, incl);
      wbase = __builtin_amdgcn_readlane(wbase, 63);
      const uint32_t off = wbase + incl - mine;
      uint32_t og = off & 0xFFFFu, oc = off >> 16;
      while (gm) {
        const int j = __ffs(gm) - 1;
        gm &= gm - 1u;
        if (og < DSA_MAX_TOP_K) gt_list[og] = s0 + j;
        ++og;
      }
#pragma unroll
      for (int j = 0; j < kSelPer; ++j)
        if ((cm >> j) & 1u) {
          if (oc < (uint32_t)kCand) { c_key[oc] = key_of(v, j); c_pos[oc] = s0 + j; }
          ++oc;
        }
    });
    lds_barrier();
    if (nseg > 1) {
      // publish this segment's lists; the last segment to finish carries on with the row
      const uint32_t cnt = S.cursor;
      const uint32_t ng = min(cnt & 0xFFFFu, (uint32_t)DSA_MAX_TOP_K), nc = min(cnt >> 16, (uint32_t)kCand);
      uint32_t* ctl = a.ctl + (size_t)row * kCtl;
      if (tid == 0) {
        S.pub[0] = atomicAdd(&ctl[1], ng);
        S.pub[1] = atomicAdd(&ctl[2], nc);
      }
      lds_barrier();
      const uint32_t gb = S.pub[0], cb = S.pub[1];
      int32_t* g_gt = a.g_gt + (size_t)row * DSA_MAX_TOP_K;
      uint2* g_c = a.g_cand + (size_t)row * kCandCap;
      // The lists travel through device-coherent (agent-scope) stores and loads, which go past
      // the per-XCD L2s, so finishing the stores (vmcnt) before the counter update is enough to
      // publish them; a full release/acquire fence would write back and invalidate the whole L2
      // for every segment.
      for (uint32_t i = tid; i < ng; i += NT)
        if (gb + i < DSA_MAX_TOP_K)
          __hip_atomic_store(&g_gt[gb + i], gt_list[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (uint32_t i = tid; i < nc; i += NT)
        if (cb + i < (uint32_t)kCandCap) {
          const uint64_t e = (uint64_t)c_key[i] | ((uint64_t)(uint32_t)c_pos[i] << 32);
          __hip_atomic_store(reinterpret_cast<uint64_t*>(&g_c[cb + i]), e, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      wait_vmcnt<0>();
      lds_barrier();
      if (tid == 0) S.pub[2] = atomicAdd(&ctl[0], 1u);
      lds_barrier();
      if (S.pub[2] != (uint32_t)(nseg - 1)) return;
      // every segment has read the histogram and updated the counters
      sel_leave_clear<NT>(a, row);
      for (uint32_t i = tid; i < G; i += NT)
        gt_list[i] = __hip_atomic_load(&g_gt[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (uint32_t i = tid; i < C; i += NT) {
        const uint64_t e = __hip_atomic_load(reinterpret_cast<uint64_t*>(&g_c[i]), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        c_key[i] = (uint32_t)e;
        c_pos[i] = (int32_t)(e >> 32);
      }
      lds_barrier();
    }
    SEL_STAMP(5);
    const int ng = (int)min(G2, (uint32_t)DSA_MAX_TOP_K), nc = (int)C;
    // remaining digits over the candidates (each digit's histogram is used once)
    if (resolved == 1) {
      for (int i = tid; i < nc; i += NT) atomicAdd(&h1[(c_key[i] >> 10) & 2047u], 1u);
      lds_barrier();
      uint32_t cnt;
      const uint32_t d = sel_find_bin<kBins, NT>(h1, need, S, phase, above, cnt);
      need -= above;
      prefix = (prefix << 11) | d;
      resolved = 2;
    }
    if (resolved == 2) {
      for (int i = tid; i < nc; i += NT) {
        const uint32_t k = c_key[i];
        if ((k >> 10) == prefix) atomicAdd(&h2[k & 1023u], 1u);
      }
      lds_barrier();
      uint32_t cnt;
      const uint32_t d = sel_find_bin<1024, NT>(h2, need, S, phase, above, cnt);
      need -= above;
      prefix = (prefix << 10) | d;
    }
    const uint32_t theta = prefix;       // the exact threshold key; `need` of its ties are kept
    SEL_STAMP(6);
    for (int c0 = 0; c0 < n; c0 += kMapB) {
      const int c1 = min(n, c0 + kMapB);
      bm_sel[2 * tid] = 0u; bm_sel[2 * tid + 1] = 0u;
      bm_tie[2 * tid] = 0u; bm_tie[2 * tid + 1] = 0u;
      lds_barrier();
      for (int i = tid; i < ng; i += NT) {
        const int p = gt_list[i];
        if (p >= c0 && p < c1) atomicOr(&bm_sel[(p - c0) >> 5], 1u << ((p - c0) & 31));
      }
      for (int i = tid; i < nc; i += NT) {
        const int p = c_pos[i];
        const uint32_t k = c_key[i];
        if (p >= c0 && p < c1 && k >= theta)
          atomicOr(k > theta ? &bm_sel[(p - c0) >> 5] : &bm_tie[(p - c0) >> 5], 1u << ((p - c0) & 31));
      }
      lds_barrier();
      const uint32_t sw[2] = {bm_sel[2 * tid], bm_sel[2 * tid + 1]};
      const uint32_t tw[2] = {bm_tie[2 * tid], bm_tie[2 * tid + 1]};
      emit_words<NT>(sw, tw, c0, need, a.K, out, S, phase, run_out, run_tie);
    }
  } else {
    // theta is exact (all digits resolved) and its ties exceed the staging space: the bitmap
    // words come straight from the keys
    const uint32_t theta = prefix;
    for (int c0 = 0; c0 < n; c0 += kMapB) {
      uint32_t sw[2] = {0u, 0u}, tw[2] = {0u, 0u};
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int p0 = c0 + 64 * tid + 32 * w;
        for (int u = 0; u < 8; ++u) {
          if (p0 + 4 * u >= n) break;
          const u32x4 v = *reinterpret_cast<const u32x4*>(keys + p0 + 4 * u);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool ok = p0 + 4 * u + j < n;
            sw[w] |= (ok && v[j] > theta) ? (1u << (4 * u + j)) : 0u;
            tw[w] |= (ok && v[j] == theta) ? (1u << (4 * u + j)) : 0u;
          }
        }
      }
      emit_words<NT>(sw, tw, c0, need, a.K, out, S, phase, run_out, run_tie);
    }
  }
  for (int j = (int)run_out + tid; j < a.K; j += NT) out[j] = -1;
  SEL_STAMP(7);
#undef SEL_STAMP
}

// ------------------------------------------------------------------------------------------------
static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

#ifdef DSA_TIMELINE
extern "C" int dsa_timeline_reset_indexer(void) {
  static unsigned long long zeros[kTimelineWgs][8];
  return hipMemcpyToSymbol(HIP_SYMBOL(g_timeline), zeros, sizeof zeros, 0, hipMemcpyHostToDevice) == hipSuccess ? 0 : 2;
}

extern "C" int dsa_timeline_fetch_indexer(unsigned long long* host, int wgs) {
  if (wgs < 0 || wgs > kTimelineWgs) return 1;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_timeline), (size_t)wgs * 8 * sizeof(unsigned long long), 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? 0 : 2;
}
#endif

hipError_t indexer_take_input_flags(uint32_t* flags) {
  uint32_t z = 0;
  hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_input_flags), sizeof(uint32_t), 0, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(g_input_flags), &z, sizeof z, 0, hipMemcpyHostToDevice);
  return e;
}

IndexerPlan plan_indexer(const dsa_paged_layout& L, const dsa_indexer_shape& S) {
  IndexerPlan p;
  p.rows = L.batch * S.T;
  p.row_stride = (int)align_up((size_t)L.max_seq_len, 64);
  p.n_chunks = (L.max_seq_len + kChunkKeys - 1) / kChunkKeys;
  p.tq = S.T == 1 ? 1 : (S.T == 2 ? 2 : 4);
  p.n_qtiles = (S.T + p.tq - 1) / p.tq;
  size_t off = 0;
  // the select's per-row control words follow the histograms so one clear covers both
  p.off_hist = off; off = align_up(off + (size_t)p.rows * (kBins + kCtl) * 4, 256);
  p.off_keys = off; off = align_up(off + (size_t)p.rows * p.row_stride * 4, 256);
  p.n_seg = (L.max_seq_len + seg_len_of(L.max_seq_len) - 1) / seg_len_of(L.max_seq_len);
  p.off_gt = p.off_cand = 0;
  if (p.n_seg > 1) {
    p.off_gt = off; off = align_up(off + (size_t)p.rows * DSA_MAX_TOP_K * 4, 256);
    p.off_cand = off; off = align_up(off + (size_t)p.rows * kCandCap * 8, 256);
  }
  p.total = off;
  return p;
}

bool indexer_supported(int heads, int dim) {
  return (heads == 8 || heads == 16 || heads == 32 || heads == 64) && (dim == 64 || dim == 128);
}

// Score kernel per call: the decode kernel (T = 1), the grouped kernel (query groups of up to four
// rows: verify, with the keys streamed past the caches, and causal prefill chunks, whose query
// groups reread the same keys and keep them cached), the two-row persistent kernel (T = 2), or the
// chunked grid when the work list would not fit a workgroup's LDS.
enum class ScoreMode { kChunked, kDecode, kVerify, kPrefill, kPersist2 };

template <int HI, int DI, bool FP8, bool MX>
static void launch_score_mode(const ScoreArgs& s, ScoreMode mode, int tq, int grid, hipStream_t st) {
  switch (mode) {
    case ScoreMode::kDecode: hipLaunchKernelGGL((li_score_decode<HI, DI, FP8, MX, 1>), dim3(grid), dim3(256), 0, st, s); return;
    case ScoreMode::kVerify: hipLaunchKernelGGL((li_score_decode<HI, DI, FP8, MX, 4, true>), dim3(grid), dim3(512), 0, st, s); return;
    case ScoreMode::kPrefill: hipLaunchKernelGGL((li_score_decode<HI, DI, FP8, MX, 4, false>), dim3(grid), dim3(512), 0, st, s); return;
    case ScoreMode::kPersist2: hipLaunchKernelGGL((li_score_persist<HI, DI, FP8, 2, MX>), dim3(grid), dim3(kThreads), 0, st, s); return;
    case ScoreMode::kChunked:
      if (tq == 1) hipLaunchKernelGGL((li_score<HI, DI, FP8, 1, MX>), dim3(grid), dim3(kThreads), 0, st, s);
      else if (tq == 2) hipLaunchKernelGGL((li_score<HI, DI, FP8, 2, MX>), dim3(grid), dim3(kThreads), 0, st, s);
      else hipLaunchKernelGGL((li_score<HI, DI, FP8, 4, MX>), dim3(grid), dim3(kThreads), 0, st, s);
      return;
  }
}

template <int HI, int DI>
static void launch_score_dt(const ScoreArgs& s, bool fp8, bool mx, ScoreMode mode, int tq, int grid, hipStream_t st) {
  if (mx) launch_score_mode<HI, DI, true, true>(s, mode, tq, grid, st);
  else if (fp8) launch_score_mode<HI, DI, true, false>(s, mode, tq, grid, st);
  else launch_score_mode<HI, DI, false, false>(s, mode, tq, grid, st);
}

// MXFP8 runs on every score path (decode, verify, chunked prefill).
bool indexer_mx_supported(int batch, int T) { return batch >= 1 && T >= 1; }

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

hipError_t launch_indexer(const IndexerArgs& a, const IndexerPlan& p, hipStream_t st) {
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  uint32_t* hist = reinterpret_cast<uint32_t*>(ws + p.off_hist);
  const size_t hist_words = (size_t)p.rows * (kBins + kCtl);   // histograms + control words
  const long long groups4 = (long long)a.B * ((a.T + 3) / 4);
  const ScoreMode mode = a.T == 1 ? (a.B <= kMaxSeqPersist ? ScoreMode::kDecode : ScoreMode::kChunked)
                       : a.T == 2 ? (a.B <= kMaxSeqPersist ? ScoreMode::kPersist2 : ScoreMode::kChunked)
                       : groups4 <= kMaxGroupsPersist ? (a.T <= 4 ? ScoreMode::kVerify : ScoreMode::kPrefill)
                       : ScoreMode::kChunked;
  // the decode and grouped kernels clear their rows' histograms themselves (tag handshake); the
  // others need them clear
  const bool self_clear = mode == ScoreMode::kDecode || mode == ScoreMode::kVerify || mode == ScoreMode::kPrefill;
  if (!self_clear) {
    const int zgrid = (int)std::min<size_t>((hist_words / 4 + 255) / 256, 2048);
    LaunchScope ls("li_zero_hist", st);
    hipLaunchKernelGGL(li_zero_hist, dim3(zgrid), dim3(256), 0, st, hist, hist_words);
  }

  ScoreArgs s;
  s.q = static_cast<const unsigned char*>(a.q);
  s.q_scale = a.fp8 ? static_cast<const float*>(a.q_scale) : nullptr;
  s.w = a.w;
  s.kc = static_cast<const unsigned char*>(a.k_cache);
  s.k_scale = a.fp8 ? static_cast<const float*>(a.k_scale) : nullptr;
  s.q_e8 = a.mx ? static_cast<const unsigned char*>(a.q_scale) : nullptr;
  s.k_e8 = a.mx ? static_cast<const unsigned char*>(a.k_scale) : nullptr;
  s.block_table = a.block_table;
  s.seq_lens = a.seq_lens;
  s.keys = reinterpret_cast<uint32_t*>(ws + p.off_keys);
  s.hist = hist;
  s.ctl = hist + (size_t)p.rows * kBins;
  s.tag = self_clear ? next_call_tag() : 0ull;
  // Test hooks for the bounded tag wait (read per call; unset in normal use):
  // DSA_TEST_SYNC_SPIN_CAP overrides the number of sleeps before a wait gives up, and
  // DSA_TEST_WITHHOLD_TAG=1 makes the clearing workgroups publish no tag, so every wait times out.
  s.spin_cap = kSyncSpinCap;
  s.withhold_tag = 0;
  if (self_clear) {
    if (const char* e = getenv("DSA_TEST_SYNC_SPIN_CAP")) s.spin_cap = (unsigned)strtoul(e, nullptr, 10);
    if (const char* e = getenv("DSA_TEST_WITHHOLD_TAG")) s.withhold_tag = atoi(e) != 0;
  }
  s.B = a.B; s.T = a.T; s.max_pages = a.max_pages; s.num_pages = a.num_pages; s.K = a.top_k;
  s.n_chunks = p.n_chunks; s.n_qtiles = p.n_qtiles; s.row_stride = p.row_stride;
  s.max_seq_len = a.max_seq_len;
  int grid = a.B * p.n_qtiles * p.n_chunks;
  if (mode != ScoreMode::kChunked) {
    // decode: two 4-wave workgroups per CU over (sequence, 128-key tile); grouped: one 8-wave
    // workgroup per CU over (query group, 128-key tile); two rows: two per CU over 64-key tiles
    const bool two = mode == ScoreMode::kPersist2;
    const int kt = two ? 64 : 128;
    const long long units = mode == ScoreMode::kDecode || two ? a.B : groups4;
    const long long max_tiles = units * ((a.max_seq_len + kt - 1) / kt);
    const long long per_cu = mode == ScoreMode::kDecode || two ? 2 : 1;
    grid = (int)std::max<long long>(1, std::min<long long>(per_cu * device_cus(), (max_tiles + 1) / 2));
    // a workgroup's range (at most ceil(max_tiles / grid) tiles) must fit its tile table:
    // kDecodeMaxItems tiles in the decode and grouped kernels, kMaxPagesPersist pages in the other
    if (!two) grid = (int)std::max<long long>(grid, (max_tiles + kDecodeMaxItems - 1) / kDecodeMaxItems);
    else grid = (int)std::max<long long>(grid, (max_tiles * (kt / kPage) + kMaxPagesPersist - 1) / kMaxPagesPersist);
  }
  if (grid > 0) {
    LaunchScope ls("li_score", st);
    switch (a.heads * 1000 + a.dim) {
      case 8064: launch_score_dt<8, 64>(s, a.fp8, a.mx, mode, p.tq, grid, st); break;
      case 8128: launch_score_dt<8, 128>(s, a.fp8, a.mx, mode, p.tq, grid, st); break;
      case 16064: launch_score_dt<16, 64>(s, a.fp8, a.mx, mode, p.tq, grid, st); break;
      case 16128: launch_score_dt<16, 128>(s, a.fp8, a.mx, mode, p.tq, grid, st); break;
      case 32064: launch_score_dt<32, 64>(s, a.fp8, a.mx, mode, p.tq, grid, st); break;
      case 32128: launch_score_dt<32, 128>(s, a.fp8, a.mx, mode, p.tq, grid, st); break;
      case 64064: launch_score_dt<64, 64>(s, a.fp8, a.mx, mode, p.tq, grid, st); break;
      case 64128: launch_score_dt<64, 128>(s, a.fp8, a.mx, mode, p.tq, grid, st); break;
      default: return hipErrorInvalidValue;
    }
  }
  SelectArgs sa;
  sa.keys = s.keys;
  sa.hist = hist;
  sa.ctl = hist + (size_t)p.rows * kBins;
  sa.g_gt = reinterpret_cast<int32_t*>(ws + p.off_gt);
  sa.g_cand = reinterpret_cast<uint2*>(ws + p.off_cand);
  sa.seq_lens = a.seq_lens;
  sa.idx_out = a.idx_out;
  sa.tag = s.tag;
  sa.T = a.T; sa.K = a.top_k; sa.row_stride = p.row_stride; sa.max_seq_len = a.max_seq_len;
  {
    LaunchScope ls("li_select", st);
    // rows of at most kShortRow keys (one segment each): the 256-thread shape, four rows per CU
    if (a.max_seq_len <= kShortRow)
      hipLaunchKernelGGL(li_select<kSelThreadsShort>, dim3(p.rows, 1), dim3(kSelThreadsShort), 0, st, sa);
    else
      hipLaunchKernelGGL(li_select<kSelThreads>, dim3(p.rows, p.n_seg), dim3(kSelThreads), 0, st, sa);
  }
  return hipGetLastError();
}

}  // namespace dsa
