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
//   li_zero_hist    clears the per-row 2048-bin histograms of the score keys' top 11 bits.
//   li_score        one workgroup per (sequence, tile of query rows, chunk of 1024 keys): streams
//                   the chunk's pages (page-table resolved) through LDS, MFMA score GEMM
//                   [heads x dim] x [dim x keys], ReLU and head-weight reduction in registers,
//                   order-preserving u32 keys to the row scratch, LDS histogram -> global.
//   li_select_split one workgroup per (row, slice of 4096 keys): from the row histogram finds the
//                   bin holding the K'-th key, then an ordered compaction of its slice emits the
//                   positions above that bin and the (key, position) candidates inside it.
//   li_select_final one workgroup per row: refines the threshold key over the candidates (two
//                   more radix digits), picks candidates above it plus the lowest-position ties up
//                   to the quota, and merges them with the above-bin positions into idx_out.
// A row with n <= K selects every visible position and skips the score scratch.
#include <algorithm>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

constexpr int kTileKeys = 128;    // keys staged in LDS per step (two pages)
constexpr int kChunkKeys = 1024;  // keys per score workgroup
constexpr int kBins = 2048;       // first radix digit: key bits 31..21
constexpr int kSlice = 4096;      // keys per select-phase-1 workgroup
constexpr int kMaxSlices = 256;   // rows up to 1M keys
constexpr int kThreads = 256;

// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void li_zero_hist(uint32_t* __restrict__ hist, size_t n_words) {
  u32x4* p = reinterpret_cast<u32x4*>(hist);
  const size_t n4 = n_words / 4;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
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

template <int HI, int DI, bool FP8, int TQ>
__global__ __launch_bounds__(256) void li_score(ScoreArgs a) {
  using C = ScoreCfg<HI, DI, FP8, TQ>;
  typedef typename AFrag<FP8>::T frag_t;
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[C::TILEB];
  __shared__ uint32_t lds_hist[TQ * kBins];
  __shared__ float lds_ksc[kTileKeys / kPage];

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
  frag_t afrag[C::MB][C::KS];
#pragma unroll
  for (int m = 0; m < C::MB; ++m) {
    const int head = 32 * m + nl;
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
        if constexpr (FP8) wv *= a.q_scale[row * HI + head];
      }
      wreg[m][r] = wv;
    }

  const int ntiles = (s_end - s_begin + kTileKeys - 1) / kTileKeys;
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
  u32x4 pre[C::LPT];

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
  };
  auto commit = [&](int tile) {
    const int ts = s_begin + tile * kTileKeys;
#pragma unroll
    for (int j = 0; j < C::LPT; ++j) {
      const int i = tid + kThreads * j;
      const int key = i / C::CPK, c = i % C::CPK;
      *reinterpret_cast<u32x4*>(lds_k + key * C::ROWB + 16 * (c ^ (key & (C::CPK - 1)))) = pre[j];
    }
    if constexpr (FP8) {
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
#pragma unroll
        for (int kk = 0; kk < C::KS; ++kk) {
          if constexpr (FP8) {
            const long bf = *reinterpret_cast<const long*>(
                lds_k + kt * C::ROWB + 16 * (kk ^ (kt & (C::CPK - 1))) + 8 * hh);
#pragma unroll
            for (int m = 0; m < C::MB; ++m) acc[m] = mfma_fp8(afrag[m][kk], bf, acc[m]);
          } else {
            const bf16x8 bf = as_bf16x8(*reinterpret_cast<const u32x4*>(
                lds_k + kt * C::ROWB + 16 * ((2 * kk + hh) ^ (kt & (C::CPK - 1)))));
#pragma unroll
            for (int m = 0; m < C::MB; ++m) acc[m] = mfma_bf16(afrag[m][kk], bf, acc[m]);
          }
        }
        float part = 0.f;
#pragma unroll
        for (int m = 0; m < C::MB; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) part = fmaf(wreg[m][r], fmaxf(acc[m][r], 0.f), part);
        part += __shfl_xor(part, 32, 64);
        if constexpr (FP8) part *= lds_ksc[kt / kPage];
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

template <int HI, int DI, bool FP8, int TQ>
__global__ __launch_bounds__(256, 2) void li_score_persist(ScoreArgs a) {
  using C = PCfg<HI, DI, FP8, TQ>;
  typedef typename AFrag<FP8>::T frag_t;
  __shared__ __attribute__((aligned(16))) unsigned char lds_k[2][C::TILEB];
  __shared__ uint32_t lds_hist[TQ * kBins];
  __shared__ float lds_ksc[2][C::KT / kPage > 0 ? C::KT / kPage : 1];
  __shared__ int lds_tstart[kMaxSeqPersist + 1];
  __shared__ int lds_len[kMaxSeqPersist];       // clamped sequence length (= visible keys of the last query row)
  __shared__ int lds_page[kMaxPagesPersist];    // physical pages of this workgroup's tiles, in order
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
  const int n_items = hi - lo;
  if (n_items <= 0) return;

  auto locate = [&](int f) -> int {   // sequence holding flat tile f
    int l = 0, h = a.B;
    while (h - l > 1) {
      const int m = (l + h) >> 1;
      if (lds_tstart[m] <= f) l = m; else h = m;
    }
    return l;
  };
  // physical page ids of this workgroup's tiles (one round of block-table loads, off the
  // per-tile critical path); a range longer than the LDS table reads the block table directly
  constexpr int PPT = C::KT / kPage > 0 ? C::KT / kPage : 1;   // pages per tile
  const bool page_cached = n_items * PPT <= kMaxPagesPersist;
  if (page_cached) {
    for (int i = tid; i < n_items * PPT; i += kThreads) {
      const int f = lo + i / PPT;
      const int b = locate(f);
      const int lp = (f - lds_tstart[b]) * PPT + i % PPT;
      lds_page[i] = lp * kPage < lds_len[b]
          ? clamp_page(a.block_table[(size_t)b * a.max_pages + lp], a.num_pages) : 0;
    }
  }
  __syncthreads();
  auto page_of = [&](int f, int b, int lp) -> int {
    if (page_cached) return lds_page[(f - lo) * PPT + (lp % PPT)];
    return clamp_page(a.block_table[(size_t)b * a.max_pages + lp], a.num_pages);
  };

  const int qi = wave / C::WPQ, nsub = wave % C::WPQ;
  const bool qvalid = qi < a.T;
  frag_t afrag[C::MB][C::KS];
  float wreg[C::MB][16];
  auto load_q = [&](int b) {
    const size_t row = (size_t)b * a.T + (qvalid ? qi : 0);
#pragma unroll
    for (int m = 0; m < C::MB; ++m) {
      const int head = 32 * m + nl;
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
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int hd = 32 * m + 8 * (r >> 2) + 4 * hh + (r & 3);
        float wv = 0.f;
        if (hd < HI) {
          wv = a.w[row * HI + hd];
          if constexpr (FP8) wv *= a.q_scale[row * HI + hd];
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

  u32x4 pre0[C::LPT], pre1[C::LPT];
  int pb0 = 0, pj0 = 0, pb1 = 0, pj1 = 0;
  auto issue = [&](int f, u32x4 (&pre)[C::LPT], int& pb, int& pj) {
    const int b = locate(f);
    const int j = f - lds_tstart[b];
    pb = b; pj = j;
    const int nmax = lds_len[b];
    const int ts = j * C::KT;
#pragma unroll
    for (int q = 0; q < C::LPT; ++q) {
      const int i = tid + kThreads * q;
      const int key = i / C::CPK, c = i % C::CPK;
      const int lp = ts / kPage + key / kPage;
      if (lp * kPage < nmax) {
        const int phys = page_of(f, b, lp);
        pre[q] = *reinterpret_cast<const u32x4*>(a.kc + ((size_t)phys * kPage + (key % kPage)) * C::ROWB + 16 * c);
      }
    }
  };
  auto commit = [&](const u32x4 (&pre)[C::LPT], int buf, int b, int j) {
#pragma unroll
    for (int q = 0; q < C::LPT; ++q) {
      const int i = tid + kThreads * q;
      const int key = i / C::CPK, c = i % C::CPK;
      *reinterpret_cast<u32x4*>(lds_k[buf] + key * C::ROWB + 16 * (c ^ (key & (C::CPK - 1)))) = pre[q];
    }
    if constexpr (FP8) {
      if (tid < PPT) {
        const int lp = j * C::KT / kPage + tid;
        lds_ksc[buf][tid] = (lp * kPage < lds_len[b]) ? a.k_scale[page_of(lds_tstart[b] + j, b, lp)] : 0.f;
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
#pragma unroll
      for (int kk = 0; kk < C::KS; ++kk) {
        if constexpr (FP8) {
          const long bf = *reinterpret_cast<const long*>(
              lds_k[buf] + kt * C::ROWB + 16 * (kk ^ (kt & (C::CPK - 1))) + 8 * hh);
#pragma unroll
          for (int m = 0; m < C::MB; ++m) acc[m] = mfma_fp8(afrag[m][kk], bf, acc[m]);
        } else {
          const bf16x8 bf = as_bf16x8(*reinterpret_cast<const u32x4*>(
              lds_k[buf] + kt * C::ROWB + 16 * ((2 * kk + hh) ^ (kt & (C::CPK - 1)))));
#pragma unroll
          for (int m = 0; m < C::MB; ++m) acc[m] = mfma_bf16(afrag[m][kk], bf, acc[m]);
        }
      }
      float part = 0.f;
#pragma unroll
      for (int m = 0; m < C::MB; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) part = fmaf(wreg[m][r], fmaxf(acc[m][r], 0.f), part);
      part += __shfl_xor(part, 32, 64);
      if constexpr (FP8) part *= lds_ksc[buf][kt / kPage];
      const int s = j * C::KT + kt;
      if (hh == 0 && s < n_me) {
        const uint32_t key = float_key(part);
        a.keys[row * a.row_stride + s] = key;
        atomicAdd(&lds_hist[qi * kBins + (key >> 21)], 1u);
      }
    }
  };

  for (int i = tid; i < TQ * kBins; i += kThreads) lds_hist[i] = 0u;
  issue(lo, pre0, pb0, pj0);
  if (n_items > 1) issue(lo + 1, pre1, pb1, pj1);
  int b_cur = -1;
  auto step = [&](int i, u32x4 (&pre)[C::LPT], int& pb, int& pj, int buf) {
    commit(pre, buf, pb, pj);
    const int b = pb, j = pj;
    lds_barrier();                    // keeps the next tile's loads in flight
    if (b != b_cur) {                 // new sequence: publish the old histogram, load new q
      if (b_cur >= 0) flush(b_cur);
      load_q(b);
      b_cur = b;
      lds_barrier();
    }
    if (i + 2 < n_items) issue(lo + i + 2, pre, pb, pj);
    compute(buf, b, j);
  };
  for (int i = 0; i < n_items; i += 2) {
    step(i, pre0, pb0, pj0, 0);
    if (i + 1 < n_items) step(i + 1, pre1, pb1, pj1, 1);
  }
  __syncthreads();
  flush(b_cur);
}

// ------------------------------------------------------------------------------------------------
// Finds the bin holding the need-th largest element of a histogram of NB bins (bins ordered by
// key).  Returns the bin and, through `above`, the number of elements in higher bins.  All threads
// of the workgroup get the result.  `sh` needs kThreads/64 + 2 words.
template <int NB, int NT = kThreads>
__device__ __forceinline__ int find_bin(const uint32_t* hist, uint32_t need, uint32_t* sh, uint32_t& above) {
  constexpr int PER = NB / NT;          // bins per thread; thread 0 owns the highest bins
  static_assert(PER >= 1 && NB % NT == 0, "bins per thread");
  const int tid = threadIdx.x;
  const int hi = NB - PER * tid;       // exclusive upper end of my bins
  uint32_t mine = 0;
  if (tid == 0) { sh[NT / 64] = 0u; sh[NT / 64 + 1] = 0u; }
#pragma unroll
  for (int i = 1; i <= PER; ++i) mine += hist[hi - i];
  uint32_t tot;
  const uint32_t pre = block_exclusive_scan<NT>(mine, sh, tot);
  if (pre < need && pre + mine >= need) {
    uint32_t run = pre;
#pragma unroll
    for (int i = 1; i <= PER; ++i) {
      const uint32_t h = hist[hi - i];
      if (run < need && run + h >= need) {
        sh[NT / 64] = hi - i;
        sh[NT / 64 + 1] = run;
      }
      run += h;
    }
  }
  __syncthreads();
  const int bin = (int)sh[NT / 64];
  above = sh[NT / 64 + 1];
  __syncthreads();
  return bin;
}

struct SelectArgs {
  const uint32_t* keys;
  const uint32_t* hist;
  const int32_t* seq_lens;
  int32_t* gt_pos;      // [rows, n_slices, gt_cap]
  uint2* cand;          // [rows, n_slices, kSlice]  (key, position)
  int32_t* cnt;         // [rows, n_slices, 2]
  int32_t* idx_out;     // [rows, K]
  int T, max_pages, K, n_slices, row_stride, gt_cap, max_seq_len;
};

__global__ __launch_bounds__(256) void li_select_split(SelectArgs a) {
  __shared__ uint32_t sh_hist[kBins];
  __shared__ uint32_t sh[8];
  const int tid = threadIdx.x;
  const int row = blockIdx.x, slice = blockIdx.y;
  const int b = row / a.T, t = row % a.T;
  const int n = row_visible(a.seq_lens, b, a.T, t, a.max_seq_len);
  if (n <= a.K || slice * kSlice >= n) return;
  const uint32_t kp = (uint32_t)min(a.K, n);

  // the slice's keys (16 consecutive per thread) load while the histogram is scanned
  constexpr int PT = kSlice / kThreads;
  const int s0 = slice * kSlice + tid * PT;
  uint32_t kv[PT];
#pragma unroll
  for (int j = 0; j < PT / 4; ++j) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(a.keys + (size_t)row * a.row_stride + s0 + 4 * j);
    kv[4 * j] = v[0]; kv[4 * j + 1] = v[1]; kv[4 * j + 2] = v[2]; kv[4 * j + 3] = v[3];
  }
  for (int i = tid; i < kBins; i += kThreads) sh_hist[i] = a.hist[(size_t)row * kBins + i];
  __syncthreads();
  uint32_t above;
  const uint32_t b1 = (uint32_t)find_bin<kBins>(sh_hist, kp, sh, above);

  // ordered compaction of this slice
  uint32_t ngt = 0, nc = 0;
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const bool ok = s0 + j < n;
    const uint32_t d = kv[j] >> 21;
    ngt += (ok && d > b1) ? 1u : 0u;
    nc += (ok && d == b1) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t pre = block_exclusive_scan<kThreads>(ngt | (nc << 16), sh, tot);
  uint32_t og = pre & 0xFFFFu, oc = pre >> 16;
  const size_t sl = (size_t)row * a.n_slices + slice;
  int32_t* gt_out = a.gt_pos + sl * a.gt_cap;
  uint2* c_out = a.cand + sl * kSlice;
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const int s = s0 + j;
    const bool ok = s < n;
    const uint32_t d = kv[j] >> 21;
    if (ok && d > b1 && og < (uint32_t)a.gt_cap) gt_out[og++] = s;
    if (ok && d == b1 && oc < (uint32_t)kSlice) c_out[oc++] = make_uint2(kv[j], (uint32_t)s);
  }
  if (tid == 0) {
    a.cnt[sl * 2] = (int32_t)(tot & 0xFFFFu);
    a.cnt[sl * 2 + 1] = (int32_t)(tot >> 16);
  }
}

__device__ __forceinline__ int lower_bound_lds(const int32_t* v, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (v[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

constexpr int kSelThreads = 1024;
constexpr int kCandCap = 8192;     // candidates staged in LDS; more fall back to global reads

__global__ __launch_bounds__(1024) void li_select_final(SelectArgs a) {
  constexpr int NT = kSelThreads;
  __shared__ uint32_t sh_hist[kBins];
  __shared__ uint32_t sh[NT / 64 + 2];
  __shared__ int32_t off_g[kMaxSlices + 1], off_c[kMaxSlices + 1];
  __shared__ int32_t gt_list[DSA_MAX_TOP_K];
  __shared__ int32_t sel_list[DSA_MAX_TOP_K];
  __shared__ uint32_t c_key[kCandCap];
  __shared__ int32_t c_pos[kCandCap];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int b = row / a.T, t = row % a.T;
  const int n = row_visible(a.seq_lens, b, a.T, t, a.max_seq_len);
  int32_t* out = a.idx_out + (size_t)row * a.K;
  if (n <= a.K) {
    for (int j = tid; j < a.K; j += NT) out[j] = j < n ? j : -1;
    return;
  }
  const int kp = a.K;   // n > K
  const int S = (n + kSlice - 1) / kSlice;

  // slice offsets (S <= kMaxSlices <= NT)
  uint32_t g = 0, c = 0;
  if (tid < S) {
    const size_t sl = (size_t)row * a.n_slices + tid;
    g = (uint32_t)a.cnt[sl * 2];
    c = (uint32_t)a.cnt[sl * 2 + 1];
  }
  uint32_t G, Cn;
  const uint32_t og = block_exclusive_scan<NT>(g, sh, G);
  const uint32_t oc = block_exclusive_scan<NT>(c, sh, Cn);
  if (tid < S) { off_g[tid] = (int32_t)og; off_c[tid] = (int32_t)oc; }
  if (tid == 0) { off_g[S] = (int32_t)G; off_c[S] = (int32_t)Cn; }
  __syncthreads();
  auto slice_of = [&](const int32_t* off, int i) -> int {   // largest slice with off[slice] <= i
    int lo = 0, hi = S;
    while (hi - lo > 1) { const int mid = (lo + hi) >> 1; if (off[mid] <= i) lo = mid; else hi = mid; }
    return lo;
  };
  const uint2* cand = a.cand + (size_t)row * a.n_slices * kSlice;
  const bool staged = Cn <= (uint32_t)kCandCap;
  // one pass: candidates (position order) and the positions above the threshold bin into LDS
  if (staged) {
    for (int i = tid; i < (int)Cn; i += NT) {
      const int sl = slice_of(off_c, i);
      const uint2 e = cand[(size_t)sl * kSlice + (i - off_c[sl])];
      c_key[i] = e.x;
      c_pos[i] = (int32_t)e.y;
    }
  }
  for (int i = tid; i < (int)G && i < DSA_MAX_TOP_K; i += NT) {
    const int sl = slice_of(off_g, i);
    gt_list[i] = a.gt_pos[((size_t)row * a.n_slices + sl) * a.gt_cap + (i - off_g[sl])];
  }
  for (int i = tid; i < kBins; i += NT) sh_hist[i] = 0u;
  __syncthreads();
  auto key_at = [&](int i) -> uint32_t {
    if (staged) return c_key[i];
    const int sl = slice_of(off_c, i);
    return cand[(size_t)sl * kSlice + (i - off_c[sl])].x;
  };
  auto pos_at = [&](int i) -> int32_t {
    if (staged) return c_pos[i];
    const int sl = slice_of(off_c, i);
    return (int32_t)cand[(size_t)sl * kSlice + (i - off_c[sl])].y;
  };

  // refine the threshold: digit 2 = bits 20..10, digit 3 = bits 9..0
  uint32_t need = (uint32_t)kp - G;
  for (int i = tid; i < (int)Cn; i += NT) atomicAdd(&sh_hist[(key_at(i) >> 10) & 2047u], 1u);
  __syncthreads();
  uint32_t above;
  const uint32_t b2 = (uint32_t)find_bin<kBins, NT>(sh_hist, need, sh, above);
  need -= above;
  for (int i = tid; i < kBins; i += NT) sh_hist[i] = 0u;
  __syncthreads();
  for (int i = tid; i < (int)Cn; i += NT) {
    const uint32_t k = key_at(i);
    if (((k >> 10) & 2047u) == b2) atomicAdd(&sh_hist[k & 1023u], 1u);
  }
  const uint32_t b1 = Cn > 0 ? key_at(0) >> 21 : 0u;
  __syncthreads();
  const uint32_t b3 = (uint32_t)find_bin<1024, NT>(sh_hist, need, sh, above);
  need -= above;                           // ties of the threshold key to keep (>= 1)
  const uint32_t theta = (b1 << 21) | (b2 << 10) | b3;

  // candidates above theta, plus the first `need` ties in position order
  uint32_t run_sel = 0, run_tie = 0;
  for (int base = 0; base < (int)Cn; base += NT) {
    const int i = base + tid;
    uint32_t k = 0;
    int32_t p = 0;
    if (i < (int)Cn) { k = key_at(i); p = pos_at(i); }
    const bool tie = i < (int)Cn && k == theta;
    const bool above_t = i < (int)Cn && k > theta;
    uint32_t tot;
    const uint32_t pre = block_exclusive_scan<NT>((tie ? 1u : 0u) | (above_t ? 0x10000u : 0u), sh, tot);
    const uint32_t rank = run_tie + (pre & 0xFFFFu);          // ties before this one
    const uint32_t n_above = pre >> 16;                       // above-theta before this one (tile)
    const bool sel = above_t || (tie && rank < need);
    // selected before this one in the tile: all above-theta ones, plus ties with rank < need
    const uint32_t ties_sel_before = min(rank, need) - min(run_tie, need);
    const uint32_t pos = run_sel + n_above + ties_sel_before;
    if (sel && pos < DSA_MAX_TOP_K) sel_list[pos] = p;
    run_sel += (tot >> 16) + (min(run_tie + (tot & 0xFFFFu), need) - min(run_tie, need));
    run_tie += tot & 0xFFFFu;
  }
  __syncthreads();
  const int ng = min((int)G, a.K), ns = min((int)run_sel, a.K - ng);   // ng + ns == K
  for (int i = tid; i < ng; i += NT) {
    const int p = gt_list[i];
    out[i + lower_bound_lds(sel_list, ns, p)] = p;
  }
  for (int j = tid; j < ns; j += NT) {
    const int p = sel_list[j];
    out[j + lower_bound_lds(gt_list, ng, p)] = p;
  }
  for (int j = ng + ns + tid; j < a.K; j += NT) out[j] = -1;
}

// ------------------------------------------------------------------------------------------------
static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

IndexerPlan plan_indexer(const dsa_paged_layout& L, const dsa_indexer_shape& S) {
  IndexerPlan p;
  p.rows = L.batch * S.T;
  p.row_stride = (int)align_up((size_t)L.max_seq_len, kSlice);
  p.n_slices = p.row_stride / kSlice;
  p.gt_cap = S.top_k < kSlice ? S.top_k : kSlice;
  p.n_chunks = (L.max_seq_len + kChunkKeys - 1) / kChunkKeys;
  p.tq = S.T == 1 ? 1 : (S.T == 2 ? 2 : 4);
  p.n_qtiles = (S.T + p.tq - 1) / p.tq;
  size_t off = 0;
  p.off_hist = off; off = align_up(off + (size_t)p.rows * kBins * 4, 256);
  p.off_keys = off; off = align_up(off + (size_t)p.rows * p.row_stride * 4, 256);
  p.off_gt = off;   off = align_up(off + (size_t)p.rows * p.n_slices * p.gt_cap * 4, 256);
  p.off_cand = off; off = align_up(off + (size_t)p.rows * p.n_slices * kSlice * 8, 256);
  p.off_cnt = off;  off = align_up(off + (size_t)p.rows * p.n_slices * 2 * 4, 256);
  p.total = off;
  return p;
}

bool indexer_supported(int heads, int dim) {
  return (heads == 8 || heads == 16 || heads == 32 || heads == 64) && (dim == 64 || dim == 128);
}

template <int HI, int DI, bool FP8>
static void launch_score(const ScoreArgs& s, int tq, int grid, bool persist, hipStream_t st) {
  if (persist) {
    if (tq == 1) hipLaunchKernelGGL((li_score_persist<HI, DI, FP8, 1>), dim3(grid), dim3(kThreads), 0, st, s);
    else if (tq == 2) hipLaunchKernelGGL((li_score_persist<HI, DI, FP8, 2>), dim3(grid), dim3(kThreads), 0, st, s);
    else hipLaunchKernelGGL((li_score_persist<HI, DI, FP8, 4>), dim3(grid), dim3(kThreads), 0, st, s);
    return;
  }
  if (tq == 1) hipLaunchKernelGGL((li_score<HI, DI, FP8, 1>), dim3(grid), dim3(kThreads), 0, st, s);
  else if (tq == 2) hipLaunchKernelGGL((li_score<HI, DI, FP8, 2>), dim3(grid), dim3(kThreads), 0, st, s);
  else hipLaunchKernelGGL((li_score<HI, DI, FP8, 4>), dim3(grid), dim3(kThreads), 0, st, s);
}

template <int HI, int DI>
static void launch_score_dt(const ScoreArgs& s, bool fp8, int tq, int grid, bool persist, hipStream_t st) {
  if (fp8) launch_score<HI, DI, true>(s, tq, grid, persist, st);
  else launch_score<HI, DI, false>(s, tq, grid, persist, st);
}

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
  const size_t hist_words = (size_t)p.rows * kBins;
  const int zgrid = (int)std::min<size_t>((hist_words / 4 + 255) / 256, 2048);
  {
    LaunchScope ls("li_zero_hist", st);
    hipLaunchKernelGGL(li_zero_hist, dim3(zgrid), dim3(256), 0, st, hist, hist_words);
  }

  ScoreArgs s;
  s.q = static_cast<const unsigned char*>(a.q);
  s.q_scale = a.q_scale;
  s.w = a.w;
  s.kc = static_cast<const unsigned char*>(a.k_cache);
  s.k_scale = a.k_scale;
  s.block_table = a.block_table;
  s.seq_lens = a.seq_lens;
  s.keys = reinterpret_cast<uint32_t*>(ws + p.off_keys);
  s.hist = hist;
  s.B = a.B; s.T = a.T; s.max_pages = a.max_pages; s.num_pages = a.num_pages; s.K = a.top_k;
  s.n_chunks = p.n_chunks; s.n_qtiles = p.n_qtiles; s.row_stride = p.row_stride;
  s.max_seq_len = a.max_seq_len;
  const bool persist = a.T <= 4 && a.B <= kMaxSeqPersist;
  int grid = a.B * p.n_qtiles * p.n_chunks;
  if (persist) {
    const int kt = p.tq == 1 ? 128 : 64;
    const long long max_tiles = (long long)a.B * ((a.max_seq_len + kt - 1) / kt);
    grid = (int)std::max<long long>(1, std::min<long long>(2LL * device_cus(), (max_tiles + 1) / 2));
  }
  if (grid > 0) {
    LaunchScope ls("li_score", st);
    switch (a.heads * 1000 + a.dim) {
      case 8064: launch_score_dt<8, 64>(s, a.fp8, p.tq, grid, persist, st); break;
      case 8128: launch_score_dt<8, 128>(s, a.fp8, p.tq, grid, persist, st); break;
      case 16064: launch_score_dt<16, 64>(s, a.fp8, p.tq, grid, persist, st); break;
      case 16128: launch_score_dt<16, 128>(s, a.fp8, p.tq, grid, persist, st); break;
      case 32064: launch_score_dt<32, 64>(s, a.fp8, p.tq, grid, persist, st); break;
      case 32128: launch_score_dt<32, 128>(s, a.fp8, p.tq, grid, persist, st); break;
      case 64064: launch_score_dt<64, 64>(s, a.fp8, p.tq, grid, persist, st); break;
      case 64128: launch_score_dt<64, 128>(s, a.fp8, p.tq, grid, persist, st); break;
      default: return hipErrorInvalidValue;
    }
  }
  SelectArgs sa;
  sa.keys = s.keys;
  sa.hist = hist;
  sa.seq_lens = a.seq_lens;
  sa.gt_pos = reinterpret_cast<int32_t*>(ws + p.off_gt);
  sa.cand = reinterpret_cast<uint2*>(ws + p.off_cand);
  sa.cnt = reinterpret_cast<int32_t*>(ws + p.off_cnt);
  sa.idx_out = a.idx_out;
  sa.T = a.T; sa.max_pages = a.max_pages; sa.K = a.top_k; sa.n_slices = p.n_slices;
  sa.row_stride = p.row_stride; sa.gt_cap = p.gt_cap; sa.max_seq_len = a.max_seq_len;
  {
    LaunchScope ls("li_select_split", st);
    hipLaunchKernelGGL(li_select_split, dim3(p.rows, p.n_slices), dim3(kThreads), 0, st, sa);
  }
  {
    LaunchScope ls("li_select_final", st);
    hipLaunchKernelGGL(li_select_final, dim3(p.rows), dim3(kSelThreads), 0, st, sa);
  }
  return hipGetLastError();
}

}  // namespace dsa
