// sfa.hip -- Sparse Flash Attention over the selected MLA latent rows, for gfx950.
//
// Pages: "Inference Optimization for Kimi K3.1 Pro" §1 (DSA step 3: attend over the KV rows at
// the indexer's selected positions) and §2 (indices resolve to pages in place); "Optimizing Kimi
// K3.1 Pro Sparse Attention Inference", "Inheritance and Extension of Core Operators" (blockwise
// attention over fixed-size KV blocks, reduced across blocks without a global softmax).
//
// One workgroup handles one query row, up to 128 heads (one wave per 32 heads) and a contiguous
// range of the row's selected indices (a "split").  Per 32-index tile it gathers the 1152-byte
// latent rows (page-table resolved) into an LDS ring with direct-to-LDS loads, so every KV row is
// fetched once for all heads.  With the key tile as MFMA operand A and the wave's query rows (all
// 576 columns, held in VGPRs) as operand B it computes S^T = X q^T: each lane owns one head and
// 16 of the tile's keys, the other 16 sit in the lane 32 apart, so the online-softmax max and sum
// need one cross-half exchange, and the probabilities feed the value product O^T += V^T P^T as
// operand B without leaving the lane.  The value product reads V^T straight from the row-major
// tile with transposed LDS reads.  The accumulator O^T (512 x 32 per wave, 256 registers) lives in
// the accumulation registers; the running max is kept in the log2 domain (exp2 with log2(e) folded
// into the scale).  With one split the workgroup normalises and writes bf16 output and the
// natural-log LSE; with several, each writes (m, l, O) partials and sfa_combine merges them:
// M = max m_i, L = sum_i 2^(m_i - M) l_i, O = sum_i 2^(m_i - M) O_i / L.
//
// FP8 latent cache ([P1] §4: the SFA cache in FP8 with per-token scales over 128-wide tiles, BF16
// products, the dequantised BF16 tile filling the matrix unit's input buffer directly): rows are
// 576 E4M3 codes plus 8 fp32 scales per token (tiles 0-127, 128-255, 256-383, 384-511, 512-575;
// 3 unused).  The gather ring then holds the raw codes and scales, and each tile is dequantised
// (float32 product, bf16 rounding) straight into the same swizzled bf16 tile the bf16 cache is
// gathered into, so the products run unchanged.
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
constexpr float kRefMargin = 64.f;         // reference max = first tile's max + this (log2 units)
constexpr float kRefLimit = 100.f;         // a logit above reference + this restarts the split

struct SfaArgs {
  const unsigned char* q;       // [rows, H, 576] bf16
  const unsigned char* kv;      // [P, 64, 576] bf16, or E4M3 codes for the fp8 cache
  const unsigned char* kv_sc;   // fp8 cache: [P, 64, 8] fp32 tile scales (32 bytes per token)
  const int32_t* idx;           // [rows, K]
  const int32_t* block_table;
  const int32_t* seq_lens;
  __bf16* out;                  // [rows, H, 512]
  float* lse;                   // [rows, H] or null
  float* part_ml;               // [rows, splits, H, 2]
  uint32_t* part_o;             // [rows, splits, head groups, 16 blocks, 2 halves, 64 lanes, 4] bf16 pairs
  int T, H, K, max_pages, num_pages, n_splits, keys_per_split, max_seq_len;
  float scale_log2;             // sm_scale * log2(e)
};

// LDS layout of a gathered tile (36864 bytes) in two regions:
//   A: the 512 value columns of each row, 1024 bytes (64 chunks of 16 bytes), row r at 1024*r;
//   B: the 64 rope columns, 128 bytes (8 chunks), row r at kRegionB + 128*r.
// Chunk c of row r sits at slot c ^ swa(r) in A and c ^ swb(r) in B.  A region-A row is exactly
// one wave-wide direct-to-LDS load (64 lanes x 16 bytes), so a gather is one scalar-addressed load
// per row.  The XORs keep the reads free of bank conflicts (16-byte slots, 16 per 256-byte bank
// cycle): the score product's 16 lanes read one chunk of 16 consecutive rows, and swa is a
// permutation of the row's low four bits; the value product's transposed 8-byte reads take 2
// chunks (c, c^1) of 4 consecutive rows, and swa >> 1 differs between those rows.
constexpr int kRegionB = 32768;
__device__ __forceinline__ int swa(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3); }
__device__ __forceinline__ int swb(int r) { return (r >> 1) & 7; }


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two floats to packed bf16 (round to nearest even) with gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

constexpr int kTileBytes = kBK * kRowBytes;          // 36864
constexpr int kDmaPerTile = kTileBytes / 1024;       // 36 wave-wide loads: 32 value rows + 4 rope blocks
constexpr int kStages = 4;                           // gather ring depth (the main loop is unrolled by it)
constexpr int kRingA = 4;                            // score-product A fragments in flight (LDS reads)
constexpr int kRingV = 4;                            // value-product A fragments in flight (deeper spills)
constexpr int kMaxSplitKeys = DSA_MAX_TOP_K;

// FP8 cache tile in the gather ring: the 32 rows' codes (576 bytes each) then their scale rows
// (32 bytes each), as 16-byte chunks in order: 1152 code chunks + 64 scale chunks, one spare
// wave-wide load to make 20 (a multiple of every wave count).  The bf16 tile the products read sits
// in the first kTileBytes of the ring; the fp8 slots follow it.
constexpr int kRowBytes8 = kDimQK;                      // 576
constexpr int kCodeChunks8 = kBK * kRowBytes8 / 16;     // 1152
constexpr int kChunks8 = kCodeChunks8 + kBK * 2;        // 1216
constexpr int kDmaPerTile8 = 20;
constexpr int kSlotBytes8 = kDmaPerTile8 * 1024;        // 20480
static_assert(kDmaPerTile8 * 64 >= kChunks8 && kTileBytes + 4 * kSlotBytes8 <= 4 * kTileBytes, "fp8 ring");

// Waits until this wave's loads of the tile being consumed have landed; `later` of its later
// tiles (n loads each) may stay in flight.
template <int n>
__device__ __forceinline__ void wait_ring(int later) {
  if (later >= 2) wait_vmcnt<(2 * n > 63 ? 63 : 2 * n)>();   // the counter saturates at 63
  else if (later == 1) wait_vmcnt<n>();
  else wait_vmcnt<0>();
}

template <int NW, bool KV8 = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sfa_main(SfaArgs a) {
  constexpr int NT = NW * 64;               // one wave per 32-head group
  constexpr int kDmaWave = (KV8 ? kDmaPerTile8 : kDmaPerTile) / NW;
  static_assert(kDmaPerTile % NW == 0 && kDmaPerTile8 % NW == 0, "per-wave load count must be uniform");
  static_assert(kStages - 2 <= 2, "wait_ring handles up to two later tiles");
  __shared__ __attribute__((aligned(1024))) unsigned char lds_kv[kStages][kTileBytes];
  __shared__ int lds_rows[kMaxSplitKeys];   // physical row of each selected index, -1 = skip

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: LDS DMA bases stay in SGPRs
  const int nl = lane & 31, hh = lane >> 5;
  const int row = blockIdx.x, split = blockIdx.y;
  const int NGT = (a.H + 31) / 32;          // 32-head groups over all workgroups of a row
  const int gg = blockIdx.z * NW + wave;    // this wave's global head group
  const int b = row / a.T, t = row % a.T;
  const int n = row_visible(a.seq_lens, b, a.T, t, a.max_seq_len);
  const int k_begin = split * a.keys_per_split;
  const int k_end = min(a.K, k_begin + a.keys_per_split);
  const int nkeys = k_end - k_begin;
  const int ntiles = (nkeys + kBK - 1) / kBK;
  const int head = gg * 32 + nl;
  const bool hvalid = head < a.H;

  // Row table for this split (one round of idx + block-table loads): lds_rows[j] = physical row
  // of selected index j, -1 if it is not a visible position; lds_valid[tile] = its 32-bit mask.
  __shared__ int lds_fill;                  // first j with a visible position
  __shared__ uint32_t lds_valid[kMaxSplitKeys / kBK];
  __shared__ int lds_epoch;                 // restarts requested by any wave (see below)
  if (tid == 0) { lds_fill = kMaxSplitKeys; lds_epoch = 0; }
  const int32_t* idx = a.idx + (size_t)row * a.K + k_begin;
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;
  // The first round of index loads goes out first: the index -> page-table chain then overlaps
  // the q loads below.
  const int s_first = tid < nkeys ? idx[tid] : -1;

  // B operand of the score product: this lane's head row of q (36 K steps of 16 columns).  The
  // workgroup's q rows (NW * 32 heads x 1152 bytes = NW ring slots, free until the first gathers)
  // are first copied into LDS with direct-to-LDS loads that each read eight whole 128-byte lines;
  // read straight into the MFMA layout, every load instruction would touch 32 rows, a quarter of
  // a line each.  16-byte chunk c of head h sits at slot 72h + (c ^ ((h >> 1) & 7)): the XOR stays
  // inside a 128-byte line and makes the fragment reads (16 lanes = 16 heads, one chunk) free of
  // bank conflicts.  Heads beyond H copy head 0; their results are never stored.
  bf16x8 qf[kQSteps];
  unsigned char* const q_img = &lds_kv[0][0];
  {
    const unsigned char* qrow = a.q + (size_t)row * a.H * kRowBytes;
    const int head0 = blockIdx.z * NW * 32;
#pragma unroll 4
    for (int u = 0; u < kQSteps; ++u) {
      const int i = wave * kQSteps + u;        // this load fills q image bytes 1024*i ..
      const int sl = 64 * i + lane;
      const int hl = sl / 72, cp = sl % 72;
      const int hq = head0 + hl < a.H ? head0 + hl : 0;
      lds_dma16(qrow + (size_t)hq * kRowBytes + 16 * (cp ^ ((hl >> 1) & 7)), q_img + 1024 * i);
    }
  }
  lds_barrier();
  for (int j = tid; j < ntiles * kBK; j += NT) {   // NT is a multiple of 64: whole waves
    const int s = j == tid ? s_first : (j < nkeys ? idx[j] : -1);
    if (s < -1 || s >= n) flag_input(kFlagIndex);
    const int r = s >= 0 && s < n ? clamp_page(bt[s / kPage], a.num_pages) * kPage + (s % kPage) : -1;
    lds_rows[j] = r;
    const uint64_t bal = __ballot(r >= 0);
    if ((lane & 31) == 0) lds_valid[j >> 5] = (uint32_t)(bal >> (lane & 32));
    if (r >= 0) atomicMin(&lds_fill, j);
  }
  // the table's loads and this wave's q image loads have landed (vmcnt 0) ... for every wave
  __builtin_amdgcn_s_waitcnt(0x0F70);
  lds_barrier();
  // Keys that are not selected are gathered from the split's first selected row (finite data, so
  // their zero probabilities never meet a NaN); a split without any selected key skips its tiles.
  const int fill_j = lds_fill;
  const int fill_row = fill_j < kMaxSplitKeys ? lds_rows[fill_j] : 0;
  const int ntiles_run = fill_j < kMaxSplitKeys ? ntiles : 0;
  {
    const int h = wave * 32 + nl;
    const unsigned char* qh = q_img + h * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qh + 16 * ((2 * ks + hh) ^ ((h >> 1) & 7))));
  }
  lds_barrier();                            // every wave holds its q: the ring is free

  // Gather tile `tile` into ring slot `buf`.  This wave loads the value columns of rows
  // wave, wave + NW, ... (one load per row: the row id is wave-uniform, so the row's address is a
  // scalar base and each lane adds its own swizzled 16-byte chunk) and the rope blocks
  // wave, wave + NW, ... < 4 (8 rows x 8 chunks per load, lane i: row 8k + i/8, slot i%8).  Every
  // wave issues the same number of loads per tile, which the ring's counter waits rely on.
  constexpr int kRows = kBK / NW, kRope = 4 / NW;
  auto gather_row = [&](int pr, int buf, int u) __attribute__((always_inline)) {   // pr: physical row (wave-uniform) or -1
    const int r = wave + u * NW;
    pr = pr < 0 ? fill_row : pr;
    lds_dma16_rows(a.kv + (size_t)(uint32_t)pr * kRowBytes, (uint32_t)(16 * lane) ^ (uint32_t)(16 * swa(r)),
                   lds_kv[buf] + 1024 * r);
  };
  auto gather_rope = [&](int pr, int buf, int u) __attribute__((always_inline)) {  // pr: this lane's row, read by rope_row()
    const int k = wave + u * NW;
    const int r = 8 * k + (lane >> 3);
    pr = pr < 0 ? fill_row : pr;
    const unsigned char* src = a.kv + (size_t)(uint32_t)pr * kRowBytes + 2 * kDimV + 16 * ((lane & 7) ^ swb(r));
    lds_dma16(src, lds_kv[buf] + kRegionB + 1024 * k);
  };
  auto rope_row = [&](int tile, int u) __attribute__((always_inline)) { return lds_rows[tile * kBK + 8 * (wave + u * NW) + (lane >> 3)]; };
  // fp8 cache: load L = u * NW + wave of the tile covers 16-byte chunks 64L .. 64L + 63 (lane i:
  // chunk 64L + i): code chunk c of row r for k < 1152 (k = 36r + c), then the two scale chunks of
  // each row, then a spare load that rereads fill_row's codes into the slot's unused tail.
  auto issue8 = [&](int tile, int buf) __attribute__((always_inline)) {
    unsigned char* slot = &lds_kv[0][0] + kTileBytes + kSlotBytes8 * buf;
    int ln = lane;                          // opaque: keeps the per-load offsets out of the tile loop
    asm volatile("" : "+v"(ln));
    int prs[kDmaWave];                      // the tile's row-table reads go out together
#pragma unroll
    for (int u = 0; u < kDmaWave; ++u) {
      const int k = 64 * (u * NW + wave) + ln;
      const int r = k < kCodeChunks8 ? k / 36 : (k < kChunks8 ? (k - kCodeChunks8) >> 1 : 0);
      prs[u] = k < kChunks8 ? lds_rows[tile * kBK + r] : -1;
    }
#pragma unroll
    for (int u = 0; u < kDmaWave; ++u) {
      const int L = u * NW + wave;
      const int k = 64 * L + ln;
      const int pr = prs[u] < 0 ? fill_row : prs[u];
      const unsigned char* src = k < kCodeChunks8
          ? a.kv + (size_t)(uint32_t)pr * kRowBytes8 + 16 * (k % 36)
          : (k < kChunks8 ? a.kv_sc + (size_t)(uint32_t)pr * 32 + 16 * ((k - kCodeChunks8) & 1)
                          : a.kv + (size_t)(uint32_t)pr * kRowBytes8 + 16 * (ln % 36));
      lds_dma16(src, slot + 1024 * L);
    }
  };
  // fp8 cache: dequantise ring slot `buf` into the bf16 tile.  Value part: lane l converts codes
  // 8l..8l+7 (bf16 chunk l) of rows wave, wave + NW, ...: the row is wave-uniform, so its swizzle
  // and scale address are too.  Rope part: thread t converts chunk t % 8 of row t / 8 (NT <= 256:
  // 256 / NT rounds).  All LDS reads go out before the first conversion (one wave per SIMD: nothing
  // else hides their latency), and no offset needs a division or a branch.
  constexpr int kValRows = kBK / NW;                      // value rows per wave
  constexpr int kRopeRounds = (kBK * 8) / NT;             // rope units per thread
  auto cvt8 = [&](const uint2 w, float sc) __attribute__((always_inline)) {
    u32x4 o8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t word = h ? w.y : w.x;
      const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
      const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
      o8[2 * h] = pack_bf16(lo[0] * sc, lo[1] * sc);
      o8[2 * h + 1] = pack_bf16(hi[0] * sc, hi[1] * sc);
    }
    return o8;
  };
  auto dequant8 = [&](int buf) __attribute__((always_inline)) {
    const unsigned char* slot = &lds_kv[0][0] + kTileBytes + kSlotBytes8 * buf;
    unsigned char* dst = &lds_kv[0][0];
    // opaque copies of the thread ids: offsets hoisted out of the tile loop would hold registers
    // across the products
    int ln = lane, td = tid;
    asm volatile("" : "+v"(ln), "+v"(td));
    constexpr int VB = kValRows < 8 ? kValRows : 8;        // value rows per batch of reads
#pragma unroll
    for (int j0 = 0; j0 < kValRows; j0 += VB) {
      uint2 wv[VB];
      float sv[VB];
#pragma unroll
      for (int j = 0; j < VB; ++j) {
        const int r = wave + NW * (j0 + j);
        wv[j] = *reinterpret_cast<const uint2*>(slot + kRowBytes8 * r + 8 * ln);
        sv[j] = *reinterpret_cast<const float*>(slot + kBK * kRowBytes8 + 32 * r + 4 * (ln >> 4));
      }
#pragma unroll
      for (int j = 0; j < VB; ++j) {
        const int r = wave + NW * (j0 + j);
        *reinterpret_cast<u32x4*>(dst + 1024 * r + 16 * (ln ^ swa(r))) = cvt8(wv[j], sv[j]);
      }
    }
    uint2 wr[kRopeRounds];
    float sr[kRopeRounds];
#pragma unroll
    for (int j = 0; j < kRopeRounds; ++j) {
      const int u = td + NT * j, r = u >> 3;
      wr[j] = *reinterpret_cast<const uint2*>(slot + kRowBytes8 * r + kDimV + 8 * (u & 7));
      sr[j] = *reinterpret_cast<const float*>(slot + kBK * kRowBytes8 + 32 * r + 16);
    }
#pragma unroll
    for (int j = 0; j < kRopeRounds; ++j) {
      const int u = td + NT * j, r = u >> 3;
      *reinterpret_cast<u32x4*>(dst + kRegionB + 128 * r + 16 * ((u & 7) ^ swb(r))) = cvt8(wr[j], sr[j]);
    }
  };
  auto issue = [&](int tile, int buf) __attribute__((always_inline)) {
    if constexpr (KV8) { issue8(tile, buf); return; }
    int prow[kRows];                        // read together, made scalar one at a time
#pragma unroll
    for (int u = 0; u < kRows; ++u) prow[u] = lds_rows[tile * kBK + wave + u * NW];
#pragma unroll
    for (int u = 0; u < kRope; ++u) gather_rope(rope_row(tile, u), buf, u);
#pragma unroll
    for (int u = 0; u < kRows; ++u) gather_row(__builtin_amdgcn_readfirstlane(prow[u]), buf, u);
  };

  // O^T: 512 latent columns (16 blocks of 32) x 32 heads
  f32x16 o[kVBlocks];
#pragma unroll
  for (int mb = 0; mb < kVBlocks; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  // Fixed softmax reference per head (log2 units), set from the first tile with a valid key:
  // its max plus kRefMargin.  Probabilities 2^(s - m_ref) stay below 2^kRefLimit as long as no
  // logit exceeds m_ref + kRefLimit, so the accumulator never needs rescaling.  A logit beyond
  // that (a spread of more than 164 log2 units inside the row) raises the reference and restarts
  // the split from its first tile.  The finite floor keeps masked (-inf) logits at probability 0.
  constexpr float kNoRef = -1e30f;
  float m_run = kNoRef, l_run = 0.f;
  int epoch = 0;                            // restarts seen by this wave

  // Per-lane LDS byte offsets.  Score A operand: row nl, chunk c = 2*ks + hh.  For ks < 32
  // (region A) write ks = 8g + v: the slot is 16g + ((2v + hh) ^ swa), i.e. byte
  // 256g + 16*((hh ^ swa) & 1) + 32*(v ^ (swa >> 1)); the last term only uses bits 5-7, so the
  // address is qa ^ 32v (+ 256g).  Region B likewise: qb ^ 32v' for ks = 32 + v'.
  const int sa_nl = swa(nl), sb_nl = swb(nl);
  const int qa = 1024 * nl + 16 * ((hh ^ sa_nl) & 1) + 32 * (sa_nl >> 1);
  const int qb = kRegionB + 128 * nl + 16 * ((hh ^ sb_nl) & 1) + 32 * (sb_nl >> 1);
  // Value A operand (transposed 8-byte reads): key = 16*k2 + 8*q + kq, columns 8*cl + 4*(lane&1)
  // + 32*mb, cl = chunk within the 32-column block.  With mb = 4g + m' the byte offset is
  // 16384*k2 + 256g + (pv[q] ^ 64m'): swa(key) only sees key bits 0-3 = 8q + kq.
  const int kq = 4 * hh + ((lane & 15) >> 2);
  const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  int pv[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int sa = swa(8 * q + kq);
    pv[q] = 1024 * (8 * q + kq) + 16 * (cl ^ (sa & 3)) + 64 * (sa >> 2) + 8 * (lane & 1);
  }

  // One tile of the main loop.  The ring slot is a compile-time constant (the loop is unrolled by
  // the ring depth), so every LDS address below is a per-lane base plus an immediate offset.
  auto step = [&](int it, auto slot) {
    constexpr int buf = decltype(slot)::value;
    wait_ring<kDmaWave>(min(kStages - 2, ntiles_run - 1 - it));
    lds_barrier();                          // tile `it` landed for every wave; slot it-1 is free
    if (it + kStages - 1 < ntiles_run) issue(it + kStages - 1, (buf + kStages - 1) % kStages);
    if constexpr (KV8) {                    // every wave is past the previous tile's products
      dequant8(buf);
      lds_barrier();
    }
    const unsigned char* tile = KV8 ? lds_kv[0] : lds_kv[buf];
    const uint32_t valid = lds_valid[it];

    // S^T = X q^T: rows = the tile's 32 keys, columns = this wave's 32 heads.  The A fragments
    // stream through a 4-deep register ring: the read for step ks + 4 is issued right behind the
    // MFMA of step ks, so LDS latency hides under the MFMAs in between.
    // The XOR-ed offsets are formed per read (one VALU op each) from bases the compiler may not
    // hoist: precomputing all 36 + 64 of them would hold that many registers across the loop.
    int qa_t = qa, qb_t = qb, pv0 = pv[0], pv1 = pv[1];
    asm volatile("" : "+v"(qa_t), "+v"(qb_t), "+v"(pv0), "+v"(pv1));
    auto a_frag = [&](int ks) {
      const int off = ks < 32 ? (qa_t ^ (32 * (ks & 7))) + 256 * (ks >> 3) : qb_t ^ (32 * (ks - 32));
      return *reinterpret_cast<const u32x4*>(tile + off);
    };
    auto v_frag = [&](int j, int q) {     // j = 16*k2 + mb
      const int mb = j & 15;
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(
          tile + ((q ? pv1 : pv0) ^ (64 * (mb & 3))) + 256 * (mb >> 2) + 16384 * (j >> 4)));
    };
    u32x4 aring[kRingA];
#pragma unroll
    for (int j = 0; j < kRingA; ++j) aring[j] = a_frag(j);
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks) {
      const bf16x8 af = as_bf16x8(aring[ks % kRingA]);
      if (ks + kRingA < kQSteps) aring[ks % kRingA] = a_frag(ks + kRingA);
      s = mfma_bf16(af, qf[ks], s);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first value-product fragments load while the softmax runs
    s16x4 vring[kRingV][2];
#pragma unroll
    for (int j = 0; j < kRingV; ++j) { vring[j][0] = v_frag(j, 0); vring[j][1] = v_frag(j, 1); }

    // Online softmax over the 16 keys this lane holds (+ the other half-wave's 16).  The
    // probabilities 2^(s - m_ref) need only the fixed reference, not this tile's max, which serves
    // the first tile (it sets the reference) and the restart check.  So the keys of the value
    // product's first K step are exponentiated right away and the rest of the softmax (the other 8
    // exponentials, the sums, the cross-half max) runs between its MFMAs, under the matrix pipe.
    // A restart discards this pass, so a tile exponentiated against a reference it then raises
    // never reaches the output.
    float mloc = -INFINITY;
    if (valid == 0xFFFFFFFFu) {             // wave-uniform: every key of the tile is selected
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] *= a.scale_log2;
        mloc = fmaxf(mloc, s[r]);
      }
    } else {
      const uint32_t vmask = valid >> (4 * hh);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + (r & 3);        // + 4*hh, folded into `vmask`
        s[r] = ((vmask >> key) & 1u) ? s[r] * a.scale_log2 : -INFINITY;
        mloc = fmaxf(mloc, s[r]);
      }
    }
    // every lane sets its reference on the same tile (the first with a selected key): uniform
    if (__builtin_amdgcn_readfirstlane(m_run == kNoRef ? 1 : 0)) {
      const float m0 = xor32_max(mloc);
      if (m0 > -INFINITY) m_run = m0 + kRefMargin;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) s[r] = __builtin_amdgcn_exp2f(s[r] - m_run);
    // P^T as the B operand of the value product: K step k2 covers keys 16*k2 .. 16*k2 + 15; this
    // lane's 8 values are keys 16*k2 + {0..3, 8..11} + 4*hh (accumulator rows of the score tile)
    auto pack_p = [&](int k2) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = pack_bf16(s[8 * k2 + 2 * e], s[8 * k2 + 2 * e + 1]);
      return as_bf16x8(v);
    };
    bf16x8 pf[2];
    pf[0] = pack_p(0);
    float mx = mloc, psum = 0.f;
    // O^T += V^T P^T.  The A operand (latent column m, the same 8 keys) comes from two transposed
    // reads of the row-major tile: a 16-lane group reading 8 bytes (4 columns) of 4 consecutive
    // keys hands lane i the 4 keys of column i.  Same 4-deep ring as the score product;
    // consecutive MFMAs go to different accumulators.
#pragma unroll
    for (int j = 0; j < 2 * kVBlocks; ++j) {
      const int k2 = j >> 4, mb = j & 15;
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vring[j % kRingV][0], vring[j % kRingV][1], 0, 1, 2, 3, 4, 5, 6, 7));
      if (j + kRingV < 2 * kVBlocks) {
        vring[j % kRingV][0] = v_frag(j + kRingV, 0);
        vring[j % kRingV][1] = v_frag(j + kRingV, 1);
      }
      o[mb] = mfma_bf16(vf, pf[k2], o[mb]);
      // the rest of the softmax, one slice after each MFMA of the first K step
      if (j < 8) {
        s[8 + j] = __builtin_amdgcn_exp2f(s[8 + j] - m_run);
      } else if (j == 8) {
        pf[1] = pack_p(1);
      } else if (j == 9) {
#pragma unroll
        for (int r = 0; r < 16; ++r) psum += s[r];
      } else if (j == 10) {
        psum = xor32_sum(psum);
        mx = xor32_max(mx);
      } else if (j == 11) {
        l_run += psum;
        if (mx > m_run + kRefLimit) {       // too far above the reference: restart with a new one
          m_run = mx + kRefMargin;
          lds_epoch = epoch + 1;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // First gathers; the first step waits for tile 0 alone and computes while tiles 1 and 2 land.
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (i < ntiles_run) issue(i, i);
  for (;;) {
    for (int it = 0; it < ntiles_run; it += kStages) {
      step(it, std::integral_constant<int, 0>{});
      if (it + 1 < ntiles_run) step(it + 1, std::integral_constant<int, 1>{});
      if (it + 2 < ntiles_run) step(it + 2, std::integral_constant<int, 2>{});
      if (it + 3 < ntiles_run) step(it + 3, std::integral_constant<int, 3>{});
    }
    static_assert(kStages == 4, "the main loop above is unrolled for a 4-slot ring");
    // every wave sees the same restart request after the barrier; the gathers of this pass have
    // all been waited for (the last step waits for vmcnt 0)
    lds_barrier();
    const int req = lds_epoch;
    if (req == epoch) break;
    epoch = req;                            // raised references stay; accumulation starts over
    l_run = 0.f;
#pragma unroll
    for (int mb = 0; mb < kVBlocks; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
    lds_barrier();                          // all waves read the request before slot 0 is refilled
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i)
      if (i < ntiles_run) issue(i, i);
  }
  if (a.n_splits == 1) {
    if (hvalid) {
      const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + ((size_t)row * a.H + head) * kDimV;
#pragma unroll
      for (int mb = 0; mb < kVBlocks; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d = 32 * mb + 8 * j + 4 * hh;
          uint2 v;
          v.x = pack_bf16(o[mb][4 * j] * inv, o[mb][4 * j + 1] * inv);
          v.y = pack_bf16(o[mb][4 * j + 2] * inv, o[mb][4 * j + 3] * inv);
          *reinterpret_cast<uint2*>(dst + d) = v;
        }
      if (a.lse != nullptr && hh == 0)
        a.lse[(size_t)row * a.H + head] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
    }
  } else {
    const size_t ps = (size_t)row * a.n_splits + split;
    if (hvalid && hh == 0) {
      a.part_ml[(ps * a.H + head) * 2] = m_run;
      a.part_ml[(ps * a.H + head) * 2 + 1] = l_run;
    }
    // Partial O (not divided by l: the combine folds 1/l into its weights) as bf16 pairs
    // (registers 2k, 2k+1) in the accumulator's own lane order, [head group][block][half][lane]
    // [4 pairs]: each store instruction writes 1 KB contiguous (16 bytes per lane).  Half the
    // bytes of fp32 partials; bf16 keeps 2^-9 relative to each value, far inside the output
    // tolerance, and its range covers the accumulator's (probabilities stay below 2^kRefLimit).
    if (gg >= NGT) return;
    uint32_t* dst = a.part_o + ((ps * NGT + gg) * kVBlocks) * 8 * 64;
#pragma unroll
    for (int mb = 0; mb < kVBlocks; ++mb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = 4 * half + q;
          v[q] = pack_bf16(o[mb][2 * k], o[mb][2 * k + 1]);
        }
        *reinterpret_cast<u32x4*>(dst + ((mb * 2 + half) * 64 + lane) * 4) = v;
      }
  }
}

// Merges the split partials.  Grid (query row, 32-head group, chunk): the 8*SG chunks of a
// (row, group) share its 8192 bf16 pairs, 4 pairs (one 16-byte load) of one head per thread;
// with SG > 1 the workgroup's SG thread groups take every SG-th split and are summed in LDS at
// the end (more workgroups in flight when there are many splits).  Every workgroup first rebuilds
// the per-head merge weights of its group: with unnormalised partials O_i the weight of split i
// is 2^(m_i - M) / L, L = sum_i 2^(m_i - M) l_i.

struct CombineArgs {
  const float* part_ml;
  const uint32_t* part_o;
  __bf16* out;
  float* lse;
  int H, n_splits, waves;
};

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

template <int SG>
__global__ __launch_bounds__(256) void sfa_combine(CombineArgs a) {
  constexpr int kMaxSplits = 64;
  __shared__ float wgt[kMaxSplits][32];
  __shared__ float sm[kMaxSplits][32];
  const int tid = threadIdx.x;
  const int row = blockIdx.x, g = blockIdx.y, chunk = blockIdx.z;
  const int S = a.n_splits, NG = a.waves;
  // (m_i, l_i) of every split and head of the group: all loads in one round
  for (int i = tid >> 5; i < S; i += 8) {
    const int head = g * 32 + (tid & 31);
    float m = -INFINITY, l = 0.f;
    if (head < a.H) {
      const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (((size_t)row * S + i) * a.H + head) * 2);
      m = ml.x; l = ml.y;
    }
    sm[i][tid & 31] = m;
    wgt[i][tid & 31] = l;
  }
  __syncthreads();
  if (tid < 32) {
    const int head = g * 32 + tid;
    float M = -INFINITY;
    for (int i = 0; i < S; ++i) M = fmaxf(M, sm[i][tid]);
    float L = 0.f;
    for (int i = 0; i < S; ++i) {
      const float e = M != -INFINITY ? exp2f(sm[i][tid] - M) : 0.f;
      L += e * wgt[i][tid];
      wgt[i][tid] = e;
    }
    const float inv_L = L > 0.f ? 1.f / L : 0.f;
    for (int i = 0; i < S; ++i) wgt[i][tid] *= inv_L;
    if (a.lse != nullptr && head < a.H && chunk == 0)
      a.lse[(size_t)row * a.H + head] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  // this thread's 16-byte unit u of the group's [mb][half][lane][4 pairs] block (8192 pairs):
  // 4 register pairs of one head (accumulator lane), i.e. output columns d0 .. d0 + 3 and
  // d0 + 8 .. d0 + 11
  constexpr int TG = 256 / SG;              // threads per split group
  const int sg = tid / TG, t64 = tid % TG;
  const int u = chunk * TG + t64;
  const int lane = u & 63, half = (u >> 6) & 1, mb = u >> 7;
  const int nl = lane & 31, hh = lane >> 5;
  const size_t per_split = (size_t)NG * kVBlocks * 8 * 64;
  const uint32_t* src = a.part_o + (size_t)row * S * per_split + (size_t)g * kVBlocks * 8 * 64 + 4 * (size_t)u;
  float acc[4][2] = {};
#pragma unroll 4
  for (int sp = sg; sp < S; sp += SG) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + sp * per_split);
    const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
    const float wq = wgt[sp][nl];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[q][0] = fmaf(wq, bf16_lo(vv[q]), acc[q][0]);
      acc[q][1] = fmaf(wq, bf16_hi(vv[q]), acc[q][1]);
    }
  }
  if constexpr (SG > 1) {
    __shared__ float red[SG - 1][TG][8];
    if (sg > 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) { red[sg - 1][t64][2 * q] = acc[q][0]; red[sg - 1][t64][2 * q + 1] = acc[q][1]; }
    }
    __syncthreads();
    if (sg != 0) return;
#pragma unroll
    for (int k = 0; k < SG - 1; ++k)
#pragma unroll
      for (int q = 0; q < 4; ++q) { acc[q][0] += red[k][t64][2 * q]; acc[q][1] += red[k][t64][2 * q + 1]; }
  }
  // register pair k = 4*half + q holds columns 32mb + 8(k >> 1) + 4hh + 2(k & 1) + {0, 1}
  const int head = g * 32 + nl;
  if (head < a.H) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + ((size_t)row * a.H + head) * kDimV + 32 * mb + 16 * half + 4 * hh;
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16(acc[0][0], acc[0][1]), pack_bf16(acc[1][0], acc[1][1]));
    *reinterpret_cast<uint2*>(dst + 8) = make_uint2(pack_bf16(acc[2][0], acc[2][1]), pack_bf16(acc[3][0], acc[3][1]));
  }
}

// ------------------------------------------------------------------------------------------------
static size_t align_up(size_t x, size_t al) { return (x + al - 1) / al * al; }

hipError_t attn_take_input_flags(uint32_t* flags) {
  uint32_t z = 0;
  hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_input_flags), sizeof(uint32_t), 0, hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(g_input_flags), &z, sizeof z, 0, hipMemcpyHostToDevice);
  return e;
}

AttnPlan plan_attn(const dsa_paged_layout& L, const dsa_attn_shape& S) {
  AttnPlan p;
  p.waves = (S.heads + 31) / 32;                       // 32-head groups
  p.groups_per_wg = p.waves >= 4 ? 4 : (p.waves >= 2 ? 2 : 1);
  p.head_chunks = (p.waves + p.groups_per_wg - 1) / p.groups_per_wg;
  const int rows = L.batch * S.T;
  // splits: enough workgroups (rows x head chunks x splits) to cover the GPU's 256 compute units,
  // at most 64 splits, each holding a whole number of 32-row tiles.  A split of fewer than 4 tiles
  // pays more for its partial output (written, then read back by the combine) and its prologue
  // than its extra parallelism returns, so splits keep 4 tiles as long as the grid still has 128
  // workgroups (8 rows at K = 2048: 16 splits of 4 tiles measured faster than 32 of 2).
  const int tiles = (S.top_k + kBK - 1) / kBK;
  const int per_split = std::max(rows * p.head_chunks, 1);
  int splits = (256 + per_split - 1) / per_split;
  const int min_splits = (128 + per_split - 1) / per_split;
  splits = std::max(min_splits, std::min(splits, tiles / 4));
  splits = std::max(1, std::min(splits, std::min(64, tiles)));
  const int tiles_per = (tiles + splits - 1) / splits;
  p.keys_per_split = tiles_per * kBK;
  p.n_splits = (tiles + tiles_per - 1) / tiles_per;
  size_t off = 0;
  if (p.n_splits > 1) {
    p.off_ml = off; off = align_up(off + (size_t)rows * p.n_splits * S.heads * 2 * 4, 256);
    p.off_part = off; off = align_up(off + (size_t)rows * p.n_splits * p.waves * kVBlocks * 8 * 64 * 4, 256);
  }
  p.total = off;
  return p;
}

hipError_t launch_attn(const AttnArgs& a, const AttnPlan& p, hipStream_t st) {
  SfaArgs s;
  s.q = static_cast<const unsigned char*>(a.q);
  s.kv = static_cast<const unsigned char*>(a.kv_cache);
  s.kv_sc = static_cast<const unsigned char*>(a.kv_scale);
  s.idx = a.idx;
  s.block_table = a.block_table;
  s.seq_lens = a.seq_lens;
  s.out = static_cast<__bf16*>(a.out);
  s.lse = a.lse;
  unsigned char* ws = static_cast<unsigned char*>(a.workspace);
  s.part_ml = p.n_splits > 1 ? reinterpret_cast<float*>(ws + p.off_ml) : nullptr;
  s.part_o = p.n_splits > 1 ? reinterpret_cast<uint32_t*>(ws + p.off_part) : nullptr;
  s.T = a.T; s.H = a.heads; s.K = a.top_k; s.max_pages = a.max_pages; s.num_pages = a.num_pages;
  s.n_splits = p.n_splits; s.keys_per_split = p.keys_per_split; s.max_seq_len = a.max_seq_len;
  s.scale_log2 = a.sm_scale * kLog2e;
  const int rows = a.B * a.T;
  const dim3 grid(rows, p.n_splits, p.head_chunks);
  {
    LaunchScope ls("sfa_main", st);
    const bool kv8 = a.kv_scale != nullptr;
    if (p.groups_per_wg == 4) {
      if (kv8) hipLaunchKernelGGL((sfa_main<4, true>), grid, dim3(256), 0, st, s);
      else hipLaunchKernelGGL(sfa_main<4>, grid, dim3(256), 0, st, s);
    } else if (p.groups_per_wg == 2) {
      if (kv8) hipLaunchKernelGGL((sfa_main<2, true>), grid, dim3(128), 0, st, s);
      else hipLaunchKernelGGL(sfa_main<2>, grid, dim3(128), 0, st, s);
    } else {
      if (kv8) hipLaunchKernelGGL((sfa_main<1, true>), grid, dim3(64), 0, st, s);
      else hipLaunchKernelGGL(sfa_main<1>, grid, dim3(64), 0, st, s);
    }
  }
  if (p.n_splits > 1) {
    LaunchScope ls("sfa_combine", st);
    CombineArgs c;
    c.part_ml = s.part_ml; c.part_o = s.part_o; c.out = s.out; c.lse = a.lse;
    c.H = a.heads; c.n_splits = p.n_splits; c.waves = p.waves;
    if (p.n_splits > 16) hipLaunchKernelGGL(sfa_combine<4>, dim3(rows, p.waves, 32), dim3(256), 0, st, c);
    else if (p.n_splits > 8) hipLaunchKernelGGL(sfa_combine<2>, dim3(rows, p.waves, 16), dim3(256), 0, st, c);
    else hipLaunchKernelGGL(sfa_combine<1>, dim3(rows, p.waves, 8), dim3(256), 0, st, c);
  }
  return hipGetLastError();
}

}  // namespace dsa
