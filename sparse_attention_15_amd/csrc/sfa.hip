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
// the accumulation registers; the softmax runs in the log2 domain (exp2 with log2(e) folded into
// the scale) against a fixed per-head reference, so the accumulator is never rescaled.
//
// The bf16 kernel is software-pipelined by one tile: iteration i issues the score product of tile
// i+1 (with the gathers of tile i+3 spread between its MFMAs) and then the value product of tile
// i, with the softmax of tile i+1 spread between those MFMAs.  The matrix pipe thus never waits
// for the exponentials or the gather issue of the same tile.
//
// A row with several splits is merged in the same launch: each split publishes its partial
// (m, l and the unnormalised O in bf16), then sets its ready flags (one per combine part) to the
// call's 64-bit tag; combine workgroups, placed after all split workgroups in the grid, wait until
// every split of their (row, head group) shows the tag, clear those flags again, and merge
//     M = max_i m_i,  L = sum_i 2^(m_i - M) l_i,  out = sum_i 2^(m_i - M) O_i / L,  lse = (M + log2 L) ln 2
// summing the splits in index order, so the output does not depend on which split finished first.
//
// FP8 latent cache ([P1] §4: the SFA cache in FP8 with per-token scales over 128-wide tiles, BF16
// products, the dequantised BF16 tile filling the matrix unit's input buffer directly): rows are
// 576 E4M3 codes plus 8 fp32 scales per token (tiles 0-127, 128-255, 256-383, 384-511, 512-575;
// 3 unused).  The gather ring then holds the raw codes and scales, and each tile is dequantised
// (float32 product, bf16 rounding) straight into the same swizzled bf16 tile the bf16 cache is
// gathered into, so the products run unchanged.
#include <algorithm>
#include <cmath>
#include <mutex>
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
constexpr float kNoRef = -1e30f;           // no reference yet (finite: masked logits stay at p = 0)
constexpr unsigned kMergeSpinCap = 1u << 20;   // a merge wait gives up after ~50 ms (flagged)
constexpr int kPartWords = kVBlocks * 2 * 64 * 4;   // partial O of one 32-head group: 8192 bf16 pairs

struct SfaArgs {
  const unsigned char* q;       // [rows, H, 576] bf16
  const unsigned char* kv;      // [P, 64, 576] bf16, or E4M3 codes for the fp8 cache
  const unsigned char* kv_sc;   // fp8 cache: [P, 64, 8] fp32 tile scales (32 bytes per token)
  const int32_t* idx;           // [rows, K]
  const int32_t* block_table;
  const int32_t* seq_lens;
  __bf16* out;                  // [rows, H, 512]
  float* lse;                   // [rows, H] or null
  float* part_ml;               // [rows, splits, H, 2]: (m, l) of a published partial
  uint32_t* part_o;             // [rows, splits, head groups, 16 blocks, 2 halves, 64 lanes, 4] bf16 pairs
  unsigned long long* sync;     // [rows, head groups, combine parts, splits]: ready flags
  unsigned long long tag;       // this call's tag (never 0)
  int T, H, K, max_pages, num_pages, n_splits, keys_per_split, max_seq_len;
  int rows, head_chunks, comb_parts;   // grid roles (see sfa_role)
  uint32_t kv_bytes;            // bytes of the latent cache when it spans less than 4 GiB, else 0
  float scale_log2;             // sm_scale * log2(e)
};

// LDS layout of a gathered tile (36864 bytes) in two regions:
//   A: the 512 value columns of each row, 1024 bytes (64 chunks of 16 bytes), row r at 1024*r;
//   B: the 64 rope columns, 128 bytes (8 chunks), row r at kRegionB + 128*r.
// Chunk c of row r sits at slot c ^ swa(r) in A and c ^ swb(r) in B.  A region-A row is exactly
// one wave-wide direct-to-LDS load (64 lanes x 16 bytes), so a gather is one scalar-addressed load
// per row.  The XORs keep the reads free of bank conflicts whether the LDS serves 128 or 256 bytes
// per cycle (16-byte slots, 8 or 16 per bank cycle).  The score product's 16-byte reads take one
// chunk of 8 or 16 consecutive rows per cycle: swa permutes a row's low four bits, and its low
// three bits alone permute the low three.  The value product's transposed 8-byte reads take
// chunks 4m + {0, 1} (16 lanes) or 4m + {0..3} (32 lanes) of 4 consecutive rows 4p .. 4p + 3:
// bits 1-2 and bits 2-3 of swa each take four different values over those rows.  With row bits
// r0..r3: swa = r2 | r1 << 1 | r0 << 2 | (r0 ^ r1 ^ r3) << 3.
constexpr int kRegionB = 32768;
__device__ __forceinline__ int swa(int r) {
  const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
  return r2 | (r1 << 1) | (r0 << 2) | ((r0 ^ r1 ^ r3) << 3);
}
__device__ __forceinline__ int swb(int r) { return (r >> 1) & 7; }


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two floats to packed bf16 (round to nearest even) with gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

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
// tiles (n loads each) may stay in flight.  The counter saturates at 63: a larger count is
// clamped, which only waits longer.
template <int n>
__device__ __forceinline__ void wait_ring(int later) {
  if (later >= 2) wait_vmcnt<(2 * n > 63 ? 63 : 2 * n)>();
  else if (later == 1) wait_vmcnt<(n > 63 ? 63 : n)>();
  else wait_vmcnt<0>();
}

// Register-class pins (empty asm, no instruction of its own): the output accumulator O^T takes
// 256 registers, the whole accumulation file.  Every MFMA result is selected into that file, so
// the score accumulator S (16 registers) only fits if it leaves right after its product and one
// O^T block waits in the VGPR file during it.  Pinning those points keeps the compiler from
// shuffling several blocks per tile; in the merge, each updated block is pinned back.
__device__ __forceinline__ void pin_v(f32x16& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin_a(f32x16& x) { asm volatile("" : "+a"(x)); }

// Partial O of one 32-head group as a buffer resource (its 32 KiB are the bound: the hardware
// drops any access outside).  Its loads and stores carry the agent-scope coherence bit (sc1), as
// agent-scope atomics do, so they bypass the per-XCD L2s; unlike atomics they are ordinary
// 16-byte accesses that the compiler batches.
constexpr int kCoherent = 16;                       // cache policy: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(uint32_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, kPartWords * 4, 0x00020000);
}

// Ready flags of a split row: flag[row][head group][part][split] holds the call's tag once that
// split's partial of that head group is published.  Every combine part has its own copy of the
// flags, so no word is shared by two writers or two readers; a part resets its copies once it has
// read them, so a replay of the same launch (same tag) starts from clean flags.

// ------------------------------------------------------------------------------------------------
// End of a split.  One split: write out = O / l (bf16) and lse.  Several: publish this split's
// partial (m, l and the unnormalised O in bf16, in the accumulator's own lane order) and count it
// in the (row, head group) word; the combine workgroups (sfa_combine_part) merge the row.
template <int NW>
__device__ __forceinline__ void finish_split(const SfaArgs& a, f32x16 (&o)[kVBlocks], float m_run, float l_run,
                                             int row, int split, int gg, int tid) {
  const int lane = tid & 63, nl = lane & 31, hh = lane >> 5;
  const int NGT = (a.H + 31) / 32;
  const int head = gg * 32 + nl;
  const bool hvalid = head < a.H;
  if (a.n_splits > 1) {
    if (gg >= NGT) return;
    const size_t ps = (size_t)row * a.n_splits + split;
    if (hvalid && hh == 0)
      __hip_atomic_store(reinterpret_cast<uint64_t*>(a.part_ml + (ps * a.H + head) * 2),
                         (uint64_t)__float_as_uint(m_run) | ((uint64_t)__float_as_uint(l_run) << 32),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // this lane's 16 bytes of every 1 KiB unit (block, half); the unit's offset goes in the
    // instructions' scalar offset, so one VGPR serves all 32 units
    int lane16 = 16 * lane;
    asm volatile("" : "+v"(lane16));
    const __amdgpu_buffer_rsrc_t po = part_rsrc(a.part_o + (ps * NGT + gg) * kPartWords);
#pragma unroll
    for (int mb = 0; mb < kVBlocks; ++mb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = pack_bf16(o[mb][8 * half + 2 * q], o[mb][8 * half + 2 * q + 1]);
        __builtin_amdgcn_raw_buffer_store_b128(v, po, lane16, 1024 * (mb * 2 + half), kCoherent);
      }
    // the stores are complete (device-coherent) before the flags that publish them
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (lane < a.comb_parts)
      __hip_atomic_store(a.sync + (((size_t)row * NGT + gg) * a.comb_parts + lane) * a.n_splits + split, a.tag,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
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
}

// Combine workgroup: merges part `part` (of comb_parts) of head group g of a split row once all S
// splits have published.  With unnormalised partials O_i the weight of split i is
// 2^(m_i - M) / L, M = max_i m_i, L = sum_i 2^(m_i - M) l_i, and lse = (M + log2 L) ln 2.  The
// splits are summed in index order, so the result does not depend on which split finished first.
// These workgroups come after every split workgroup in the grid; the hardware dispatches
// workgroups in index order, so the splits a combine part waits for are already running (the wait
// is bounded all the same: past it the merge goes ahead and the debug flag records it).
//
// Each thread owns NU 16-byte units (4 bf16 pairs of one head) of the group's [block][half][lane]
// layout and keeps 32 loads in flight: NU units x 32/NU splits per batch.
template <int NT, int NU>
__device__ __forceinline__ void combine_units(const SfaArgs& a, int row, int g, int part, const float* wgt) {
  constexpr int SB = 32 / NU;                               // splits per batch
  const int S = a.n_splits, NGT = (a.H + 31) / 32;
  const int tid = threadIdx.x;
  const int u0 = part * NT * NU + tid;                      // units u0, u0 + NT, ...
  float acc[NU][8];
#pragma unroll
  for (int j = 0; j < NU; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  for (int s0 = 0; s0 < S; s0 += SB) {
    u32x4 v[NU][SB];
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      if (s0 + k < S) {
        const __amdgpu_buffer_rsrc_t rs = part_rsrc(a.part_o + (((size_t)row * S + s0 + k) * NGT + g) * kPartWords);
#pragma unroll
        for (int j = 0; j < NU; ++j) v[j][k] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (u0 + j * NT), 0, kCoherent);
      }
    }
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      if (s0 + k < S) {
#pragma unroll
        for (int j = 0; j < NU; ++j) {
          const int nl = (u0 + j * NT) & 31;
          const float wk = wgt[2 * ((s0 + k) * 32 + nl)];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[j][2 * q] = fmaf(wk, bf16_lo(v[j][k][q]), acc[j][2 * q]);
            acc[j][2 * q + 1] = fmaf(wk, bf16_hi(v[j][k][q]), acc[j][2 * q + 1]);
          }
        }
      }
    }
  }
  // register pair k = 4*half + q holds columns 32mb + 8(k >> 1) + 4hh + 2(k & 1) + {0, 1}
#pragma unroll
  for (int j = 0; j < NU; ++j) {
    const int u = u0 + j * NT;
    const int ln = u & 63, half = (u >> 6) & 1, mb = u >> 7;
    const int nl = ln & 31, hh = ln >> 5;
    const int head = g * 32 + nl;
    if (head < a.H) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + ((size_t)row * a.H + head) * kDimV + 32 * mb + 16 * half + 4 * hh;
      *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16(acc[j][0], acc[j][1]), pack_bf16(acc[j][2], acc[j][3]));
      *reinterpret_cast<uint2*>(dst + 8) = make_uint2(pack_bf16(acc[j][4], acc[j][5]), pack_bf16(acc[j][6], acc[j][7]));
    }
  }
}

template <int NW>
__device__ __forceinline__ void sfa_combine_part(const SfaArgs& a, int row, int g, int part, float* wgt) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int S = a.n_splits, NGT = (a.H + 31) / 32;
  unsigned long long* flags = a.sync + (((size_t)row * NGT + g) * a.comb_parts + part) * S;
  // The splits are lower-numbered workgroups of this launch, so with workgroups dispatched in index
  // order the wait always ends; past its cap it gives up, the outputs this part writes become NaN
  // and the debug flag is set.
  __shared__ int timed_out;
  if (tid < 64) {
    // lane i watches the flags of splits i, i + 64, ...; polls back off (up to ~4000 cycles apart)
    unsigned spins = 0, nap = 1;
    int late = 0;
    for (;;) {
      bool ready = true;
      for (int sp = lane; sp < S; sp += 64)
        ready &= __hip_atomic_load(&flags[sp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.tag;
      if (__builtin_amdgcn_readfirstlane(__ballot(!ready) == 0ull ? 1 : 0)) break;
      if (++spins > kMergeSpinCap / 16) { if (lane == 0) flag_input(kFlagSync); late = 1; break; }
      for (unsigned k = 0; k < nap; ++k) __builtin_amdgcn_s_sleep(4);
      nap = nap < 16 ? 2 * nap : 16;
    }
    // only this part reads these flags: reset them for the next call
    for (int sp = lane; sp < S; sp += 64)
      __hip_atomic_store(&flags[sp], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) timed_out = late;
  }
  lds_barrier();
  DSA_STAMP(5);
  // merge weights of every split and head of the group (wgt[S][32]), the row's lse from part 0
  for (int i = tid; i < S * 32; i += NT) {
    const int sp = i >> 5, h = g * 32 + (i & 31);
    const uint64_t ml = h < a.H ? __hip_atomic_load(reinterpret_cast<const uint64_t*>(
                                      a.part_ml + (((size_t)row * S + sp) * a.H + h) * 2), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : 0ull;
    wgt[2 * i] = h < a.H ? __uint_as_float((uint32_t)ml) : -INFINITY;
    wgt[2 * i + 1] = __uint_as_float((uint32_t)(ml >> 32));
  }
  lds_barrier();
  if (tid < 32) {
    float M = -INFINITY;
    for (int sp = 0; sp < S; ++sp) M = fmaxf(M, wgt[2 * (sp * 32 + tid)]);
    float L = 0.f;
    for (int sp = 0; sp < S; ++sp) {
      const float e = M != -INFINITY ? __builtin_amdgcn_exp2f(wgt[2 * (sp * 32 + tid)] - M) : 0.f;
      L += e * wgt[2 * (sp * 32 + tid) + 1];
      wgt[2 * (sp * 32 + tid)] = e;
    }
    const float inv = timed_out ? __builtin_nanf("") : (L > 0.f ? 1.f / L : 0.f);
    for (int sp = 0; sp < S; ++sp) wgt[2 * (sp * 32 + tid)] *= inv;
    const int h = g * 32 + tid;
    if (a.lse != nullptr && part == 0 && h < a.H)
      a.lse[(size_t)row * a.H + h] = timed_out ? __builtin_nanf("") : (L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY);
  }
  lds_barrier();
  // units per thread: the group's 2048 units over comb_parts parts of NT threads
  const int nu = (kPartWords / 4) / (a.comb_parts * NT);
  if (nu >= 8) combine_units<NT, 8>(a, row, g, part, wgt);
  else if (nu == 4) combine_units<NT, 4>(a, row, g, part, wgt);
  else if (nu == 2) combine_units<NT, 2>(a, row, g, part, wgt);
  else combine_units<NT, 1>(a, row, g, part, wgt);
}

// Workgroup roles of the 1-D grid: the first rows * splits * head chunks workgroups run the
// splits (row fastest, so the splits of a row share an XCD when the row count is a multiple of
// 8); the rest are combine parts, (row, head group, part), row fastest.
struct SfaRole {
  bool combine;
  int row, split, chunk, g, part;
};
__device__ __forceinline__ SfaRole sfa_role(const SfaArgs& a) {
  SfaRole r;
  const int rows = a.rows;
  const int n_main = rows * a.n_splits * a.head_chunks;
  int b = blockIdx.x;
  r.combine = b >= n_main;
  if (!r.combine) {
    r.row = b % rows; b /= rows;
    r.split = b % a.n_splits; r.chunk = b / a.n_splits;
    r.g = r.part = 0;
  } else {
    b -= n_main;
    const int NGT = (a.H + 31) / 32;
    r.row = b % rows; b /= rows;
    r.g = b % NGT; r.part = b / NGT;
    r.split = r.chunk = 0;
  }
  return r;
}

// Direct-to-LDS load of 16 bytes per lane through a buffer resource: lane i's 16 bytes from
// byte offset soff + voff (soff wave-uniform, voff per lane) land at LDS address lds_dst + 16 i.
// Inline assembly for the reason given at lds_dma16; the resource's size bounds every access.
// NT: the nontemporal cache policy, for rows no other workgroup of the launch reads.
template <bool NT = false>
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t rsrc, uint32_t soff, uint32_t voff,
                                              const void* lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_dst));
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds" ::"s"(base), "v"(voff),
                 "s"(rsrc), "s"(soff)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(base), "v"(voff),
                 "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// ------------------------------------------------------------------------------------------------
// Softmax pieces shared by both kernels (same arithmetic, so an FP8-cache call over a cache that
// holds exact bf16 values gives the bf16 call's bits).  Register r of a lane holds key
// 8(r/4) + 4hh + r%4 of the tile.
// Keys that are not selected get logit -inf (a wave-uniform test skips this for full tiles).
__device__ __forceinline__ void mask_keys(f32x16& s, uint32_t valid, int hh) {
  if (valid == 0xFFFFFFFFu) return;
  const uint32_t vmask = valid >> (4 * hh);
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = ((vmask >> (8 * (r >> 2) + (r & 3))) & 1u) ? s[r] : -INFINITY;
}
// Max of the raw logits r0..r1-1 (positive scaling commutes with max, rounding included).
__device__ __forceinline__ float raw_max(const f32x16& s, int r0, int r1, float m) {
#pragma unroll
  for (int r = r0; r < r1; ++r) m = fmaxf(m, s[r]);
  return m;
}
// 2^(z - m) with z = scale * s rounded once (fma): masked keys (-inf) give 0.
__device__ __forceinline__ float prob(float s, float scale, float m) {
  return __builtin_amdgcn_exp2f(fmaf(s, scale, -m));
}

// ------------------------------------------------------------------------------------------------
// bf16 latent cache, software-pipelined (see the file comment).  BUF: the cache spans less than
// 4 GiB, so the row table holds each selected row's 32-bit byte offset and the gathers address it
// through a buffer resource (a scalar offset per value row, no 64-bit address arithmetic).
template <int NW, bool BUF, bool NTG = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sfa_pipe(SfaArgs a) {
  constexpr int NT = NW * 64;               // one wave per 32-head group
  constexpr int kRows = kBK / NW, kRope = 4 / NW;
  constexpr int kDmaWave = kRows + kRope;   // wave-wide loads per tile: value rows, then rope blocks
  constexpr int kPerSlot = kDmaWave / 9;    // loads issued after every fourth score MFMA (9 places)
  static_assert(kDmaPerTile % NW == 0 && kDmaWave % 9 == 0, "per-wave load count must be uniform");
  __shared__ __attribute__((aligned(1024))) unsigned char lds_kv[kStages][kTileBytes];
  __shared__ int lds_rows[kMaxSplitKeys];   // physical row of each selected index, -1 = skip
  __shared__ uint32_t lds_valid[kMaxSplitKeys / kBK];   // per tile: its selected keys as a bit mask
  __shared__ int lds_first, lds_last;       // first and last j with a visible position
  __shared__ int lds_epoch;                 // restarts requested by any wave (see below)

  const SfaRole role = sfa_role(a);
  if (role.combine) {
    DSA_STAMP(4);
    sfa_combine_part<NW>(a, role.row, role.g, role.part, reinterpret_cast<float*>(&lds_kv[0][0]));
    DSA_STAMP(6);
    return;
  }
  DSA_STAMP(0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: LDS DMA bases stay in SGPRs
  const int nl = lane & 31, hh = lane >> 5;
  const int row = role.row, split = role.split;
  const int gg = role.chunk * NW + wave;    // this wave's global head group
  const int b = row / a.T, t = row % a.T;
  const int n = row_visible(a.seq_lens, b, a.T, t, a.max_seq_len);
  const int k_begin = split * a.keys_per_split;
  const int nkeys = max(0, min(a.K, k_begin + a.keys_per_split) - k_begin);
  const int ntiles = (nkeys + kBK - 1) / kBK;
  const int head = gg * 32 + nl;
  const bool hvalid = head < a.H;
  const int32_t* idx = a.idx + (size_t)row * a.K + k_begin;
  const int32_t* bt = a.block_table + (size_t)b * a.max_pages;

  if (tid == 0) { lds_first = kMaxSplitKeys; lds_last = -1; lds_epoch = 0; }
  // Prologue, split between the waves: the counter that orders a wave's loads is per wave, so wave
  // 0 resolves the first index batch (index loads, then their block-table loads) without waiting
  // for the q copy, which the other waves issue meanwhile (with one wave, it does both).
  //
  // q copy: the B operand of the score product is this lane's head row of q, columns 16 ks + 8 hh
  // .. + 7 for K step ks.  The workgroup's q rows (NW x 32 heads x 1152 bytes: one ring slot per
  // head group, free until the first gathers) go to LDS with direct-to-LDS loads of eight whole
  // 128-byte lines each; read straight into the MFMA layout, every load instruction would touch 32
  // rows, a quarter of a line each.  16-byte chunk c of head h sits at slot 72h + (c ^ ((h >> 1) &
  // 7)): the XOR stays inside a 128-byte line and keeps the fragment reads (16 lanes = 16 heads,
  // one chunk) free of bank conflicts.  Heads beyond H copy head 0; their results are never stored.
  constexpr int kCopyWaves = NW > 1 ? NW - 1 : 1;
  constexpr int kCopyLoads = (NW * kQSteps + kCopyWaves - 1) / kCopyWaves;   // per copying wave
  if (NW == 1 || wave > 0) {
    const unsigned char* qrow = a.q + (size_t)row * a.H * kRowBytes;
    const int head0 = role.chunk * NW * 32;
    const int w0 = NW > 1 ? wave - 1 : 0;
#pragma unroll 4
    for (int u = 0; u < kCopyLoads; ++u) {
      const int i = w0 * kCopyLoads + u;                 // fills image bytes 1024 i .. of the workgroup
      if (i < NW * kQSteps) {
        const int sl = 64 * i + lane;
        const int hl = sl / 72, cp = sl % 72;
        const int hq = head0 + hl < a.H ? head0 + hl : 0;
        lds_dma16(qrow + (size_t)hq * kRowBytes + 16 * (cp ^ ((hl >> 1) & 7)), &lds_kv[0][0] + 1024 * i);
      }
    }
  }
  // Row table: lds_rows[j] = physical row of selected index j, -1 if it is not a visible position;
  // lds_valid[tile] = its mask.  Eight index loads per lane go out together, then their block-table
  // loads: wave 0 takes the first 512 keys, all waves the rest (after the copy).
  constexpr int kBatch = 8;
  // first and last selected j of this wave, from the batches' ballots (scalar ops: a per-lane LDS
  // atomic would become a loop over the active lanes)
  int w_first = kMaxSplitKeys, w_last = -1;
  auto table = [&](int j0, int stride, int lid) __attribute__((always_inline)) {
    int s[kBatch], pg[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + u * stride + lid;
      s[u] = j < nkeys ? idx[j] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) pg[u] = s[u] >= 0 && s[u] < n ? bt[s[u] / kPage] : 0;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + u * stride + lid;
      if (s[u] < -1 || s[u] >= n) flag_input(kFlagIndex);
      const int r = s[u] >= 0 && s[u] < n ? clamp_page(pg[u], a.num_pages) * kPage + (s[u] % kPage) : -1;
      const uint64_t bal = __ballot(r >= 0);
      if (j < ntiles * kBK) {
        lds_rows[j] = BUF && r >= 0 ? (int)((uint32_t)r * kRowBytes) : r;   // BUF: byte offset
        if ((lane & 31) == 0) lds_valid[j >> 5] = (uint32_t)(bal >> (lane & 32));
      }
      if (bal != 0) {                       // lanes hold consecutive j from jw on
        const int jw = j0 + u * stride + (lid - lane);
        w_first = min(w_first, jw + (int)__builtin_ctzll(bal));
        w_last = max(w_last, jw + 63 - (int)__builtin_clzll(bal));
      }
    }
  };
  constexpr int kFirstKeys = kBatch * 64;
  lds_barrier();                            // the bounds are initialised
  if (wave == 0) table(0, 64, lane);
  if (ntiles * kBK > kFirstKeys) {          // long splits: the rest with every wave
    __builtin_amdgcn_s_waitcnt(0x0F70);
    lds_barrier();
    for (int j0 = kFirstKeys; j0 < ntiles * kBK; j0 += kBatch * NT) table(j0, NT, tid);
  }
  if (lane == 0 && w_last >= 0) { atomicMin(&lds_first, w_first); atomicMax(&lds_last, w_last); }
  // the q copy and the table's loads have landed (a compiler-visible vmcnt(0): no wait for them is
  // left for the main loop, whose gathers the compiler does not count) ... for every wave
  __builtin_amdgcn_s_waitcnt(0x0F70);
  lds_barrier();
  bf16x8 qf[kQSteps];
  {
    const unsigned char* qh = lds_kv[wave] + nl * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < kQSteps; ++ks)
      qf[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(qh + 16 * ((2 * ks + hh) ^ ((nl >> 1) & 7))));
  }
  lds_barrier();                            // every wave holds its q: the ring is free
  DSA_STAMP(1);
  // Tiles run from the first through the last tile holding a selected key (a causal row with
  // fewer visible positions than K leaves its trailing tiles empty).  Keys that are not selected
  // are gathered from the first selected row (finite data: their zero probabilities never meet a
  // NaN).
  const int first = lds_first, last = lds_last;
  const int ft = first / kBK;
  const int nt = last >= 0 ? last / kBK - ft + 1 : 0;
  const int fill_row = last >= 0 ? lds_rows[first] : 0;   // BUF: its byte offset

  // Gathers.  This wave loads the value columns of rows wave, wave + NW, ... (one load per row:
  // the row id is wave-uniform, so the row's address is a scalar base and each lane adds its own
  // swizzled 16-byte chunk) and the rope blocks wave, wave + NW, ... < 4 (8 rows x 8 chunks per
  // load, lane i: row 8k + i/8, slot i%8).  Every wave issues the same number of loads per tile,
  // which the counter waits rely on.  Load L < kRows is value row u = L; the rest are rope blocks.
  // row_id(i, L): the physical row (value load: wave-uniform; rope load: this lane's) of load L.
  auto row_id = [&](int i, int L) __attribute__((always_inline)) {
    const int* tr = &lds_rows[(ft + i) * kBK];
    return L < kRows ? tr[wave + L * NW] : tr[8 * (wave + (L - kRows) * NW) + (lane >> 3)];
  };
  // BUF: the cache as a buffer (its size, at most 2^32 - 1 bytes, bounds the gathers)
  const __amdgpu_buffer_rsrc_t kv_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<unsigned char*>(a.kv), 0, BUF ? (int)a.kv_bytes : 0, 0x00020000);
  auto gather_one = [&](int L, unsigned char* slot, int id) __attribute__((always_inline)) {
    if (L < kRows) {
      const int r = wave + L * NW;
      int pr = __builtin_amdgcn_readfirstlane(id);
      pr = pr == -1 ? fill_row : pr;        // -1: not selected (a BUF offset may exceed 2^31)
      if constexpr (BUF)
        lds_dma16_buf<NTG>(kv_rsrc, (uint32_t)pr, (uint32_t)(16 * lane) ^ (uint32_t)(16 * swa(r)), slot + 1024 * r);
      else
        lds_dma16_rows(a.kv + (size_t)(uint32_t)pr * kRowBytes, (uint32_t)(16 * lane) ^ (uint32_t)(16 * swa(r)),
                       slot + 1024 * r);
    } else {
      const int k = wave + (L - kRows) * NW;
      const int r = 8 * k + (lane >> 3);
      const int pr = id == -1 ? fill_row : id;
      if constexpr (BUF)
        lds_dma16_buf<NTG>(kv_rsrc, 0u, (uint32_t)pr + 2 * kDimV + 16 * ((lane & 7) ^ swb(r)), slot + kRegionB + 1024 * k);
      else
        lds_dma16(a.kv + (size_t)(uint32_t)pr * kRowBytes + 2 * kDimV + 16 * ((lane & 7) ^ swb(r)),
                  slot + kRegionB + 1024 * k);
    }
  };
  auto issue_tile = [&](int i, unsigned char* slot) __attribute__((always_inline)) {
    int ids[kDmaWave];
#pragma unroll
    for (int L = 0; L < kDmaWave; ++L) ids[L] = row_id(i, L);
#pragma unroll
    for (int L = 0; L < kDmaWave; ++L) gather_one(L, slot, ids[L]);
  };

  // O^T: 512 latent columns (16 blocks of 32) x 32 heads
  f32x16 o[kVBlocks];
#pragma unroll
  for (int mb = 0; mb < kVBlocks; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  // Fixed softmax reference per head (log2 units), set from the split's first tile (which holds a
  // selected key): its max plus kRefMargin.  Probabilities 2^(s - m_ref) stay below 2^kRefLimit
  // as long as no logit exceeds m_ref + kRefLimit, so the accumulator never needs rescaling.  A
  // logit beyond that (a spread of more than 164 log2 units inside the split) raises the reference
  // and restarts the split from its first tile.
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

  // S^T = X q^T for the tile in ring slot `buf`: rows = the tile's 32 keys, columns = this wave's
  // 32 heads.  The A fragments stream through a 4-deep register ring (the read for step ks + 4
  // goes out right behind the MFMA of step ks).  With GATHER, the loads of tile gi into slot
  // `gbuf` go out after every fourth MFMA, kPerSlot at a time; the row ids of each group are read
  // one group (four MFMAs) ahead.  Slots are runtime bases: every per-lane offset below only
  // touches address bits 4-11 and a slot starts at a multiple of 36864 = 0x9000, so slot base and
  // offset add without carries into the XORed bits.
  auto score = [&](int buf, int gi, int gbuf, auto gather_c) __attribute__((always_inline)) {
    constexpr bool GATHER = decltype(gather_c)::value;
    int ids[kPerSlot];
    if constexpr (GATHER) {
#pragma unroll
      for (int e = 0; e < kPerSlot; ++e) ids[e] = row_id(gi, e);
    }
    const unsigned char* tile = lds_kv[0];
    int qa_t = qa + buf * kTileBytes, qb_t = qb + buf * kTileBytes;
    asm volatile("" : "+v"(qa_t), "+v"(qb_t));
    auto a_frag = [&](int ks) {
      const int off = ks < 32 ? (qa_t ^ (32 * (ks & 7))) + 256 * (ks >> 3) : qb_t ^ (32 * (ks - 32));
      return *reinterpret_cast<const u32x4*>(tile + off);
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
      if constexpr (GATHER) {
        if ((ks & 3) == 1) {
          const int g = ks >> 2;
#pragma unroll
          for (int e = 0; e < kPerSlot; ++e) gather_one(g * kPerSlot + e, lds_kv[gbuf], ids[e]);
          if (g + 1 < 9) {
#pragma unroll
            for (int e = 0; e < kPerSlot; ++e) ids[e] = row_id(gi, (g + 1) * kPerSlot + e);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return s;
  };

  // P^T as the B operand of the value product: K step k2 covers keys 16*k2 .. 16*k2 + 15; this
  // lane's 8 values are keys 16*k2 + {0..3, 8..11} + 4*hh (accumulator rows of the score tile)
  auto pack_p = [&](const f32x16& p, int k2) {
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = pack_bf16(p[8 * k2 + 2 * e], p[8 * k2 + 2 * e + 1]);
    return as_bf16x8(v);
  };
  // The whole softmax of one tile at once (the split's first tile: it sets the reference).
  // Logits are in log2 units (the scale carries log2 e).
  auto softmax_now = [&](f32x16& s, uint32_t valid, bf16x8 (&pn)[2]) {
    mask_keys(s, valid, hh);
    const float mx = xor32_max(raw_max(s, 0, 16, -INFINITY) * a.scale_log2);
    if (m_run == kNoRef) m_run = mx + kRefMargin;   // the first tile holds a selected key: mx > -inf
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s[r] = prob(s[r], a.scale_log2, m_run); psum += s[r]; }
    l_run += xor32_sum(psum);
    if (mx > m_run + kRefLimit) { m_run = mx + kRefMargin; lds_epoch = epoch + 1; }
    pn[0] = pack_p(s, 0);
    pn[1] = pack_p(s, 1);
  };

  // O^T += V^T P^T for the tile in slot `buf` with probabilities pc.  The A operand (latent column
  // m, the same 8 keys) comes from two transposed reads of the row-major tile: a 16-lane group
  // reading 8 bytes (4 columns) of 4 consecutive keys hands lane i the 4 keys of column i.  Same
  // 4-deep ring as the score product; consecutive MFMAs go to different accumulators, block 15
  // first in each K step (it moves to the VGPR file for the next score product, which then does
  // not wait for its last MFMA).  With SOFT, the next tile's logits s leave the accumulation
  // registers after the first MFMA and its softmax (mask `valid`) runs between the following
  // MFMAs, one slice after each, leaving its probabilities in pn.
  auto value = [&](int buf, const bf16x8 (&pc)[2], f32x16& s, uint32_t valid, bf16x8 (&pn)[2], auto soft_c)
      __attribute__((always_inline)) {
    constexpr bool SOFT = decltype(soft_c)::value;
    const unsigned char* tile = lds_kv[0];
    int pv0 = pv[0] + buf * kTileBytes, pv1 = pv[1] + buf * kTileBytes;
    asm volatile("" : "+v"(pv0), "+v"(pv1));
    auto block_of = [](int j) { return ((j & 15) + 15) & 15; };   // MFMA j's O^T block: 15, 0, 1, ..., 14
    auto v_frag = [&](int j, int q) {
      const int mb = block_of(j), k2 = j >> 4;
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(
          tile + ((q ? pv1 : pv0) ^ (64 * (mb & 3))) + 256 * (mb >> 2) + 16384 * k2));
    };
    s16x4 vring[kRingV][2];
#pragma unroll
    for (int j = 0; j < kRingV; ++j) { vring[j][0] = v_frag(j, 0); vring[j][1] = v_frag(j, 1); }
    float mraw = -INFINITY, psum = 0.f, mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2 * kVBlocks; ++j) {
      const int k2 = j >> 4, mb = block_of(j);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vring[j % kRingV][0], vring[j % kRingV][1], 0, 1, 2, 3, 4, 5, 6, 7));
      if (j + kRingV < 2 * kVBlocks) {
        vring[j % kRingV][0] = v_frag(j + kRingV, 0);
        vring[j % kRingV][1] = v_frag(j + kRingV, 1);
      }
      o[mb] = mfma_bf16(vf, pc[k2], o[mb]);
      if constexpr (SOFT) {
        if (j == 0) {
          pin_v(s);                         // S leaves the accumulation registers
          mask_keys(s, valid, hh);
        } else if (j == 1) {
          mraw = raw_max(s, 0, 8, mraw);
        } else if (j == 2) {
          mraw = raw_max(s, 8, 16, mraw);
        } else if (j < 11) {
          const int r = 2 * (j - 3);
          s[r] = prob(s[r], a.scale_log2, m_run);
          s[r + 1] = prob(s[r + 1], a.scale_log2, m_run);
        } else if (j == 11) {
          pn[0] = pack_p(s, 0);
        } else if (j == 12) {
          pn[1] = pack_p(s, 1);
        } else if (j == 13) {
#pragma unroll
          for (int r = 0; r < 16; ++r) psum += s[r];
        } else if (j == 14) {
          psum = xor32_sum(psum);
          mx = xor32_max(mraw * a.scale_log2);
        } else if (j == 15) {
          l_run += psum;
          if (mx > m_run + kRefLimit) {     // too far above the reference: restart with a new one
            m_run = mx + kRefMargin;
            lds_epoch = epoch + 1;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Iteration `it` of the pipelined loop; the ring slot of tile i is i % 4.  MODE 0: score tile
  // it+1 while gathering tile it+3, then the value product of tile it with the softmax of tile
  // it+1; MODE 1: the same without a gather (it+3 is past the end); MODE 2: the value product of
  // the last tile only.  Before the score product, tile it+1 must have landed (tile it+2 may stay
  // in flight); the barrier also tells every wave that the previous iteration's value product is
  // done, so slot (it+3) % 4, which held tile it-1, takes tile it+3.
  bf16x8 pc[2];
  auto iter = [&](int it, auto mode_c) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_c)::value;
    f32x16 s;
    uint32_t valid = 0;
    bf16x8 pn[2];
    if constexpr (MODE < 2) {
      wait_ring<kDmaWave>(MODE == 0 ? 1 : min(1, nt - 2 - it));
      lds_barrier();
      valid = lds_valid[ft + it + 1];
      pin_v(o[kVBlocks - 1]);
      s = score((it + 1) & 3, it + 3, (it + 3) & 3, std::integral_constant<bool, MODE == 0>{});
      value(it & 3, pc, s, valid, pn, std::true_type{});
      pc[0] = pn[0];
      pc[1] = pn[1];
    } else {
      value(it & 3, pc, s, valid, pn, std::false_type{});
    }
  };

  for (;;) {
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i)
      if (i < nt) issue_tile(i, lds_kv[i]);
    if (nt > 0) {
      wait_ring<kDmaWave>(min(2, nt - 1));   // tile 0 landed; tiles 1 and 2 may be in flight
      lds_barrier();
      f32x16 s = score(0, 0, 0, std::false_type{});
      softmax_now(s, lds_valid[ft], pc);
    }
    static_assert(kStages == 4, "slot (i % 4) and the two tiles of lead assume a 4-slot ring");
    int it = 0;
    for (; it < nt - 3; ++it) iter(it, std::integral_constant<int, 0>{});
    for (; it < nt - 1; ++it) iter(it, std::integral_constant<int, 1>{});
    if (it < nt) iter(it, std::integral_constant<int, 2>{});
    // every wave sees the same restart request after the barrier; the gathers of this pass have
    // all been waited for (the last wait of the loop is for the last tile with no later one)
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
  }
  DSA_STAMP(2);
  finish_split<NW>(a, o, m_run, l_run, row, split, gg, tid);
  DSA_STAMP(3);
}

// ------------------------------------------------------------------------------------------------
// FP8 latent cache: the same products over tiles dequantised from E4M3 codes and tile scales.
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void sfa_main_kv8(SfaArgs a) {
  constexpr int NT = NW * 64;               // one wave per 32-head group
  constexpr int kDmaWave = kDmaPerTile8 / NW;
  static_assert(kDmaPerTile8 % NW == 0, "per-wave load count must be uniform");
  static_assert(kStages - 2 <= 2, "wait_ring handles up to two later tiles");
  __shared__ __attribute__((aligned(1024))) unsigned char lds_kv[kStages][kTileBytes];
  __shared__ int lds_rows[kMaxSplitKeys];   // physical row of each selected index, -1 = skip

  const SfaRole role = sfa_role(a);
  if (role.combine) {
    sfa_combine_part<NW>(a, role.row, role.g, role.part, reinterpret_cast<float*>(&lds_kv[0][0]));
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: LDS DMA bases stay in SGPRs
  const int nl = lane & 31, hh = lane >> 5;
  const int row = role.row, split = role.split;
  const int gg = role.chunk * NW + wave;    // this wave's global head group
  const int b = row / a.T, t = row % a.T;
  const int n = row_visible(a.seq_lens, b, a.T, t, a.max_seq_len);
  const int k_begin = split * a.keys_per_split;
  const int nkeys = max(0, min(a.K, k_begin + a.keys_per_split) - k_begin);
  const int ntiles = (nkeys + kBK - 1) / kBK;

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
  // are first copied into LDS with direct-to-LDS loads that each read eight whole 128-byte lines.
  // 16-byte chunk c of head h sits at slot 72h + (c ^ ((h >> 1) & 7)): the XOR stays inside a
  // 128-byte line and makes the fragment reads (16 lanes = 16 heads, one chunk) free of bank
  // conflicts.  Heads beyond H copy head 0; their results are never stored.
  bf16x8 qf[kQSteps];
  unsigned char* const q_img = &lds_kv[0][0];
  {
    const unsigned char* qrow = a.q + (size_t)row * a.H * kRowBytes;
    const int head0 = role.chunk * NW * 32;
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
  int w_fill = kMaxSplitKeys;               // first selected j of this wave (from the ballots)
  for (int j = tid; j < ntiles * kBK; j += NT) {   // NT is a multiple of 64: whole waves
    const int s = j == tid ? s_first : (j < nkeys ? idx[j] : -1);
    if (s < -1 || s >= n) flag_input(kFlagIndex);
    const int r = s >= 0 && s < n ? clamp_page(bt[s / kPage], a.num_pages) * kPage + (s % kPage) : -1;
    lds_rows[j] = r;
    const uint64_t bal = __ballot(r >= 0);
    if ((lane & 31) == 0) lds_valid[j >> 5] = (uint32_t)(bal >> (lane & 32));
    if (bal != 0) w_fill = min(w_fill, j - lane + (int)__builtin_ctzll(bal));
  }
  if (lane == 0 && w_fill < kMaxSplitKeys) atomicMin(&lds_fill, w_fill);
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

  // O^T: 512 latent columns (16 blocks of 32) x 32 heads
  f32x16 o[kVBlocks];
#pragma unroll
  for (int mb = 0; mb < kVBlocks; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  // Fixed softmax reference per head (log2 units), set from the first tile with a valid key:
  // its max plus kRefMargin (see sfa_pipe).
  float m_run = kNoRef, l_run = 0.f;
  int epoch = 0;                            // restarts seen by this wave

  const int sa_nl = swa(nl), sb_nl = swb(nl);
  const int qa = 1024 * nl + 16 * ((hh ^ sa_nl) & 1) + 32 * (sa_nl >> 1);
  const int qb = kRegionB + 128 * nl + 16 * ((hh ^ sb_nl) & 1) + 32 * (sb_nl >> 1);
  const int kq = 4 * hh + ((lane & 15) >> 2);
  const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  int pv[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int sa = swa(8 * q + kq);
    pv[q] = 1024 * (8 * q + kq) + 16 * (cl ^ (sa & 3)) + 64 * (sa >> 2) + 8 * (lane & 1);
  }

  // One tile: gathers for a later tile, dequantisation, then the two products with the softmax
  // spread over the value product.
  auto step = [&](int it, auto slot) {
    constexpr int buf = decltype(slot)::value;
    wait_ring<kDmaWave>(min(kStages - 2, ntiles_run - 1 - it));
    lds_barrier();                          // tile `it` landed for every wave; slot it-1 is free
    if (it + kStages - 1 < ntiles_run) issue8(it + kStages - 1, (buf + kStages - 1) % kStages);
    dequant8(buf);                          // every wave is past the previous tile's products
    lds_barrier();
    const unsigned char* tile = lds_kv[0];
    const uint32_t valid = lds_valid[it];

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
    s16x4 vring[kRingV][2];
#pragma unroll
    for (int j = 0; j < kRingV; ++j) { vring[j][0] = v_frag(j, 0); vring[j][1] = v_frag(j, 1); }

    mask_keys(s, valid, hh);
    const float mloc = raw_max(s, 0, 16, -INFINITY) * a.scale_log2;
    // every lane sets its reference on the same tile (the first with a selected key): uniform
    if (__builtin_amdgcn_readfirstlane(m_run == kNoRef ? 1 : 0)) {
      const float m0 = xor32_max(mloc);
      if (m0 > -INFINITY) m_run = m0 + kRefMargin;
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) s[r] = prob(s[r], a.scale_log2, m_run);
    auto pack_p = [&](int k2) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = pack_bf16(s[8 * k2 + 2 * e], s[8 * k2 + 2 * e + 1]);
      return as_bf16x8(v);
    };
    bf16x8 pf[2];
    pf[0] = pack_p(0);
    float mx = mloc, psum = 0.f;
#pragma unroll
    for (int j = 0; j < 2 * kVBlocks; ++j) {
      const int k2 = j >> 4, mb = j & 15;
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vring[j % kRingV][0], vring[j % kRingV][1], 0, 1, 2, 3, 4, 5, 6, 7));
      if (j + kRingV < 2 * kVBlocks) {
        vring[j % kRingV][0] = v_frag(j + kRingV, 0);
        vring[j % kRingV][1] = v_frag(j + kRingV, 1);
      }
      o[mb] = mfma_bf16(vf, pf[k2], o[mb]);
      if (j < 8) {
        s[8 + j] = prob(s[8 + j], a.scale_log2, m_run);
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
#pragma unroll
  for (int i = 0; i < kStages - 1; ++i)
    if (i < ntiles_run) issue8(i, i);
  for (;;) {
    for (int it = 0; it < ntiles_run; it += kStages) {
      step(it, std::integral_constant<int, 0>{});
      if (it + 1 < ntiles_run) step(it + 1, std::integral_constant<int, 1>{});
      if (it + 2 < ntiles_run) step(it + 2, std::integral_constant<int, 2>{});
      if (it + 3 < ntiles_run) step(it + 3, std::integral_constant<int, 3>{});
    }
    static_assert(kStages == 4, "the main loop above is unrolled for a 4-slot ring");
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
      if (i < ntiles_run) issue8(i, i);
  }
  finish_split<NW>(a, o, m_run, l_run, row, split, gg, tid);
}

// ------------------------------------------------------------------------------------------------
static size_t align_up(size_t x, size_t al) { return (x + al - 1) / al * al; }

// Scratch of dsa_sparse_attn_noalloc: one copy per GPU, held until the process ends.  Host code
// never passes this name to a kernel (on the host it is only a handle); it resolves the device
// address once per device with hipGetSymbolAddress and passes that.  Nothing in it has to start at
// zero: the ready flags are compared with the call's own tag and cleared by their reader.
constexpr size_t kAttnScratchBytes = DSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

size_t attn_scratch_bytes() { return kAttnScratchBytes; }

hipError_t attn_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

#ifdef DSA_TIMELINE
extern "C" int dsa_timeline_reset_attn(void) {
  static unsigned long long zeros[kTimelineWgs][8];
  return hipMemcpyToSymbol(HIP_SYMBOL(g_timeline), zeros, sizeof zeros, 0, hipMemcpyHostToDevice) == hipSuccess ? 0 : 2;
}

extern "C" int dsa_timeline_fetch_attn(unsigned long long* host, int wgs) {
  if (wgs < 0 || wgs > kTimelineWgs) return 1;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_timeline), (size_t)wgs * 8 * sizeof(unsigned long long), 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? 0 : 2;
}
#endif

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
  // pays more for its partial output and its prologue than its extra parallelism returns, so
  // splits keep 4 tiles as long as the grid still has 128 workgroups.
  const int tiles = (S.top_k + kBK - 1) / kBK;
  const int per_split = std::max(rows * p.head_chunks, 1);
  int splits = (256 + per_split - 1) / per_split;
  const int min_splits = (128 + per_split - 1) / per_split;
  splits = std::max(min_splits, std::min(splits, tiles / 4));
  splits = std::max(1, std::min(splits, std::min(64, tiles)));
  const int tiles_per = (tiles + splits - 1) / splits;
  p.keys_per_split = tiles_per * kBK;
  p.n_splits = (tiles + tiles_per - 1) / tiles_per;
  // combine parts per (row, head group): about 256 combine workgroups in all; a part gives each
  // of its threads 1, 2, 4 or 8 of the group's 2048 units
  const int groups = std::max(rows * p.waves, 1);
  const int nt = 64 * p.groups_per_wg;
  const int max_parts = 2048 / nt, min_parts = std::max(1, 2048 / (8 * nt));
  int parts = min_parts;
  while (parts < max_parts && groups * parts * 2 <= 256) parts *= 2;
  p.comb_parts = parts;
  size_t off = 0;
  if (p.n_splits > 1) {
    p.off_ml = off; off = align_up(off + (size_t)rows * p.n_splits * S.heads * 2 * 4, 256);
    p.off_part = off; off = align_up(off + (size_t)rows * p.n_splits * p.waves * kPartWords * 4, 256);
    p.off_sync = off; off = align_up(off + (size_t)rows * p.waves * parts * p.n_splits * 8, 256);
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
  const bool split = p.n_splits > 1;
  s.part_ml = split ? reinterpret_cast<float*>(ws + p.off_ml) : nullptr;
  s.part_o = split ? reinterpret_cast<uint32_t*>(ws + p.off_part) : nullptr;
  s.sync = split ? reinterpret_cast<unsigned long long*>(ws + p.off_sync) : nullptr;
  s.tag = split ? next_call_tag() : 0ull;
  s.T = a.T; s.H = a.heads; s.K = a.top_k; s.max_pages = a.max_pages; s.num_pages = a.num_pages;
  s.n_splits = p.n_splits; s.keys_per_split = p.keys_per_split;
  s.max_seq_len = a.max_seq_len;
  s.scale_log2 = a.sm_scale * kLog2e;
  const int rows = a.B * a.T;
  s.rows = rows; s.head_chunks = p.head_chunks; s.comb_parts = p.comb_parts;
  // split workgroups first, then (several splits) the combine parts
  const long long n_main = (long long)rows * p.n_splits * p.head_chunks;
  const long long n_comb = split ? (long long)rows * p.waves * p.comb_parts : 0;
  const dim3 grid((unsigned)(n_main + n_comb));
  LaunchScope ls("sfa_main", st);
  const bool kv8 = a.kv_scale != nullptr;
  const unsigned long long kv_bytes = (unsigned long long)a.num_pages * kPage * kRowBytes;
  const bool buf = kv_bytes < 0xFFFFFFFFull;
  s.kv_bytes = buf ? (uint32_t)kv_bytes : 0u;
  if (p.groups_per_wg == 4) {
    if (kv8) hipLaunchKernelGGL(sfa_main_kv8<4>, grid, dim3(256), 0, st, s);
    // one query row per sequence: no row shares its selected latent rows with another, so they
    // stream past the caches; with several query rows per sequence the rows overlap and stay cached
    else if (buf && a.T == 1) hipLaunchKernelGGL((sfa_pipe<4, true, true>), grid, dim3(256), 0, st, s);
    else if (buf) hipLaunchKernelGGL((sfa_pipe<4, true>), grid, dim3(256), 0, st, s);
    else hipLaunchKernelGGL((sfa_pipe<4, false>), grid, dim3(256), 0, st, s);
  } else if (p.groups_per_wg == 2) {
    if (kv8) hipLaunchKernelGGL(sfa_main_kv8<2>, grid, dim3(128), 0, st, s);
    else if (buf) hipLaunchKernelGGL((sfa_pipe<2, true>), grid, dim3(128), 0, st, s);
    else hipLaunchKernelGGL((sfa_pipe<2, false>), grid, dim3(128), 0, st, s);
  } else {
    if (kv8) hipLaunchKernelGGL(sfa_main_kv8<1>, grid, dim3(64), 0, st, s);
    else if (buf) hipLaunchKernelGGL((sfa_pipe<1, true>), grid, dim3(64), 0, st, s);
    else hipLaunchKernelGGL((sfa_pipe<1, false>), grid, dim3(64), 0, st, s);
  }
  return hipGetLastError();
}

}  // namespace dsa
