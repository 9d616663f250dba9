// dsa_device.h -- device-side building blocks shared by the gfx950 kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kPage = 64;          // tokens per cache page
constexpr int kDimQK = 576;        // latent row width
constexpr int kDimV = 512;         // V columns of the latent row

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// 32x32 output tile, K = 16 bf16 per instruction.  Lane l supplies A[m = l%32][k = 8(l/32)..+7]
// and B[k = 8(l/32)..+7][n = l%32]; accumulator register r of lane l holds
// C[m = 8(r/4) + 4(l/32) + r%4][n = l%32].
__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// Same tile shape with K = 16 e4m3 values (8 bytes) per lane and operand.
__device__ __forceinline__ f32x16 mfma_fp8(long a, long b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Workgroup barrier that drains only this wave's LDS operations.  __syncthreads() also waits for
// every outstanding global load (vmcnt(0)), which would serialise a load pipeline that keeps data
// for later tiles in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct-to-LDS load of 16 bytes per lane: lane i's 16 bytes from `src` land at LDS byte address
// lds_base + 16*i (lds_base wave-uniform).  Written as inline assembly on purpose: the compiler
// treats its builtin form as an unknown write to LDS and makes every later LDS read wait for all
// outstanding global loads (vmcnt(0)), which serialises a ring of tiles kept in flight.  Callers
// count these loads themselves (wait_vmcnt) and put a barrier between landing and reading.
__device__ __forceinline__ void lds_dma16(const void* src, const void* lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_dst));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base), "v"(src)
               : "memory", "m0");
}

// Same, for 16-byte chunks of one row: lane i's 16 bytes come from sbase + voff (sbase
// wave-uniform, made scalar here; voff a 32-bit per-lane byte offset).
__device__ __forceinline__ void lds_dma16_rows(const void* sbase, uint32_t voff, const void* lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_dst));
  const uint64_t sb = reinterpret_cast<uintptr_t>(sbase);
  // readfirstlane returns a signed int: widen each half through uint32_t (no sign extension)
  const uint64_t sbu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sb >> 32)) << 32) |
                       (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sb);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(base), "v"(voff),
               "s"(sbu)
               : "memory", "m0");
}

// Same, with the nontemporal cache policy: for streams read once, so they do not displace other
// lines from the caches.
__device__ __forceinline__ void lds_dma16_rows_nt(const void* sbase, uint32_t voff, const void* lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_dst));
  const uint64_t sb = reinterpret_cast<uintptr_t>(sbase);
  const uint64_t sbu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sb >> 32)) << 32) |
                       (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sb);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(base), "v"(voff),
               "s"(sbu)
               : "memory", "m0");
}

// Waits until at most N of this wave's global loads (including direct-to-LDS loads) are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// Order-preserving map float -> uint32 (larger float -> larger key); -0 is folded onto +0 so the
// two compare equal.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Inclusive prefix sum over the 64 lanes of a wave: row shifts within each 16-lane row, then the
// last lane of row 0 is added to row 1 and of row 2 to row 3, then lane 31 to rows 2 and 3.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// x combined with the value of lane i ^ 32, as one VALU exchange (v_permlane32_swap) instead of
// an LDS permute round trip.  The swap leaves lane i's value and its partner's in the two results,
// whichever half moved; both operations are commutative, so every lane gets the same bits as
// x op partner.
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Exclusive prefix sum over a workgroup of NT threads (NT a multiple of 64).  `sh` holds NT/64
// words of LDS.  Returns this thread's exclusive prefix and the workgroup total.  Its barriers
// leave global loads in flight.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wid] = x;
  lds_barrier();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    uint32_t s = sh[i];
    pre += (i < wid) ? s : 0u;
    tot += s;
  }
  lds_barrier();
  total = tot;
  return pre + x - v;
}

// Device-side input checks.  Each translation unit that includes this header has its own flag
// word; a kernel that meets a violated precondition ORs a bit into it (vector atomic, only on the
// violating path) and carries on with the clamped value, so bad inputs give wrong numbers and a
// flag, never an out-of-bounds access.  dsa_debug_status() reads and clears the words.
constexpr uint32_t kFlagPage = 1u;         // a block-table entry in use lies outside [0, num_pages)
constexpr uint32_t kFlagLen = 2u;          // a sequence length lies outside [T, max_seq_len]
constexpr uint32_t kFlagIndex = 4u;        // an attention index is neither -1 nor a visible position
constexpr uint32_t kFlagSync = 8u;         // a wait for another workgroup's histogram clear timed out
static __device__ uint32_t g_input_flags;
__device__ __forceinline__ void flag_input(uint32_t bit) { atomicOr(&g_input_flags, bit); }

// Timeline build (-DDSA_TIMELINE, libdsa_timeline.so, a measurement variant of the library):
// thread 0 of each workgroup records the 100 MHz real-time counter at numbered points of the
// decode score kernel and the attention kernel, one row of 8 points per workgroup (the first 8192
// workgroups) in a per-translation-unit array; dsa_timeline_fetch_* copies it out.  In the normal
// build the stamps compile to nothing.
#ifdef DSA_TIMELINE
constexpr int kTimelineWgs = 8192;
static __device__ unsigned long long g_timeline[kTimelineWgs][8];
#define DSA_STAMP(point)                                                                         \
  do {                                                                                           \
    if (threadIdx.x == 0 && blockIdx.x < kTimelineWgs)                                           \
      g_timeline[blockIdx.x][point] = __builtin_amdgcn_s_memrealtime();                          \
  } while (0)
#else
#define DSA_STAMP(point) do { } while (0)
#endif

// Length of query row (b, t): keys 0..pos are visible, pos = seq_len - T + t.  seq_len is clamped
// to the block-table capacity so a bad length can never address past the table.
__device__ __forceinline__ int row_visible(const int32_t* seq_lens, int b, int T, int t, int cap) {
  int L = seq_lens[b];
  if (L < T || L > cap) {
    flag_input(kFlagLen);
    L = L < 0 ? 0 : (L > cap ? cap : L);
  }
  int n = L - T + t + 1;
  return n < 0 ? 0 : n;
}

__device__ __forceinline__ int clamp_page(int p, int num_pages) {
  if (p < 0 || p >= num_pages) {
    flag_input(kFlagPage);
    p = p < 0 ? 0 : num_pages - 1;
  }
  return p;
}

}  // namespace dsa
