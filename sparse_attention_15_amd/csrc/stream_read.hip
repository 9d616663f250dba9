// stream_read.hip -- a read-only streaming kernel that measures how fast this GPU can stream bytes
// out of HBM: the practical ceiling the bandwidth-bound kernels of the library are compared with.
// It is measurement support, built into its own library (libdsa_ceiling.so), not part of the
// DSA C ABI.
//
// Every thread issues 16-byte loads; a workgroup of 256 threads reads 4 KiB x UNROLL contiguous
// bytes per step and the grid strides over the buffer.  The loaded words are folded with XOR into
// one word per workgroup, written to `sink`, so the loads cannot be dropped; the 4 bytes per
// workgroup are the only writes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "stream_read.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int UNROLL, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, long long n16,
                                                           uint32_t* __restrict__ sink) {
  const long long step = (long long)gridDim.x * 256 * UNROLL;
  uint32_t acc = 0;
  long long i = (long long)blockIdx.x * 256 * UNROLL + threadIdx.x;
  for (; i + 256LL * (UNROLL - 1) < n16; i += step) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + 256LL * u) : src[i + 256LL * u];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int u = 0; u < UNROLL; ++u) {          // the ragged end of the buffer
    const long long j = i + 256LL * u;
    if (j < n16) {
      const u32x4 v = src[j];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  __shared__ uint32_t red[4];
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

extern "C" int dsa_stream_read(const void* buf, size_t bytes, int blocks, int unroll, uint32_t* sink,
                               hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || bytes % 16 != 0 || blocks < 1 || blocks > (1 << 20) ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return 1;
  const long long n16 = (long long)(bytes / 16);
  const u32x4* p = static_cast<const u32x4*>(buf);
  switch (unroll) {   // negative: the same with nontemporal loads
    case 1: stream_read_kernel<1, false><<<blocks, 256, 0, stream>>>(p, n16, sink); break;
    case 2: stream_read_kernel<2, false><<<blocks, 256, 0, stream>>>(p, n16, sink); break;
    case 4: stream_read_kernel<4, false><<<blocks, 256, 0, stream>>>(p, n16, sink); break;
    case 8: stream_read_kernel<8, false><<<blocks, 256, 0, stream>>>(p, n16, sink); break;
    case -2: stream_read_kernel<2, true><<<blocks, 256, 0, stream>>>(p, n16, sink); break;
    case -4: stream_read_kernel<4, true><<<blocks, 256, 0, stream>>>(p, n16, sink); break;
    case -8: stream_read_kernel<8, true><<<blocks, 256, 0, stream>>>(p, n16, sink); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
