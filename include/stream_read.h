/* stream_read.h -- measurement support, not part of the DSA C ABI (libdsa_ceiling.so).
 *
 * dsa_stream_read reads `bytes` bytes of device memory at `buf` (16-byte aligned, bytes a multiple
 * of 16) with 16-byte loads, `blocks` workgroups of 256 threads striding over the buffer, each
 * thread keeping `unroll` (1, 2, 4 or 8) loads in flight (-2, -4, -8: the same with nontemporal
 * loads), and writes one 32-bit XOR of what each
 * workgroup read to sink[0 .. blocks) (device memory, caller-owned).  Asynchronous on `stream`.
 * Returns 0, 1 for a bad argument (nothing launched), 2 when the launch failed.  Timing it over a
 * buffer larger than the 256 MiB last-level cache gives the HBM streaming-read ceiling. */
#ifndef STREAM_READ_H
#define STREAM_READ_H
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>
#ifdef __cplusplus
extern "C" {
#endif
int dsa_stream_read(const void *buf, size_t bytes, int blocks, int unroll, uint32_t *sink,
                    hipStream_t stream);
#ifdef __cplusplus
}
#endif
#endif
