/*
 * nvfp4_membench.h -- HBM stream kernels of libnvfp4_membench.so, the
 * measurement companion of libnvfp4.so (not part of the quantization ABI).
 *
 * They measure the bandwidth ceilings a memory-bound kernel on this GPU is
 * compared with: a read-only stream, a write-only stream and a copy, each moving 16
 * bytes per lane per access from a persistent grid of workgroups that walk the
 * buffer in grid-stride order with several accesses in flight per lane.  Also
 * used as the known-size kernels that scale the profiler's HBM byte counters.
 *
 * Conventions: device pointers, 16-byte aligned; `bytes` a multiple of 16;
 * `stream` a hipStream_t as void*; asynchronous; the library allocates nothing.
 * Return 0 on success, 1 on a bad argument (nothing launched), 2 on a launch
 * failure.
 */
#ifndef NVFP4_MEMBENCH_H
#define NVFP4_MEMBENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[i] = src[i] for bytes / 16 vectors of 16 bytes.  grid: workgroups of 256
 * lanes (0 = four per compute unit). */
int membench_copy(void* dst, const void* src, size_t bytes, int grid, void* stream);

/* Reads every byte of src; the XOR of everything read lands in sink[0..3]
 * (four uint32, device) so that no load can be dropped. */
int membench_read(const void* src, size_t bytes, uint32_t* sink, int grid, void* stream);

/* dst[i] = value (as four uint32 per 16 bytes). */
int membench_write(void* dst, size_t bytes, uint32_t value, int grid, void* stream);

#ifdef __cplusplus
}
#endif
#endif
