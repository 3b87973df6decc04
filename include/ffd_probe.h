/*
 * ffd_probe.h -- measurement aid shipped beside libffd (libffd_probe.so); not part of the decode
 * path.  The vendor HBM peak is a theoretical figure; the bandwidth a plain streaming read reaches
 * on the same chip is the practical ceiling the decode kernels are compared with.
 */
#ifndef FFD_PROBE_H
#define FFD_PROBE_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read of `bytes` bytes at `src`, split into n_groups contiguous chunks, one work-group
 * of 256 threads each (16-byte loads with the streaming cache policy, eight in flight per lane).
 * Work-group g writes the XOR of
 * the 16-byte words of its chunk to sink[16 g .. 16 g + 15], so sink holds n_groups * 16 bytes.
 *   src, sink  caller-owned device memory, 16-byte aligned
 *   bytes      a positive multiple of 16
 *   n_groups   1 .. 65535
 * Returns 0 when the kernel was launched (asynchronously on `stream`), 1 for invalid arguments
 * (nothing launched), 2 if the launch failed.
 */
int32_t ffd_probe_stream_read(const void* src, size_t bytes, int32_t n_groups, void* sink,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FFD_PROBE_H */
