/*
 * kvq_probe.h -- measurement support exported by libkvq, outside the
 * attention path: a streaming-read kernel that gives the practical HBM
 * read-bandwidth ceiling of the device, which the decode's bandwidth is
 * compared with.  Same conventions as kvq.h (device pointers, host-side
 * validation before any device work, asynchronous on `stream`).
 */
#ifndef KVQ_PROBE_H
#define KVQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streams `bytes` of device memory at `src` through non-temporal vector loads
 * and discards them.  `src` device, 16-byte aligned, bytes a multiple of 16;
 * `sink` device, one uint32 that is written only if the XOR of everything a
 * lane read equals `key` (pick a key that no lane's fold takes, or ignore the
 * sink).  blocks: workgroups of 256 threads, 0 = eight per compute unit.
 * Returns 0, -1 (KVQ_E_ARG) on a null pointer, misalignment or a size that is
 * not a multiple of 16, or -6 (KVQ_E_HIP) if the launch fails. */
int kvq_stream_read(const void *src, size_t bytes, uint32_t key, uint32_t *sink, int32_t blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_PROBE_H */
