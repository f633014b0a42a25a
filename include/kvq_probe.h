/*
 * kvq_probe.h -- C ABI of libkvq_probe: a measurement aid that sits beside
 * libkvq and is no part of attention.  The decode's KV reads are rated against
 * the HBM rate of a plain streaming read of the same bytes made with the same
 * load instructions; this library provides that read.  Benchmarks load it,
 * the attention path never does.
 *
 * Return values are those of kvq_status (kvq.h).
 */
#ifndef KVQ_PROBE_H
#define KVQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * kvq_stream_read -- reads `bytes` (a multiple of 16) at the device pointer
 * `src` once with the loads the decode uses (non-temporal, 16 bytes per lane),
 * `workgroups` workgroups of 256 threads each reading one contiguous slice, and
 * does nothing else.  Its duration is the HBM floor for reading that many
 * bytes.  `sink` (device) must hold workgroups * 4096 bytes; a thread stores
 * there only if the XOR of what it read equals one fixed 64-bit pattern, so
 * the loads cannot be dropped.  Enqueues on `stream` (hipStream_t, NULL = the
 * null stream) and returns at once.  KVQ_EINVAL for a NULL pointer,
 * bytes % 16 != 0 or workgroups outside [1, 65535]; KVQ_EHIP for a launch
 * error.
 */
int kvq_stream_read(const void* src, size_t bytes, int32_t workgroups, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_PROBE_H */
