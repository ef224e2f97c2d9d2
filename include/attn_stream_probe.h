/*
 * attn_stream_probe.h -- read-bandwidth probe shipped with libattn_decode.so.
 *
 * Not a step of the attention method: a measurement helper.  It streams a
 * device buffer HBM -> LDS with the loads the decode kernels use for their
 * cache (16-byte LDS-DMA loads with the non-temporal hint, 16 KB tiles, a
 * 5-deep ring, 4 wavefronts per workgroup, 2048 workgroups) and discards the
 * data.  Its rate is the ceiling a cache stream of that kind reaches on the
 * GPU, and benchmarks report the attention calls' achieved bandwidth as a
 * fraction of it, next to the fraction of the datasheet peak.
 */
#ifndef ATTN_STREAM_PROBE_H
#define ATTN_STREAM_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes of the device buffer `src` once.
 *   src    device memory, 16-byte aligned, at least `bytes` long; read only.
 *   bytes  a positive multiple of 32 MiB (2048 workgroups x 16 KB tiles).
 *   sink   device memory of 2048 unsigned ints; written only if the data
 *          hash to a fixed constant (it keeps the loads from being dead),
 *          so its contents are unspecified afterwards.
 *   stream hipStream_t as void* (NULL = null stream); the call only enqueues.
 * Returns ATTN_OK, ATTN_EINVAL (null pointer or bad size) or ATTN_EHIP
 * (launch error); attn_last_error() describes a failure.
 */
int attn_stream_read_probe(const void* src, size_t bytes, unsigned int* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_STREAM_PROBE_H */
