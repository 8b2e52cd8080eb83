/*
 * kvq_bench.h — a measurement reference exported by libkvq next to the cache API (include/kvq.h).
 *
 * It is not a step of the method: it tells how fast this GPU reads a buffer of a given size when
 * nothing else is done with the bytes, so that the decode-attention kernels can be reported as a
 * fraction of that achievable bandwidth next to the HBM peak.
 */
#ifndef KVQ_BENCH_H
#define KVQ_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at device pointer `dev` once (16-byte loads, coalesced, eight in flight per
 * lane, at most 2048 workgroups of 256 threads striding over the buffer).  Each lane folds its words
 * with XOR and writes the device word *out only if the fold equals a fixed constant (so the loads
 * cannot be dropped, and in practice nothing is written).  dev: 16-byte aligned; bytes: a non-zero
 * multiple of 16 (else KVQ_EINVAL, nothing launched).  One launch on `stream`, asynchronous; reads
 * nothing past dev + bytes.  The caller owns both buffers. */
kvq_status kvq_stream_read(const void* dev, uint64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_BENCH_H */
