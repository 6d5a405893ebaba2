/*
 * kvq_probe.h - a plain streaming read, the achievable-bandwidth reference for
 * the decode kernels (C ABI).
 *
 * Decode attention streams the whole packed cache from HBM once per generated
 * token, so its speed is bounded by the memory bandwidth the chip delivers to a
 * kernel (page "TurboQuant vs OSCAR vs EpiCache: the battle over KV-cache
 * compression", section on the KV-cache memory bottleneck).  The kernel here
 * does nothing but that read: 16-byte loads over a contiguous buffer, eight in
 * flight per thread, folded into one word.  Timing it next to the decode
 * kernels shows how far they are from what a pure read reaches on the part.
 */
#ifndef KVQ_PROBE_H
#define KVQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of device memory at `src` (16-byte aligned, bytes a
 * multiple of 16) and write a value derived from all of them to the device word
 * *sink (so no load can be skipped).  Asynchronous on `stream` (a hipStream_t;
 * NULL is the default stream).  Returns 0 (KV_OK), -1 (KV_EINVAL) for a NULL or
 * misaligned pointer or a size that is zero or not a multiple of 16, or -5
 * (KV_EDEVICE) when the launch fails. */
int kv_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_PROBE_H */
