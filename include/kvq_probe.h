/*
 * kvq_probe.h - reference kernels (C ABI): a plain streaming read, the
 * achievable-bandwidth reference for the decode kernels, and a matrix-core
 * loop and an LDS read loop, the achievable compute and LDS references for
 * the latent decode.
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

/* The matrix-core reference: `blocks` workgroups of 4 waves, each wave issuing
 * 8 * iters v_mfma_f32_32x32x16_f16 products (32,768 flop each) in two
 * independent accumulation chains, with operands held in registers and no
 * memory traffic, then folding its accumulators into the device word *sink.
 * Total flop = blocks * 4 * iters * 8 * 32768.  This is the dense fp16 product
 * the latent decode runs on (one 512-channel latent shared by every query
 * head, page "How DeepSeek-V4.1-Flash cut KV-cache storage by 4x via CSA2",
 * CSA2 section), so its rate is the compute ceiling that kernel can approach
 * on the part as clocked under matrix load.  Asynchronous on `stream`.  Returns
 * 0, -1 (KV_EINVAL) for blocks outside [1, 65535], iters outside [1, 2^20] or a
 * NULL sink, or -5 (KV_EDEVICE) when the launch fails. */
int kv_mfma_probe(int32_t blocks, int32_t iters, float* sink, void* stream);

/* The LDS reference: `blocks` workgroups of 4 waves, each wave reading 8 * iters
 * 16-byte words per lane (1 KiB per wave and read) from a 64 KiB LDS array
 * with conflict-free addresses, folded into *sink.  Bytes read from LDS =
 * blocks * 4 * iters * 8 * 1024.  The latent decode reads every dequantised
 * tile from LDS once per wave, so this rate bounds it next to the matrix
 * cores.  Asynchronous on `stream`.  Returns as kv_mfma_probe. */
int kv_lds_probe(int32_t blocks, int32_t iters, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_PROBE_H */
