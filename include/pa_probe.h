/*
 * pa_probe.h -- HBM read-ceiling probes of libpa.so (measurement only).
 *
 * The decode step streams the KV cache once ("How we built the most efficient
 * inference engine for Cloudflare's network", section "Batching to feed the
 * Tensor Cores": each decoded token revisits every cached K/V of its
 * sequence), and the FP8 cache makes it memory-bound ("Cloudflare quantizes
 * Kimi and GLM caches for 41% faster inference", KV cache quantization
 * paragraph).  Its roofline is therefore the rate at which one GPU can read
 * HBM.  These two entry points measure that rate for two access patterns, so
 * the attention kernel's bandwidth can be quoted against a measured ceiling as
 * well as the nominal 8 TB/s:
 *   - pa_probe_stream: a plain contiguous read of a buffer;
 *   - pa_probe_gather: reads of whole blocks at the positions an id table
 *     gives, one run of ids per wave -- the decode kernel's pattern (a 2 KiB
 *     block is one (page, KV head) of an FP8 cache with 16 tokens of 128
 *     dims; 4 KiB the same in BF16).
 * Both load with the decode kernel's instructions (one 16-byte non-temporal
 * load per lane, so a wave reads 1 KiB contiguously) and reduce what they
 * read into one word per wave, written to `sink` so no load is dead.
 *
 * Conventions as in pa.h: device pointers, caller-owned buffers, nothing
 * allocated, asynchronous on `stream`, argument errors returned (PA_ERR_*
 * codes of pa.h) before any launch.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` of `buf` once.  `waves` waves (a multiple of 4) each read one
 * contiguous share of bytes / waves, front to back; bytes must be a multiple
 * of 1024 * waves.  buf: 16-byte aligned.  sink: uint32 [waves].  Returns
 * PA_OK, PA_ERR_INVALID_ARG or PA_ERR_LAUNCH. */
int pa_probe_stream(const void *buf, size_t bytes, int32_t waves, uint32_t *sink,
                    hipStream_t stream);

/* Block gather: wave w reads blocks ids[w * ids_per_wave + i] for i = 0 ..
 * ids_per_wave - 1, in order; block k occupies bytes [k * block_bytes,
 * (k + 1) * block_bytes) of `pool`.  block_bytes: 1024, 2048 or 4096.
 * `inflight` (1, 2, 4 or 8): blocks whose loads a wave issues before it
 * waits for them.  Ids outside [0, pool_bytes / block_bytes) are read as
 * block 0 (no access leaves the pool).  waves: a multiple of 4; ids_per_wave
 * a multiple of inflight.  pool: 16-byte aligned; ids: int32 [waves *
 * ids_per_wave]; sink: uint32 [waves].  Returns PA_OK, PA_ERR_INVALID_ARG or
 * PA_ERR_LAUNCH. */
int pa_probe_gather(const void *pool, size_t pool_bytes, const int32_t *ids, int32_t waves,
                    int32_t ids_per_wave, int32_t block_bytes, int32_t inflight,
                    uint32_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
