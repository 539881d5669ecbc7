/*
 * quest_probe.h -- C ABI of libquest_probe.so: HBM read probes for MI355X
 * (gfx950).  Measurement tools, not part of the Quest path: they time what
 * plain reads of the step's two access patterns achieve on this chip, so the
 * benchmark can report each kernel against the practical read rate beside
 * the 8 TB/s nameplate (the "one throughput benchmark" of the Sparse-vLLM
 * skill page "add-sparse-method", Validation, needs a denominator that the
 * hardware can reach).
 *
 * Conventions: device pointers, asynchronous on `stream` (a hipStream_t as
 * void*), nothing allocated, nothing copied to the host.  Each kernel folds
 * every loaded word into an XOR and writes sink[0] only if the result
 * equals `never` (choose a value no data produces), so it reads and does not
 * write.  Return: 0, -1 for a NULL pointer, -2 for a misaligned buffer or a
 * bad size, -3 for an unsupported chunk size, -6 when HIP rejects the
 * launch (nothing is launched on -1..-3).
 */
#ifndef QUEST_PROBE_H
#define QUEST_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16, buf 16-byte aligned) once, contiguously,
 * with 16-byte loads from `work_groups` work-groups of 256 threads
 * (grid-stride, 8 loads in flight per thread). */
int quest_probe_stream_read(const void *buf, size_t bytes, int work_groups, uint32_t never,
                            uint32_t *sink, void *stream);

/* Reads n_chunks pairs of chunks of chunk_bytes (2048, 4096 or 8192) each:
 * chunk c of `a` and chunk c of `b` both start at 16-byte element offset
 * chunk_offsets16[c] (device int64 array) -- one K page and one V page of one
 * KV head in the cache layout.  One wave per pair, `work_groups` work-groups
 * of 4 waves. */
int quest_probe_gather_read(const void *a, const void *b, const int64_t *chunk_offsets16,
                            int n_chunks, int chunk_bytes, int work_groups, uint32_t never,
                            uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QUEST_PROBE_H */
