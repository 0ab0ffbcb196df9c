/*
 * libfdec measurement probes. They are not part of decode attention: the
 * benchmark uses them to calibrate what the memory system delivers on this GPU
 * (a pure streaming read at the decode kernel's footprint) and to scale the
 * FETCH_SIZE / WRITE_SIZE hardware counters (a plain copy of known size).
 * Same conventions as fdec.h: caller-owned device memory, the caller's stream,
 * host-side validation before any launch.
 */
#ifndef FDEC_PROBE_H
#define FDEC_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Blocks the probes launch; `sink` must hold this many uint32 values. */
#define FDEC_PROBE_BLOCKS 2048

/*
 * Best-effort streaming read of `bytes` bytes at `src`: the attainable read
 * bandwidth the benchmark reports the decode kernels against. Two blocks per
 * compute unit, each reading one contiguous chunk with non-temporal 16-byte
 * loads (bytes a multiple of 16, src 16-byte aligned). Each block folds what
 * it read into one word of sink[FDEC_PROBE_BLOCKS] so the loads cannot be
 * dropped.
 */
int fdec_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/*
 * Streaming read through LDS, the way the split-KV map kernels stage K/V tiles
 * (global_load_lds_dwordx4 into a per-wave LDS ring, explicit waits, four waves
 * per block), without their arithmetic: the ceiling those kernels can reach.
 * per_cu (1..4) blocks per compute unit. Modes:
 *   FDEC_PROBE_STATIC   every wave streams one equal contiguous slice
 *                       (bytes a multiple of 4 KB);
 *   FDEC_PROBE_TICKETS  the bytes are cut into 256 KB items; the first
 *                       per_cu * CUs blocks take items by block index, every
 *                       later block takes the next one from a counter, so
 *                       compute units that finish early take more items
 *                       (bytes a multiple of 256 KB). The counter is
 *                       sink[FDEC_PROBE_BLOCKS] (int32): zero before the first
 *                       call on a sink; every call leaves it at zero.
 * src 256-byte aligned; sink holds FDEC_PROBE_BLOCKS + 1 uint32 values.
 */
#define FDEC_PROBE_STATIC 0
#define FDEC_PROBE_TICKETS 1
int fdec_probe_stream(const void *src, size_t bytes, uint32_t *sink, int mode, int per_cu, void *stream);

/* Plain copy of `bytes` bytes (multiple of 16, both 16-byte aligned). */
int fdec_probe_copy(void *dst, const void *src, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FDEC_PROBE_H */
