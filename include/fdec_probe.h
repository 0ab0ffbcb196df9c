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
 * Streaming read of `bytes` bytes at `src` with 16-byte vector loads (bytes a
 * multiple of 16, src 16-byte aligned). Each block folds what it read into one
 * word of sink[FDEC_PROBE_BLOCKS] so the loads cannot be dropped.
 */
int fdec_probe_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Plain copy of `bytes` bytes (multiple of 16, both 16-byte aligned). */
int fdec_probe_copy(void *dst, const void *src, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FDEC_PROBE_H */
