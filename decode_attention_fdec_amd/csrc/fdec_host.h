// Host-side helpers shared by the libfdec translation units: the thread-local
// error message behind fdec_last_error().
#pragma once

#include <cstdarg>

void fdec_clear_error();
// Records a printf-style message for fdec_last_error() and returns `status`.
int fdec_fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

#include <stddef.h>
#include <stdint.h>

struct fdec_kv;
struct fdec_append;

// fdec_decode in two steps, shared by the entry points that differ only in where
// the partial states live (a caller's workspace, or the library's own scratch).
// Validation of everything but the workspace; resolves the split count.
int fdec_decode_validate(const char *fn, const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                         int num_splits, float softmax_scale, const fdec_append *append, int fused, float *out,
                         float *lse, int *S_out);
// Bytes of the states (m, d [B, Hq, S], O~ [B, Hq, S, D], fp32, each 256-byte aligned).
size_t fdec_decode_state_bytes(int B, int Hq, int D, int S);
// The launches: states at `states` (256-byte aligned), arrival counters [B * Hkv]
// at `counters` (zero on entry, used when fused = 1).
int fdec_decode_launch(const char *fn, const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                       int S, float softmax_scale, const fdec_append *append, int fused, float *out, float *lse,
                       int *counters, char *states, void *stream);

// The debug mode (FDEC_DEBUG in the environment, or fdec_set_debug): checks the
// call's device data with fdec_check_inputs and returns FDEC_ERR_INVALID_ARG,
// before any launch, when some of it is out of range; FDEC_OK when the mode is off.
int fdec_debug_gate(const char *fn, int B, const fdec_kv *kv, const int32_t *seq_lens, const fdec_append *append,
                    const int32_t *prefix_pages, int prefix_len, void *stream);
