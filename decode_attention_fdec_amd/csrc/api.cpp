// libfdec C ABI: host-side validation, workspace layout and kernel dispatch.
// Every check runs before any launch; a failing call launches nothing.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/fdec.h"
#include "fdec_host.h"
#include "fdec_internal.h"

namespace {

thread_local char g_err[512] = "";

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Every layout starts with the fused path's arrival counters [B * Hkv] (zero
// between calls), so that a workspace shared by every kind of call keeps them
// intact: the balanced split's (first slot, count) records come after them.
size_t counter_bytes(int B, int Hkv) { return align_up((size_t)B * Hkv * sizeof(int32_t)); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct WsLayout {
    size_t cnt, pm, pd, po, total;
};

WsLayout ws_layout(int B, int Hq, int Hkv, int D, int S) {
    WsLayout w;
    const size_t states = (size_t)B * Hq * S;
    w.cnt = 0;
    w.pm = counter_bytes(B, Hkv);
    w.pd = align_up(w.pm + states * sizeof(float));
    w.po = align_up(w.pd + states * sizeof(float));
    w.total = align_up(w.po + states * D * sizeof(float));
    return w;
}

int check_hip(hipError_t e, const char *what) {
    if (e == hipSuccess) return FDEC_OK;
    return fdec_fail(FDEC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Stage timing (fdec_trace_start / fdec_trace_stop): while on, every call of
// this thread records an event on its stream before its first kernel (kind 0)
// and after its k-th kernel (kind k).
struct Trace {
    bool on = false;
    int cap = 0;
    std::vector<hipEvent_t> ev;
    std::vector<int> kind;
};
thread_local Trace g_trace;

void trace_record(hipStream_t st, int kind) {
    Trace &t = g_trace;
    if (!t.on || (int)t.kind.size() >= t.cap) return;
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return;
    if (hipEventRecord(e, st) != hipSuccess) {
        (void)hipEventDestroy(e);
        return;
    }
    t.ev.push_back(e);
    t.kind.push_back(kind);
}

// The launches of one call: records the call's start, then each kernel's end.
struct Launches {
    hipStream_t st;
    int k = 0;
    explicit Launches(hipStream_t s) : st(s) { trace_record(st, 0); }
    int done(hipError_t e, const char *what) {
        const int rc = check_hip(e, what);
        if (rc == FDEC_OK) trace_record(st, ++k);
        return rc;
    }
};

int page_shift_of(int ps) {
    if (ps <= 0 || (ps & (ps - 1))) return -1;
    int s = 0;
    while ((1 << s) < ps) ++s;
    return s;
}

// Checks shared by fdec_decode, fdec_decode_partials and fdec_cascade_decode.
int validate_common(const char *fn, const void *q, int B, int Hq, const fdec_kv *kv,
                    const int32_t *seq_lens, float softmax_scale) {
    if (!kv) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: kv is NULL", fn);
    if (B < 0) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: B = %d < 0", fn, B);
    if (Hq < 1 || kv->num_kv_heads < 1)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: Hq = %d and Hkv = %d must be >= 1", fn, Hq, kv->num_kv_heads);
    if (Hq % kv->num_kv_heads != 0)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: Hq = %d is not a multiple of Hkv = %d", fn, Hq,
                         kv->num_kv_heads);
    const int G = Hq / kv->num_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fdec_fail(FDEC_ERR_UNSUPPORTED, "%s: GQA group size %d not built (1, 2, 4, 8)", fn, G);
    if (kv->head_dim != 128 && kv->head_dim != 64)
        return fdec_fail(FDEC_ERR_UNSUPPORTED, "%s: head_dim %d not built (128, 64)", fn, kv->head_dim);
    if (kv->dtype != FDEC_F16 && kv->dtype != FDEC_BF16 && kv->dtype != FDEC_FP8_E4M3)
        return fdec_fail(FDEC_ERR_UNSUPPORTED, "%s: dtype %d not built (fp16 = 0, bf16 = 1, fp8 e4m3 = 2)", fn,
                         kv->dtype);
    const int es = kv->dtype == FDEC_FP8_E4M3 ? 1 : 2;  // bytes per element
    if (kv->page_size < 0 || kv->page_size % 16 != 0)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: page_size %d must be 0 or a multiple of 16", fn,
                         kv->page_size);
    if (B == 0) return FDEC_OK;
    if (!q || !kv->k || !kv->v || !seq_lens)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: q, kv->k, kv->v and seq_lens must be non-NULL", fn);
    if (!aligned16(q) || !aligned16(kv->k) || !aligned16(kv->v))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: q, k and v must be 16-byte aligned", fn);
    if (kv->s_outer < 0 || kv->s_token < 0 || kv->s_head < 0 || (kv->s_outer * es) % 16 ||
        (kv->s_token * es) % 16 || (kv->s_head * es) % 16)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: strides must be non-negative multiples of 16 bytes", fn);
    if ((int64_t)kv->s_token * es * 15 > INT32_MAX)
        return fdec_fail(FDEC_ERR_UNSUPPORTED, "%s: token stride too large", fn);
    if (kv->page_size == 0) {
        if (kv->capacity < 1) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: contiguous cache needs capacity >= 1", fn);
    } else {
        if (kv->cache_batch_idx)
            return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: cache_batch_idx is for contiguous caches (a paged cache "
                             "maps requests through its page table)", fn);
        if (!kv->page_table || kv->max_pages_per_seq < 1)
            return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: paged cache needs page_table and max_pages_per_seq >= 1", fn);
        const int64_t cap = (int64_t)kv->max_pages_per_seq * kv->page_size;
        if (cap > INT32_MAX) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: capacity overflows int32", fn);
        if (kv->capacity != 0 && kv->capacity != cap)
            return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: capacity %d != max_pages_per_seq * page_size = %lld", fn,
                             kv->capacity, (long long)cap);
    }
    if (!std::isfinite(softmax_scale))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: softmax_scale is not finite", fn);
    return FDEC_OK;
}

// KV heads (one wave each) per vector split-KV block: the largest divisor of
// Hkv up to 8 waves (4 when G = 8 at D = 128, whose waves need the whole
// register file) that still launches a block per compute unit; with fewer
// blocks than that even at one head per block, one head per block.
#ifndef FDEC_HPB_CAP
#define FDEC_HPB_CAP 8
#endif
constexpr int kTargetBlocks = 256;  // MI355X compute units
int heads_per_block(int B, int hkv, int G, int D, int S) {
    const int cap = std::min((G >= 8 && D >= 128) ? fdec::kMapMaxWavesBig : fdec::kMapMaxWaves, FDEC_HPB_CAP);
    for (int w = cap; w > 1; --w)
        if (hkv % w == 0 && (int64_t)B * (hkv / w) * S >= kTargetBlocks) return w;
    return 1;
}

// Prefix tokens per cascade split: a whole number of 64-token tiles.
int64_t cascade_chunk(int prefix_len, int splits) {
    int64_t per = ((int64_t)std::max(prefix_len, 1) + splits - 1) / splits;
    return (per + 63) / 64 * 64;
}

int capacity_of(const fdec_kv *kv) {
    return kv->page_size == 0 ? kv->capacity : kv->max_pages_per_seq * kv->page_size;
}

int validate_append(const char *fn, const fdec_append *a, const fdec_kv *kv) {
    if (!a) return FDEC_OK;
    if (!a->k_new || !a->v_new)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: append needs k_new and v_new", fn);
    if (a->rotary_dim < 0 || a->rotary_dim % 2 || a->rotary_dim > kv->head_dim)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: rotary_dim %d must be even and in [0, head_dim]", fn,
                         a->rotary_dim);
    if (a->rotary_dim > 0 && (!a->rope_cos || !a->rope_sin || a->rope_max_pos < 1))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: rotary needs rope_cos, rope_sin and rope_max_pos >= 1", fn);
    return FDEC_OK;
}

fdec::MapParams map_params(const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens, int S,
                           float scale, const fdec_append *append) {
    fdec::MapParams p;
    std::memset(&p, 0, sizeof(p));
    p.q = q;
    p.k = static_cast<const char *>(kv->k);
    p.v = static_cast<const char *>(kv->v);
    p.s_outer = kv->s_outer;
    p.s_token = kv->s_token;
    p.s_head = kv->s_head;
    p.page_table = kv->page_size ? kv->page_table : nullptr;
    p.max_pages = kv->max_pages_per_seq;
    p.page_size = kv->page_size;
    p.page_shift = page_shift_of(kv->page_size);
    p.seq_lens = seq_lens;
    p.batch_idx = kv->cache_batch_idx;
    p.leftpad = kv->cache_leftpad;
    p.q_len = 1;
    p.q_groups = 1;
    if (kv->dtype == FDEC_FP8_E4M3) {
        p.kv_fp8 = 1;
        p.k_descale = kv->k_descale;
        p.v_descale = kv->v_descale;
    }
    p.B = B;
    p.Hq = Hq;
    p.Hkv = kv->num_kv_heads;
    p.heads_per_block = heads_per_block(B, kv->num_kv_heads, Hq / kv->num_kv_heads, kv->head_dim, S);
    p.chunk = (int)fdec_split_chunk(capacity_of(kv), S);
    if (scale == 0.0f) scale = 1.0f / std::sqrt((float)kv->head_dim);
    p.scale_log2 = scale * 1.4426950408889634f;
    p.dtype = kv->dtype == FDEC_FP8_E4M3 ? FDEC_BF16 : kv->dtype;  // the queries' (and MFMA's) type
    p.head_dim = kv->head_dim;
    p.mode = fdec::kPlain;
    if (append) {
        p.k_new = append->k_new;
        p.v_new = append->v_new;
        p.rotary_dim = append->rotary_dim;
        p.rope_cos = append->rope_cos;
        p.rope_sin = append->rope_sin;
        p.mode = append->rotary_dim > 0 ? fdec::kAppendRope : fdec::kAppend;
    }
    // GQA groups of 4 at D = 128 run on matrix cores unless FDEC_MAP_PATH=vector.
    const char *path = std::getenv("FDEC_MAP_PATH");
    if (fdec::map_mfma_eligible(p) && !(path && std::strcmp(path, "vector") == 0)) {
        p.mfma = 1;
        p.heads_per_block = 1;
        for (int w = fdec::kMapMfmaWaves; w > 1; --w)
            if (p.Hkv % w == 0) {
                p.heads_per_block = w;
                break;
            }
    }
    return p;
}

int resolve_splits(const char *fn, int num_splits, int B, int Hq, const fdec_kv *kv, int *S) {
    if (num_splits < 0 || num_splits > FDEC_MAX_SPLITS)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: num_splits %d outside [0, %d]", fn, num_splits, FDEC_MAX_SPLITS);
    if (num_splits > 0) {
        *S = num_splits;
        return FDEC_OK;
    }
    int rc = fdec_plan_kv(B, Hq, kv->num_kv_heads, nullptr, capacity_of(kv), kv->page_size, kv->dtype, 256, S);
    return rc;
}

}  // namespace

void fdec_clear_error() { g_err[0] = '\0'; }

int fdec_fail(int status, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

extern "C" const char *fdec_status_string(int status) {
    switch (status) {
        case FDEC_OK: return "ok";
        case FDEC_ERR_INVALID_ARG: return "invalid argument";
        case FDEC_ERR_UNSUPPORTED: return "unsupported configuration";
        case FDEC_ERR_WORKSPACE: return "workspace missing or too small";
        case FDEC_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" const char *fdec_last_error(void) { return g_err; }

extern "C" size_t fdec_workspace_size(int B, int Hq, int Hkv, int head_dim, int num_splits) {
    if (B < 0 || Hq < 1 || Hkv < 1 || head_dim < 1 || num_splits < 1) return 0;
    return ws_layout(B, Hq, Hkv, head_dim, num_splits).total;
}

extern "C" int fdec_workspace_init(void *workspace, size_t bytes, void *stream) {
    fdec_clear_error();
    if (!workspace) return fdec_fail(FDEC_ERR_WORKSPACE, "fdec_workspace_init: workspace is NULL");
    if (!aligned16(workspace)) return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_workspace_init: workspace not 16-byte aligned");
    // The counters sit at the start; zero the whole counter region any call could use.
    size_t words = bytes / 4;
    return check_hip(fdec::launch_zero_words(workspace, words, static_cast<hipStream_t>(stream)),
                     "fdec_workspace_init");
}

// Validation of fdec_decode's arguments other than the workspace; resolves the
// split count (num_splits = 0: planned from the capacity).
int fdec_decode_validate(const char *fn, const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                         int num_splits, float softmax_scale, const fdec_append *append, int fused, float *out,
                         float *lse, int *S_out) {
    int rc = validate_common(fn, q, B, Hq, kv, seq_lens, softmax_scale);
    if (rc) return rc;
    if ((rc = validate_append(fn, append, kv))) return rc;
    if (fused != 0 && fused != 1) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: fused must be 0 or 1", fn);
    if ((rc = resolve_splits(fn, num_splits, B, Hq, kv, S_out))) return rc;
    if (B == 0) return FDEC_OK;
    if (!out) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if ((reinterpret_cast<uintptr_t>(out) & 7u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: out must be 8-byte and lse 4-byte aligned", fn);
    return FDEC_OK;
}

size_t fdec_decode_state_bytes(int B, int Hq, int D, int S) {
    // the state part of ws_layout, from its 256-byte aligned start
    return ws_layout(B, Hq, 1, D, S).total - counter_bytes(B, 1);
}

// fdec_decode's launches once validated: states (m, d, O~ as in ws_layout) from
// `states`, arrival counters [B * Hkv] at `counters` (all zero; fused only).
int fdec_decode_launch(const char *fn, const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                       int S, float softmax_scale, const fdec_append *append, int fused, float *out, float *lse,
                       int *counters, char *states, void *stream) {
    if (B == 0) return FDEC_OK;
    if (int rc = fdec_debug_gate(fn, B, kv, seq_lens, append, nullptr, 0, stream)) return rc;
    const WsLayout w = ws_layout(B, Hq, 1, kv->head_dim, S);
    const size_t base = counter_bytes(B, 1);
    fdec::MapParams p = map_params(q, B, Hq, kv, seq_lens, S, softmax_scale, append);
    p.pm = reinterpret_cast<float *>(states + (w.pm - base));
    p.pd = reinterpret_cast<float *>(states + (w.pd - base));
    p.po = reinterpret_cast<float *>(states + (w.po - base));
    p.s_total = S;
    p.s_offset = 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Launches run(st);
    if (fused) {
        p.counters = counters;
        p.out = out;
        p.lse = lse;
        return run.done(fdec::launch_map(p, S, st), "fdec_decode: map+merge launch");
    }
    int rc = run.done(fdec::launch_map(p, S, st), "fdec_decode: map launch");
    if (rc) return rc;
    (void)fn;
    return run.done(fdec::launch_merge(p.po, p.pm, p.pd, B, Hq, S, kv->head_dim, out, lse, st),
                    "fdec_decode: merge launch");
}

extern "C" int fdec_decode(const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                           int num_splits, float softmax_scale, const fdec_append *append, int fused,
                           float *out, float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    fdec_clear_error();
    const char *fn = "fdec_decode";
    int S = 0;
    int rc = fdec_decode_validate(fn, q, B, Hq, kv, seq_lens, num_splits, softmax_scale, append, fused, out, lse, &S);
    if (rc || B == 0) return rc;
    const WsLayout w = ws_layout(B, Hq, kv->num_kv_heads, kv->head_dim, S);
    if (!workspace || workspace_bytes < w.total)
        return fdec_fail(FDEC_ERR_WORKSPACE, "%s: workspace of %zu bytes needed for %d splits, got %zu", fn,
                         w.total, S, workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: workspace not 16-byte aligned", fn);
    char *ws = static_cast<char *>(workspace);
    return fdec_decode_launch(fn, q, B, Hq, kv, seq_lens, S, softmax_scale, append, fused, out, lse,
                              reinterpret_cast<int *>(ws + w.cnt), ws + w.pm, stream);
}

extern "C" int fdec_decode_multi(const void *q, int B, int q_len, int Hq, const fdec_kv *kv,
                                 const int32_t *seq_lens, int num_splits, float softmax_scale, float *out,
                                 float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    fdec_clear_error();
    const char *fn = "fdec_decode_multi";
    if (q_len < 1 || q_len > FDEC_MAX_QLEN)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: q_len %d outside [1, %d]", fn, q_len, FDEC_MAX_QLEN);
    int rc = validate_common(fn, q, B, Hq, kv, seq_lens, softmax_scale);
    if (rc) return rc;
    int S = 0;
    if ((rc = resolve_splits(fn, num_splits, B, Hq, kv, &S))) return rc;
    if (B == 0) return FDEC_OK;
    if (!out) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if ((reinterpret_cast<uintptr_t>(out) & 7u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: out must be 8-byte and lse 4-byte aligned", fn);
    if ((int64_t)B * q_len * Hq > INT32_MAX)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: B * q_len * Hq overflows int32", fn);
    const WsLayout w = ws_layout(B * q_len, Hq, kv->num_kv_heads, kv->head_dim, S);
    if (!workspace || workspace_bytes < w.total)
        return fdec_fail(FDEC_ERR_WORKSPACE, "%s: workspace of %zu bytes needed for %d splits, got %zu", fn,
                         w.total, S, workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: workspace not 16-byte aligned", fn);
    fdec::MapParams p = map_params(q, B, Hq, kv, seq_lens, S, softmax_scale, nullptr);
    const int G = Hq / kv->num_kv_heads;
    // one query token: fdec_decode's own map kernel (vector or matrix-core), so
    // the result is its two-kernel result bitwise for every shape
    const bool mt16 = q_len > 1 && fdec::mt16_eligible(q_len, G, kv->head_dim) &&
                      (kv->page_size == 0 || kv->page_size % 16 == 0) && std::getenv("FDEC_MULTI_PATH") == nullptr;
    if (q_len > 1 && !mt16 && !(p.mfma && G == 4))
        return fdec_fail(FDEC_ERR_UNSUPPORTED,
                         "%s: several query tokens need head_dim 128 and page_size a multiple of 16", fn);
    const int ql = fdec::mfma_tokens_per_wave(q_len);
    p.q_len = q_len;
    p.q_groups = (q_len + ql - 1) / ql;
    if ((int64_t)B * p.q_groups > 65535)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: B * ceil(q_len / %d) exceeds the grid", fn, ql);
    char *ws = static_cast<char *>(workspace);
    p.pm = reinterpret_cast<float *>(ws + w.pm);
    p.pd = reinterpret_cast<float *>(ws + w.pd);
    p.po = reinterpret_cast<float *>(ws + w.po);
    p.s_total = S;
    p.s_offset = 0;
    if ((rc = fdec_debug_gate(fn, B, kv, seq_lens, nullptr, nullptr, 0, stream))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Launches run(st);
    if ((rc = run.done(mt16 ? fdec::launch_map_mt16(p, S, st) : fdec::launch_map(p, S, st),
                       "fdec_decode_multi: map launch")))
        return rc;
    return run.done(fdec::launch_merge(p.po, p.pm, p.pd, B, Hq, S, kv->head_dim, out, lse, st, q_len),
                    "fdec_decode_multi: merge launch");
}

extern "C" int fdec_decode_partials(const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                                    int num_splits, float softmax_scale, const fdec_append *append,
                                    float *part_o, float *part_m, float *part_d, void *stream) {
    fdec_clear_error();
    const char *fn = "fdec_decode_partials";
    int rc = validate_common(fn, q, B, Hq, kv, seq_lens, softmax_scale);
    if (rc) return rc;
    if ((rc = validate_append(fn, append, kv))) return rc;
    if (num_splits < 1 || num_splits > FDEC_MAX_SPLITS)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: num_splits %d outside [1, %d]", fn, num_splits, FDEC_MAX_SPLITS);
    if (B == 0) return FDEC_OK;
    if (!part_o || !part_m || !part_d)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: part_o, part_m and part_d must be non-NULL", fn);
    if (!aligned16(part_o) || (reinterpret_cast<uintptr_t>(part_m) & 3u) || (reinterpret_cast<uintptr_t>(part_d) & 3u))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: part_o must be 16-byte aligned", fn);
    fdec::MapParams p = map_params(q, B, Hq, kv, seq_lens, num_splits, softmax_scale, append);
    p.po = part_o;
    p.pm = part_m;
    p.pd = part_d;
    p.s_total = num_splits;
    p.s_offset = 0;
    if ((rc = fdec_debug_gate(fn, B, kv, seq_lens, append, nullptr, 0, stream))) return rc;
    Launches run(static_cast<hipStream_t>(stream));
    return run.done(fdec::launch_map(p, num_splits, static_cast<hipStream_t>(stream)), "fdec_decode_partials");
}

// Balanced split: blocks per group of KV heads (0 = one per compute unit over all groups).
// Default block count of the balanced split: per_cu blocks per compute unit
// over all groups of KV heads (16-bit caches: 1; float8 caches: 2, whose
// tiles take half the LDS and whose blocks then overlap each other's latency).
int device_cus() {
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
        cu = 256;
    return cu;
}

int balanced_blocks(int Hkv, int num_blocks, int per_cu) {
    if (num_blocks > 0) return num_blocks;
    int hpb = 1;
    for (int w = fdec::kMapMfmaWaves; w > 1; --w)
        if (Hkv % w == 0) {
            hpb = w;
            break;
        }
    return std::max(1, std::min(FDEC_MAX_SPLITS, per_cu * device_cus() / (Hkv / hpb)));
}

struct BalLayout {
    size_t meta, pm, pd, po, total;
};
BalLayout bal_layout(int B, int Hq, int Hkv, int D, int nb) {
    BalLayout w;
    const size_t states = (size_t)Hq * (size_t)(nb + B);
    w.meta = counter_bytes(B, Hkv);
    w.pm = align_up(w.meta + (size_t)B * 2 * sizeof(int32_t));
    w.pd = align_up(w.pm + states * sizeof(float));
    w.po = align_up(w.pd + states * sizeof(float));
    w.total = align_up(w.po + states * D * sizeof(float));
    return w;
}

extern "C" size_t fdec_balanced_workspace_size(int B, int Hq, int Hkv, int head_dim, int num_blocks) {
    if (B < 0 || Hq < 1 || Hkv < 1 || head_dim < 1 || num_blocks < 0 || num_blocks > FDEC_MAX_SPLITS) return 0;
    // the default of either cache format fits (the float8 one is the larger)
    return bal_layout(B, Hq, Hkv, head_dim, balanced_blocks(Hkv, num_blocks, 2)).total;
}

// The balanced split for q_len query tokens per request (1: fdec_decode_balanced).
int decode_balanced_impl(const char *fn, const void *q, int B, int q_len, int Hq, const fdec_kv *kv,
                         const int32_t *seq_lens, int num_blocks, float softmax_scale, float *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream) {
    if (q_len < 1 || q_len > FDEC_MAX_QLEN)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: q_len %d outside [1, %d]", fn, q_len, FDEC_MAX_QLEN);
    int rc = validate_common(fn, q, B, Hq, kv, seq_lens, softmax_scale);
    if (rc) return rc;
    if (num_blocks < 0 || num_blocks > FDEC_MAX_SPLITS)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: num_blocks %d outside [0, %d]", fn, num_blocks, FDEC_MAX_SPLITS);
    if ((int64_t)B * (((int64_t)capacity_of(kv) + 15) / 16) >= (int64_t(1) << 31))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: B * ceil(capacity / 16) must stay below 2^31", fn);
    fdec::MapParams p = map_params(q, B, Hq, kv, seq_lens, 1, softmax_scale, nullptr);
    const int G = Hq / kv->num_kv_heads;
    // the 16x16x32 kernel: several query tokens, and one query token at G = 1, 2
    // (its 16-row block padded; G = 4 and 8 keep their own single-query kernels)
    const bool mt16 = (q_len > 1 || (G != 4 && G != 8)) && fdec::mt16_eligible(q_len, G, kv->head_dim) &&
                      (kv->page_size == 0 || kv->page_size % 16 == 0) && std::getenv("FDEC_MULTI_PATH") == nullptr;
    if (!mt16 && !(p.mfma && (G == 4 || (G == 8 && q_len == 1))))
        return fdec_fail(FDEC_ERR_UNSUPPORTED, "%s: needs head_dim 128 and page_size a multiple of 16", fn);
    if (B == 0) return FDEC_OK;
    if (!out) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if ((reinterpret_cast<uintptr_t>(out) & 7u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: out must be 8-byte and lse 4-byte aligned", fn);
    const int ql = fdec::mfma_tokens_per_wave(q_len);
    p.q_len = q_len;
    p.q_groups = (q_len + ql - 1) / ql;
    // float8 caches run two blocks per compute unit; with several query tokens the
    // Q slots take the LDS the second block would need. The 16x16x32 kernel: one
    // block per compute unit over its blocks along z, within the block count the
    // workspace size provides for
    int nb = balanced_blocks(kv->num_kv_heads, num_blocks, kv->dtype == FDEC_FP8_E4M3 && ql == 1 ? 2 : 1);
    if (mt16 && num_blocks == 0)
        nb = std::min(balanced_blocks(kv->num_kv_heads, 0, 2),
                      std::max(1, device_cus() / fdec::mt16_z_blocks(q_len, G, kv->num_kv_heads)));
    const BalLayout w = bal_layout(B, q_len * Hq, kv->num_kv_heads, kv->head_dim, nb);
    if (!workspace || workspace_bytes < w.total)
        return fdec_fail(FDEC_ERR_WORKSPACE, "%s: workspace of %zu bytes needed for %d blocks, got %zu", fn, w.total,
                         nb, workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: workspace not 16-byte aligned", fn);
    char *ws = static_cast<char *>(workspace);
    p.seg_meta = reinterpret_cast<int *>(ws + w.meta);
    p.pm = reinterpret_cast<float *>(ws + w.pm);
    p.pd = reinterpret_cast<float *>(ws + w.pd);
    p.po = reinterpret_cast<float *>(ws + w.po);
    p.nslots = nb + B;
    if ((rc = fdec_debug_gate(fn, B, kv, seq_lens, nullptr, nullptr, 0, stream))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    Launches run(st);
    if ((rc = run.done(mt16 ? fdec::launch_map_mt16_balanced(p, nb, st) : fdec::launch_map_mfma_g4_balanced(p, nb, st),
                       "balanced split: map launch")))
        return rc;
    return run.done(fdec::launch_merge_segments(p.po, p.pm, p.pd, p.seg_meta, B, Hq, p.nslots, nb, kv->head_dim, out,
                                                 lse, st, q_len),
                     "balanced split: merge launch");
}

extern "C" int fdec_decode_balanced(const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *seq_lens,
                                    int num_blocks, float softmax_scale, float *out, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    fdec_clear_error();
    return decode_balanced_impl("fdec_decode_balanced", q, B, 1, Hq, kv, seq_lens, num_blocks, softmax_scale, out, lse,
                                workspace, workspace_bytes, stream);
}

extern "C" int fdec_decode_multi_balanced(const void *q, int B, int q_len, int Hq, const fdec_kv *kv,
                                          const int32_t *seq_lens, int num_blocks, float softmax_scale, float *out,
                                          float *lse, void *workspace, size_t workspace_bytes, void *stream) {
    fdec_clear_error();
    return decode_balanced_impl("fdec_decode_multi_balanced", q, B, q_len, Hq, kv, seq_lens, num_blocks,
                                softmax_scale, out, lse, workspace, workspace_bytes, stream);
}

extern "C" int fdec_merge_states(const float *part_o, const float *part_m, const float *part_d, int B, int Hq,
                                 int S, int head_dim, float *out, float *lse, void *stream) {
    fdec_clear_error();
    const char *fn = "fdec_merge_states";
    if (B < 0 || Hq < 1) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: need B >= 0 and Hq >= 1", fn);
    if (S < 1 || S > FDEC_MAX_SPLITS)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: S = %d outside [1, %d]", fn, S, FDEC_MAX_SPLITS);
    if (head_dim != 128 && head_dim != 64)
        return fdec_fail(FDEC_ERR_UNSUPPORTED, "%s: head_dim %d not built (128, 64)", fn, head_dim);
    if (B == 0) return FDEC_OK;
    if (!part_o || !part_m || !part_d || !out)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: part_o, part_m, part_d and out must be non-NULL", fn);
    if ((reinterpret_cast<uintptr_t>(part_o) & 7u) || (reinterpret_cast<uintptr_t>(out) & 7u))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: part_o and out must be 8-byte aligned", fn);
    Launches run(static_cast<hipStream_t>(stream));
    return run.done(fdec::launch_merge(part_o, part_m, part_d, B, Hq, S, head_dim, out, lse,
                                       static_cast<hipStream_t>(stream)),
                    fn);
}

// The cascade's suffixes run on the balanced split when the matrix-core map
// kernel takes the shape (G = 4, head_dim 128): workspace = meta [B, 2], the
// prefix states [B, Hq, sp] and the suffix pieces [Hq, ss + B].
bool cascade_balanced_shape(int Hq, int Hkv, int D) { return Hq == 4 * Hkv && D == 128; }
// The single-launch cascade needs suffix blocks of four KV heads (Hkv a multiple
// of 4); FDEC_CASCADE_PATH=two keeps the prefix and suffix kernels apart.
bool cascade_single_launch(const fdec::MapParams &pb) {
    const char *path = std::getenv("FDEC_CASCADE_PATH");
    return pb.heads_per_block == fdec::kMapMfmaWaves && !(path && std::strcmp(path, "two") == 0);
}

struct CascBalLayout {
    size_t meta, ppm, ppd, ppo, pm, pd, po, total;
};
CascBalLayout casc_bal_layout(int B, int Hq, int Hkv, int D, int sp, int ss) {
    CascBalLayout w;
    const size_t pstates = (size_t)B * Hq * sp, sstates = (size_t)Hq * (size_t)(ss + B);
    w.meta = counter_bytes(B, Hkv);
    w.ppm = align_up(w.meta + (size_t)B * 2 * sizeof(int32_t));
    w.ppd = align_up(w.ppm + pstates * sizeof(float));
    w.ppo = align_up(w.ppd + pstates * sizeof(float));
    w.pm = align_up(w.ppo + pstates * D * sizeof(float));
    w.pd = align_up(w.pm + sstates * sizeof(float));
    w.po = align_up(w.pd + sstates * sizeof(float));
    w.total = align_up(w.po + sstates * D * sizeof(float));
    return w;
}

extern "C" size_t fdec_cascade_workspace_size(int B, int Hq, int Hkv, int head_dim, int splits_prefix,
                                              int splits_suffix) {
    if (splits_prefix < 1 || splits_suffix < 1 || B < 0 || Hq < 1 || Hkv < 1) return 0;
    size_t n = fdec_workspace_size(B, Hq, Hkv, head_dim, splits_prefix + splits_suffix);
    if (cascade_balanced_shape(Hq, Hkv, head_dim))
        n = std::max(n, casc_bal_layout(B, Hq, Hkv, head_dim, splits_prefix, splits_suffix).total);
    return n;
}

extern "C" int fdec_cascade_plan(int B, int Hq, int Hkv, int prefix_len, int capacity, int page_size,
                                 int cu_count, int *splits_prefix_out, int *splits_suffix_out) {
    return fdec_cascade_plan_kv(B, Hq, Hkv, prefix_len, capacity, page_size, FDEC_BF16, cu_count, splits_prefix_out,
                                splits_suffix_out);
}

extern "C" int fdec_cascade_plan_kv(int B, int Hq, int Hkv, int prefix_len, int capacity, int page_size,
                                    int kv_dtype, int cu_count, int *splits_prefix_out, int *splits_suffix_out) {
    fdec_clear_error();
    const char *fn = "fdec_cascade_plan";
    if (!splits_prefix_out || !splits_suffix_out)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: output pointers must be non-NULL", fn);
    if (kv_dtype != FDEC_F16 && kv_dtype != FDEC_BF16 && kv_dtype != FDEC_FP8_E4M3)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: kv_dtype %d is not an fdec_dtype", fn, kv_dtype);
    if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || prefix_len < 0 || capacity < 1 || page_size < 16 ||
        page_size % 16)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: bad sizes", fn);
    if (cu_count <= 0) cu_count = 256;
    // the single-launch cascade (G = 4, Hkv a multiple of 4) runs 128-row prefix
    // blocks beside one suffix block per compute unit; otherwise the prefix
    // kernel's 256-row blocks take the whole GPU first
    const char *path = std::getenv("FDEC_CASCADE_PATH");
    const bool single = Hq == 4 * Hkv && Hkv % fdec::kMapMfmaWaves == 0 && !(path && std::strcmp(path, "two") == 0);
    const int rows = B * (Hq / Hkv);
    const int chunk_rows = single ? fdec::kMapMfmaWaves * 32 : 256;
    const int row_chunks = rows > 0 ? (rows + chunk_rows - 1) / chunk_rows : 1;
    int sp = (cu_count + Hkv * row_chunks - 1) / (Hkv * row_chunks);
    if (single) {
        // at most one prefix block per compute unit (more start only when others
        // end); with 16-bit pools three quarters of the units measured faster
        // (the shared-prefix workload: 70 us at 192 prefix blocks against 76 at
        // 256), with float8 pools all of them (61 against 68)
        const int target = kv_dtype == FDEC_FP8_E4M3 ? cu_count : (3 * cu_count) / 4;
        sp = std::max(1, target / (Hkv * row_chunks));
    }
    sp = std::min(sp, std::max(1, prefix_len / 256));
    sp = std::max(1, std::min(sp, FDEC_MAX_SPLITS / 2));
    // each prefix block stages at most kPrefixPagesPerBlock - 2 page ids
    while (sp < FDEC_MAX_SPLITS / 2) {
        const int64_t chunk = cascade_chunk(prefix_len, sp);
        if (chunk / page_size + 2 <= fdec::kPrefixPagesPerBlock) break;
        ++sp;
    }
    int ss = 1;
    if (Hq == 4 * Hkv) {
        // balanced suffix (head_dim 128): one block per compute unit over all groups of KV heads
        int hpb = 1;
        for (int w = fdec::kMapMfmaWaves; w > 1; --w)
            if (Hkv % w == 0) {
                hpb = w;
                break;
            }
        // float8 pools on the separate suffix kernel: two blocks per compute unit
        // (half the bytes per tile, so more tiles in flight per compute unit), as far
        // as the merge's 256 states allow; the single launch keeps one per unit
        ss = std::max(1, cu_count / (Hkv / hpb)) * (kv_dtype == FDEC_FP8_E4M3 && !single ? 2 : 1);
    } else {
        int rc = fdec_plan_kv(B, Hq, Hkv, nullptr, capacity, page_size, kv_dtype, cu_count, &ss);
        if (rc) return rc;
    }
    ss = std::max(1, std::min(ss, FDEC_MAX_SPLITS - sp));
    *splits_prefix_out = sp;
    *splits_suffix_out = ss;
    return FDEC_OK;
}

extern "C" int fdec_cascade_decode(const void *q, int B, int Hq, const fdec_kv *kv, const int32_t *prefix_pages,
                                   int prefix_len, const int32_t *suffix_lens, int splits_prefix,
                                   int splits_suffix, float softmax_scale, float *out, float *lse,
                                   void *workspace, size_t workspace_bytes, void *stream) {
    fdec_clear_error();
    const char *fn = "fdec_cascade_decode";
    int rc = validate_common(fn, q, B, Hq, kv, suffix_lens, softmax_scale);
    if (rc) return rc;
    if (kv->page_size == 0) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: the cascade path needs a paged cache", fn);
    if (kv->cache_leftpad)
        return fdec_fail(FDEC_ERR_UNSUPPORTED, "%s: cache_leftpad is not supported with a shared prefix", fn);
    if (kv->head_dim != 128)
        return fdec_fail(FDEC_ERR_UNSUPPORTED, "%s: head_dim %d not built for the cascade path (128)", fn,
                         kv->head_dim);
    if (prefix_len < 0) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: prefix_len < 0", fn);
    if (prefix_len > 0 && !prefix_pages)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: prefix_pages is NULL with prefix_len > 0", fn);
    if (splits_prefix < 0 || splits_suffix < 0 || splits_prefix + splits_suffix > FDEC_MAX_SPLITS)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: split counts must be >= 0 with a sum <= %d", fn, FDEC_MAX_SPLITS);
    const int cap = capacity_of(kv);
    int sp = splits_prefix, ss = splits_suffix;
    if (sp == 0 || ss == 0) {
        int psp = 1, pss = 1;
        if ((rc = fdec_cascade_plan_kv(B, Hq, kv->num_kv_heads, prefix_len, cap, kv->page_size, kv->dtype, 256, &psp,
                                       &pss)))
            return rc;
        // a planned count fits beside a count the caller gave
        if (sp == 0) sp = ss ? std::max(1, std::min(psp, FDEC_MAX_SPLITS - ss)) : psp;
        if (ss == 0) ss = std::max(1, std::min(pss, FDEC_MAX_SPLITS - sp));
        if (sp + ss > FDEC_MAX_SPLITS) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: too many splits", fn);
    }
    const int64_t chunk_p = cascade_chunk(prefix_len, sp);
    if (chunk_p / kv->page_size + 2 > fdec::kPrefixPagesPerBlock)
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: %lld prefix tokens per split span too many pages; use more splits",
                         fn, (long long)chunk_p);
    if (B == 0) return FDEC_OK;
    if (!out) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if ((reinterpret_cast<uintptr_t>(out) & 7u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: out must be 8-byte and lse 4-byte aligned", fn);
    if ((rc = fdec_debug_gate(fn, B, kv, suffix_lens, nullptr, prefix_pages, prefix_len, stream))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    float scale = softmax_scale == 0.0f ? 1.0f / std::sqrt((float)kv->head_dim) : softmax_scale;
    fdec::CascadeParams cp;
    std::memset(&cp, 0, sizeof(cp));
    cp.q = q;
    cp.k = kv->k;
    cp.v = kv->v;
    cp.s_outer = kv->s_outer;
    cp.s_token = kv->s_token;
    cp.s_head = kv->s_head;
    cp.prefix_pages = prefix_pages;
    cp.prefix_len = prefix_len;
    cp.page_size = kv->page_size;
    cp.page_shift = page_shift_of(kv->page_size);
    cp.B = B;
    cp.Hq = Hq;
    cp.Hkv = kv->num_kv_heads;
    cp.chunk = (int)chunk_p;
    cp.scale_log2 = scale * 1.4426950408889634f;
    cp.kv_fp8 = kv->dtype == FDEC_FP8_E4M3;
    cp.dtype = cp.kv_fp8 ? FDEC_BF16 : kv->dtype;  // the queries' type
    cp.k_descale = cp.kv_fp8 ? kv->k_descale : nullptr;
    cp.v_descale = cp.kv_fp8 ? kv->v_descale : nullptr;

    fdec::MapParams pb = map_params(q, B, Hq, kv, suffix_lens, 1, softmax_scale, nullptr);
    if (pb.mfma && cascade_balanced_shape(Hq, kv->num_kv_heads, kv->head_dim) &&
        (int64_t)B * (((int64_t)cap + 15) / 16) < (int64_t(1) << 31)) {
        // suffixes on the balanced split, then one merge of prefix states and suffix pieces
        const CascBalLayout w = casc_bal_layout(B, Hq, kv->num_kv_heads, kv->head_dim, sp, ss);
        if (!workspace || workspace_bytes < w.total)
            return fdec_fail(FDEC_ERR_WORKSPACE, "%s: workspace of %zu bytes needed for %d + %d splits, got %zu", fn,
                             w.total, sp, ss, workspace ? workspace_bytes : (size_t)0);
        if (!aligned16(workspace))
            return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: workspace not 16-byte aligned", fn);
        char *ws = static_cast<char *>(workspace);
        cp.pm = reinterpret_cast<float *>(ws + w.ppm);
        cp.pd = reinterpret_cast<float *>(ws + w.ppd);
        cp.po = reinterpret_cast<float *>(ws + w.ppo);
        cp.s_total = sp;
        cp.s_offset = 0;
        pb.seg_meta = reinterpret_cast<int *>(ws + w.meta);
        pb.pm = reinterpret_cast<float *>(ws + w.pm);
        pb.pd = reinterpret_cast<float *>(ws + w.pd);
        pb.po = reinterpret_cast<float *>(ws + w.po);
        pb.nslots = ss + B;
        Launches run(st);
        if (cascade_single_launch(pb)) {
            // prefix and suffix blocks share the compute units (one launch)
            if ((rc = run.done(fdec::launch_cascade_fused(cp, pb, sp, ss, st),
                               "fdec_cascade_decode: prefix and suffix launch")))
                return rc;
        } else {
            if ((rc = run.done(fdec::launch_cascade_prefix(cp, sp, st), "fdec_cascade_decode: prefix launch")))
                return rc;
            if ((rc = run.done(fdec::launch_map_mfma_g4_balanced(pb, ss, st), "fdec_cascade_decode: suffix launch")))
                return rc;
        }
        return run.done(fdec::launch_merge_cascade(cp.po, cp.pm, cp.pd, sp, pb.po, pb.pm, pb.pd, pb.seg_meta, B, Hq,
                                                    pb.nslots, ss, out, lse, st),
                         "fdec_cascade_decode: merge launch");
    }

    const int S = sp + ss;
    const WsLayout w = ws_layout(B, Hq, kv->num_kv_heads, kv->head_dim, S);
    if (!workspace || workspace_bytes < w.total)
        return fdec_fail(FDEC_ERR_WORKSPACE, "%s: workspace of %zu bytes needed for %d + %d splits, got %zu", fn,
                         w.total, sp, ss, workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fdec_fail(FDEC_ERR_INVALID_ARG, "%s: workspace not 16-byte aligned", fn);
    char *ws = static_cast<char *>(workspace);
    float *pm = reinterpret_cast<float *>(ws + w.pm);
    float *pd = reinterpret_cast<float *>(ws + w.pd);
    float *po = reinterpret_cast<float *>(ws + w.po);
    cp.po = po;
    cp.pm = pm;
    cp.pd = pd;
    cp.s_total = S;
    cp.s_offset = 0;
    Launches run(st);
    if ((rc = run.done(fdec::launch_cascade_prefix(cp, sp, st), "fdec_cascade_decode: prefix launch"))) return rc;

    fdec::MapParams p = map_params(q, B, Hq, kv, suffix_lens, ss, softmax_scale, nullptr);
    p.po = po;
    p.pm = pm;
    p.pd = pd;
    p.s_total = S;
    p.s_offset = sp;
    if ((rc = run.done(fdec::launch_map(p, ss, st), "fdec_cascade_decode: suffix launch"))) return rc;
    return run.done(fdec::launch_merge(po, pm, pd, B, Hq, S, kv->head_dim, out, lse, st),
                     "fdec_cascade_decode: merge launch");
}

extern "C" int fdec_trace_start(int max_events) {
    fdec_clear_error();
    if (max_events < 2 || max_events > (1 << 20))
        return fdec_fail(FDEC_ERR_INVALID_ARG, "fdec_trace_start: max_events %d outside [2, 2^20]", max_events);
    Trace &t = g_trace;
    for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
    t.ev.clear();
    t.kind.clear();
    t.cap = max_events;
    t.on = true;
    return FDEC_OK;
}

extern "C" int fdec_trace_stop(float *intervals_ms, int *kinds, int capacity, int *count_out) {
    fdec_clear_error();
    Trace &t = g_trace;
    t.on = false;
    const int n = (int)t.ev.size();
    int rc = FDEC_OK;
    if (n > 0) rc = check_hip(hipEventSynchronize(t.ev.back()), "fdec_trace_stop");
    for (int i = 1; rc == FDEC_OK && i < n && i - 1 < capacity; ++i) {
        float ms = 0.0f;
        rc = check_hip(hipEventElapsedTime(&ms, t.ev[i - 1], t.ev[i]), "fdec_trace_stop");
        if (intervals_ms) intervals_ms[i - 1] = ms;
        if (kinds) kinds[i - 1] = t.kind[i];
    }
    for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
    t.ev.clear();
    t.kind.clear();
    if (count_out) *count_out = n;
    return rc;
}
