// Host-only stand-ins for the HIP runtime calls and kernel launchers that the
// libfdec host code (api.cpp, plan.cpp) makes, so that code can be built with
// g++ under AddressSanitizer and UndefinedBehaviorSanitizer and driven without
// a GPU (tests/test_host_sanitizers.py).
//
// The driver registers every buffer it passes as a "device" buffer (real host
// memory that nothing dereferences). Each launcher checks, from its parameters,
// that every range the kernel would read or write lies inside one registered
// buffer, and that the ranges a launch writes in a workspace do not overlap
// each other nor a reserved range (the fused path's arrival counters, which
// only a fused launch may use). A violation prints what and where, then aborts.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../decode_attention_fdec_amd/csrc/fdec_host.h"
#include "../../decode_attention_fdec_amd/csrc/fdec_internal.h"

namespace {

struct Region {
    const char *lo, *hi;
    char name[32];
};
Region g_regions[64];
int g_nregions = 0;
Region g_reserved = {nullptr, nullptr, ""};
int g_launches = 0;
char g_last[64] = "";

[[noreturn]] void fail(const char *what, const char *detail) {
    std::fprintf(stderr, "HOST-STUB VIOLATION in %s: %s\n", what, detail);
    std::fflush(stderr);
    std::abort();
}

// [p, p + bytes) lies in one registered buffer
void inside(const char *what, const void *p, size_t bytes) {
    if (bytes == 0) return;
    if (!p) fail(what, "NULL pointer for a non-empty range");
    const char *a = static_cast<const char *>(p);
    for (int i = 0; i < g_nregions; ++i)
        if (a >= g_regions[i].lo && a + bytes <= g_regions[i].hi) return;
    char msg[160];
    std::snprintf(msg, sizeof msg, "range of %zu bytes at %p is outside every registered buffer", bytes, p);
    fail(what, msg);
}

struct Range {
    const void *p;
    size_t n;
    const char *name;
};
bool overlap(const Range &a, const Range &b) {
    if (!a.p || !b.p || !a.n || !b.n) return false;
    const char *x = static_cast<const char *>(a.p), *y = static_cast<const char *>(b.p);
    return x < y + b.n && y < x + a.n;
}
// written ranges of one launch: pairwise disjoint, and off the reserved range
// (except range `counters`, the fused launch's own arrival counters)
void disjoint(const char *what, const Range *r, int n, int counters = -1) {
    for (int i = 0; i < n; ++i) {
        for (int j = i + 1; j < n; ++j)
            if (overlap(r[i], r[j])) {
                char msg[160];
                std::snprintf(msg, sizeof msg, "%s overlaps %s", r[i].name, r[j].name);
                fail(what, msg);
            }
        const Range res = {g_reserved.lo, (size_t)(g_reserved.hi - g_reserved.lo), "reserved counters"};
        if (i != counters && overlap(r[i], res)) {
            char msg[160];
            std::snprintf(msg, sizeof msg, "%s overlaps the reserved arrival counters", r[i].name);
            fail(what, msg);
        }
    }
}

void note(const char *name) {
    ++g_launches;
    std::snprintf(g_last, sizeof g_last, "%s", name);
}

size_t q_bytes(const fdec::MapParams &p) { return (size_t)p.B * p.q_len * p.Hq * p.head_dim * 2; }

// Inputs every map launch reads (K/V extents depend on device data: only non-NULL).
void map_inputs(const char *what, const fdec::MapParams &p) {
    inside(what, p.q, q_bytes(p));
    inside(what, p.seq_lens, (size_t)p.B * 4);
    if (!p.k || !p.v) fail(what, "NULL cache");
    if (p.page_table) inside(what, p.page_table, (size_t)p.B * p.max_pages * 4);
    if (p.batch_idx) inside(what, p.batch_idx, (size_t)p.B * 4);
    if (p.leftpad) inside(what, p.leftpad, (size_t)p.B * 4);
    if (p.k_descale) inside(what, p.k_descale, (size_t)p.B * p.Hkv * 4);
    if (p.v_descale) inside(what, p.v_descale, (size_t)p.B * p.Hkv * 4);
    if (p.mode != fdec::kPlain) {
        inside(what, p.k_new, (size_t)p.B * p.Hkv * p.head_dim * 2);
        inside(what, p.v_new, (size_t)p.B * p.Hkv * p.head_dim * 2);
    }
    if (p.heads_per_block < 1 || p.Hkv % p.heads_per_block) fail(what, "heads_per_block does not divide Hkv");
    if (p.chunk < 16 || p.chunk % 16) fail(what, "chunk not a positive multiple of 16");
}

// Uniform-split states: rows (request, token, head) x s_total slots.
void uniform_states(const char *what, const fdec::MapParams &p, int S) {
    if (p.s_offset < 0 || p.s_offset + S > p.s_total) fail(what, "split slots past s_total");
    const size_t rows = (size_t)p.B * p.q_len * p.Hq, slots = rows * p.s_total;
    inside(what, p.pm, slots * 4);
    inside(what, p.pd, slots * 4);
    inside(what, p.po, slots * p.head_dim * 4);
    Range r[4] = {{p.pm, slots * 4, "m"}, {p.pd, slots * 4, "d"}, {p.po, slots * p.head_dim * 4, "O~"},
                  {p.counters, p.counters ? (size_t)p.B * (p.Hkv / p.heads_per_block) * 4 : 0, "counters"}};
    disjoint(what, r, 4, 3);
    if (p.counters) {
        inside(what, p.out, rows * p.head_dim * 4);
        if (p.lse) inside(what, p.lse, rows * 4);
    }
}

// Balanced-split states: rows (token, head) x nslots; (first slot, count) per request.
void balanced_states(const char *what, const fdec::MapParams &p, int nb) {
    if (p.nslots != nb + p.B) fail(what, "nslots != blocks + B");
    const size_t slots = (size_t)p.q_len * p.Hq * p.nslots;
    inside(what, p.pm, slots * 4);
    inside(what, p.pd, slots * 4);
    inside(what, p.po, slots * p.head_dim * 4);
    inside(what, p.seg_meta, (size_t)p.B * 8);
    Range r[4] = {{p.pm, slots * 4, "m"}, {p.pd, slots * 4, "d"}, {p.po, slots * p.head_dim * 4, "O~"},
                  {p.seg_meta, (size_t)p.B * 8, "segment records"}};
    disjoint(what, r, 4);
}

}  // namespace

extern "C" {
// Driver side: register a buffer, reserve the counter range, read the launch count.
void fdec_stub_region(const void *p, size_t bytes, const char *name) {
    if (g_nregions >= 64) fail("fdec_stub_region", "too many regions");
    Region &r = g_regions[g_nregions++];
    r.lo = static_cast<const char *>(p);
    r.hi = r.lo + bytes;
    std::snprintf(r.name, sizeof r.name, "%s", name ? name : "");
}
void fdec_stub_reset(void) {
    g_nregions = 0;
    g_reserved = {nullptr, nullptr, ""};
}
void fdec_stub_reserve(const void *p, size_t bytes) {
    g_reserved.lo = static_cast<const char *>(p);
    g_reserved.hi = g_reserved.lo + bytes;
}
int fdec_stub_launches(void) { return g_launches; }
const char *fdec_stub_last(void) { return g_last; }

// The HIP runtime calls the host code makes: one device of 256 compute units,
// events that record nothing.
hipError_t hipGetDevice(int *d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *v, hipDeviceAttribute_t a, int) {
    *v = a == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}
const char *hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "stub error"; }
hipError_t hipEventCreate(hipEvent_t *e) {
    *e = reinterpret_cast<hipEvent_t>(std::malloc(8));
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t e) {
    std::free(e);
    return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float *ms, hipEvent_t, hipEvent_t) {
    *ms = 0.0f;
    return hipSuccess;
}
}

namespace fdec {

hipError_t launch_map(const MapParams &p, int S, hipStream_t) {
    note("map");
    if (S < 1) fail("launch_map", "no splits");
    map_inputs("launch_map", p);
    uniform_states("launch_map", p, S);
    if (p.mfma && !map_mfma_eligible(p)) fail("launch_map", "matrix-core kernel on an ineligible shape");
    if (p.mode == kAppendRope) {
        if (!p.rope_cos || !p.rope_sin) fail("launch_map", "rotary without tables");
    }
    return hipSuccess;
}
hipError_t launch_map_mfma_g4(const MapParams &p, int S, hipStream_t st) { return launch_map(p, S, st); }
hipError_t launch_map_mt16(const MapParams &p, int S, hipStream_t) {
    note("map_mt16");
    map_inputs("launch_map_mt16", p);
    uniform_states("launch_map_mt16", p, S);
    if (p.head_dim != 128 || (p.kv_fp8 && p.dtype != 1)) return hipErrorInvalidValue;
    return hipSuccess;
}
hipError_t launch_map_mfma_g4_balanced(const MapParams &p, int nb, hipStream_t) {
    note("map_balanced");
    if (nb < 1 || nb > 256) fail("launch_map_mfma_g4_balanced", "block count outside [1, 256]");
    map_inputs("launch_map_mfma_g4_balanced", p);
    balanced_states("launch_map_mfma_g4_balanced", p, nb);
    return hipSuccess;
}
hipError_t launch_map_mt16_balanced(const MapParams &p, int nb, hipStream_t) {
    note("map_mt16_balanced");
    map_inputs("launch_map_mt16_balanced", p);
    balanced_states("launch_map_mt16_balanced", p, nb);
    if (p.head_dim != 128 || (p.kv_fp8 && p.dtype != 1)) return hipErrorInvalidValue;
    return hipSuccess;
}
void prefix_checks(const char *w, const CascadeParams &p, int splits) {
    inside(w, p.q, (size_t)p.B * p.Hq * 128 * 2);
    if (p.kv_fp8) {  // float8 pools: bf16 queries, descales [B, Hkv] when given
        if (p.dtype != 1) fail(w, "float8 pool without bf16 queries");
        if (p.k_descale) inside(w, p.k_descale, (size_t)p.B * p.Hkv * 4);
        if (p.v_descale) inside(w, p.v_descale, (size_t)p.B * p.Hkv * 4);
    }
    if (p.prefix_len > 0) inside(w, p.prefix_pages, (size_t)((p.prefix_len + p.page_size - 1) / p.page_size) * 4);
    if (p.s_offset < 0 || p.s_offset + splits > p.s_total) fail(w, "prefix slots past s_total");
    if ((int64_t)splits * p.chunk < p.prefix_len) fail(w, "prefix splits do not cover the prefix");
    const size_t slots = (size_t)p.B * p.Hq * p.s_total;
    inside(w, p.pm, slots * 4);
    inside(w, p.pd, slots * 4);
    inside(w, p.po, slots * 128 * 4);
    Range r[3] = {{p.pm, slots * 4, "m"}, {p.pd, slots * 4, "d"}, {p.po, slots * 128 * 4, "O~"}};
    disjoint(w, r, 3);
}
hipError_t launch_cascade_prefix(const CascadeParams &p, int splits, hipStream_t) {
    note("cascade_prefix");
    prefix_checks("launch_cascade_prefix", p, splits);
    return hipSuccess;
}
hipError_t launch_cascade_fused(const CascadeParams &cp, const MapParams &pb, int sp, int ss, hipStream_t) {
    note("cascade_fused");
    const char *w = "launch_cascade_fused";
    if (pb.heads_per_block != 4 || cp.Hq != 4 * cp.Hkv || pb.Hq != cp.Hq || pb.Hkv != cp.Hkv)
        fail(w, "needs G = 4 and four KV heads per suffix block");
    if (!pb.page_table || pb.q_len != 1 || pb.kv_fp8 != cp.kv_fp8) fail(w, "suffix parameters disagree");
    if (ss < 1 || ss > 256) fail(w, "suffix block count outside [1, 256]");
    prefix_checks(w, cp, sp);
    map_inputs(w, pb);
    balanced_states(w, pb, ss);
    return hipSuccess;
}
hipError_t launch_merge(const float *po, const float *pm, const float *pd, int B, int Hq, int S, int D, float *out,
                        float *lse, hipStream_t, int q_len) {
    note("merge");
    const char *w = "launch_merge";
    const size_t rows = (size_t)B * q_len * Hq;
    inside(w, pm, rows * S * 4);
    inside(w, pd, rows * S * 4);
    inside(w, po, rows * S * D * 4);
    inside(w, out, rows * D * 4);
    if (lse) inside(w, lse, rows * 4);
    return hipSuccess;
}
hipError_t launch_merge_segments(const float *po, const float *pm, const float *pd, const int *meta, int B, int Hq,
                                 int nslots, int max_count, int D, float *out, float *lse, hipStream_t, int q_len) {
    note("merge_segments");
    const char *w = "launch_merge_segments";
    const size_t slots = (size_t)q_len * Hq * nslots, rows = (size_t)B * q_len * Hq;
    if (max_count < 1 || max_count > nslots) fail(w, "piece bound outside [1, nslots]");
    inside(w, pm, slots * 4);
    inside(w, pd, slots * 4);
    inside(w, po, slots * D * 4);
    inside(w, meta, (size_t)B * 8);
    inside(w, out, rows * D * 4);
    if (lse) inside(w, lse, rows * 4);
    return hipSuccess;
}
hipError_t launch_merge_cascade(const float *ppo, const float *ppm, const float *ppd, int sp, const float *po,
                                const float *pm, const float *pd, const int *meta, int B, int Hq, int nslots,
                                int max_count, float *out, float *lse, hipStream_t) {
    note("merge_cascade");
    const char *w = "launch_merge_cascade";
    const size_t ps = (size_t)B * Hq * sp, ss = (size_t)Hq * nslots, rows = (size_t)B * Hq;
    inside(w, ppm, ps * 4);
    inside(w, ppd, ps * 4);
    inside(w, ppo, ps * 128 * 4);
    inside(w, pm, ss * 4);
    inside(w, pd, ss * 4);
    inside(w, po, ss * 128 * 4);
    inside(w, meta, (size_t)B * 8);
    inside(w, out, rows * 128 * 4);
    if (lse) inside(w, lse, rows * 4);
    Range r[7] = {{ppm, ps * 4, "prefix m"}, {ppd, ps * 4, "prefix d"}, {ppo, ps * 512, "prefix O~"},
                  {pm, ss * 4, "suffix m"},  {pd, ss * 4, "suffix d"},  {po, ss * 512, "suffix O~"},
                  {meta, (size_t)B * 8, "segment records"}};
    disjoint(w, r, 7);
    (void)max_count;
    return hipSuccess;
}
hipError_t launch_zero_words(void *p, size_t n, hipStream_t) {
    note("zero_words");
    inside("launch_zero_words", p, n * 4);
    return hipSuccess;
}

}  // namespace fdec

// The debug mode's device-data check runs on the GPU (check.hip): off here.
int fdec_debug_gate(const char *, int, const fdec_kv *, const int32_t *, const fdec_append *, const int32_t *, int,
                    void *) {
    return 0;
}
