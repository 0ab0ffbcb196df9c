/*
 * Plain fp64 CPU oracle for single-query decode attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may link, load or call
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code, header, table or helper with the HIP library.
 *
 * Pages cited (extracted web text on FlashDecoding):
 *   [tbr8]     "FlashDecoding 与 FlashInfer 深度解析：大模型推理 Decode 阶段 Attention
 *              并行加速从原理到实战" (tbr8.org)
 *   [lpnh]     lpnh.cn/news/1601758, the FlashDecoding explainer (sections 1-5)
 *   [cookbook] "Inference Cookbook / 推理优化" (inference.lei6393.com, flash-attn docs)
 *
 * What each function follows:
 *   oracle_decode    the plain definition softmax(scale * q K^T) V for one query
 *                    token, with lse = ln sum_j exp(s_j)  ([tbr8] §2.1 step 2;
 *                    [lpnh] §1; [cookbook] §3.5 for the LSE output). No splitting,
 *                    no blocking: the method is exact, so the oracle is the
 *                    definition ([tbr8] §2.1, last paragraph).
 *   oracle_partials  the map stage: per split i the local max m_i, the local sum of
 *                    exponentials d_i and the UNNORMALISED output O~_i
 *                    ([lpnh] §2 stage 1; [tbr8] §2.1 step 2).
 *   oracle_merge     the reduce stage: m = max m_i, alpha_i = exp(m_i - m),
 *                    d = sum alpha_i d_i, O = sum alpha_i O~_i / d
 *                    ([lpnh] §2 stage 2; [tbr8] §2.1 step 3).
 *   oracle_rope_neox GPT-NeoX (non-interleaved) rotary embedding, base^(-2i/rd)
 *                    angles, in double ([cookbook] §3.4).
 *   oracle_append    writes rope(k_new) and v_new at row cache_seqlens[b] and
 *                    returns rope(q); lengths are not advanced
 *                    ([cookbook] §3.2-3.4). A float8 cache stores each new
 *                    element as the e4m3fn code of (value / descale)
 *                    ([cookbook] §7.1-7.2: value = code * descale).
 *   oracle_f32_to_f8 the e4m3fn code nearest a binary32 value: a search over
 *                    every finite code, ties to the even code ([cookbook] §7.1,
 *                    the cast to float8_e4m3fn).
 *   fp8 cache        K/V stored as float8_e4m3fn with one fp32 descale per
 *                    (request, KV head) for K and one for V; the element's value
 *                    is its e4m3 value times that descale ([cookbook] §7.1-7.2).
 *   paging           logical token j of request b lives in page
 *                    page_table[b][j / ps], slot j % ps; entries past the
 *                    request's pages are -1 and are never read ([cookbook] §4.2).
 *   cache_batch_idx  request b reads (and appends to) row batch_idx[b] of a
 *                    contiguous cache ([cookbook] §5.2).
 *   cache_leftpad    request b's valid rows start at leftpad[b]: it attends
 *                    to rows [leftpad[b], L_b) ([cookbook] §5.3).
 *   oracle_decode_multi  q_len query tokens per request (speculative decode,
 *                    [vllm-arch] spec-decode batches; softmax_lse of shape
 *                    (batch, heads, seqlen_q), [cookbook] §3.5) under the causal
 *                    mask the calls pass: token i is the request's row
 *                    L_b - q_len + i and attends to rows [leftpad[b], L_b - q_len + i].
 *
 * Readings where the pages are silent (all listed in the design notes):
 *   - empty range: out = 0, lse = -inf; an empty split is (O~=0, m=-inf, d=0)
 *     and contributes alpha = 0;
 *   - query head h reads KV head h / (Hq/Hkv) (consecutive GQA groups);
 *   - lse is the natural log of the sum of exp of the SCALED scores;
 *   - the rotated k row is rounded once (round to nearest even) to the cache
 *     dtype; q stays in double; v is copied unchanged;
 *   - cascade: request b's tokens are the shared prefix (prefix_pages) followed
 *     by its own suffix pages (page_table row b);
 *   - lengths (lens / cache_seqlens) count rows from row 0, left padding
 *     included; an appended row goes to row cache_seqlens[b] and is rotated at
 *     its position among the valid rows, cache_seqlens[b] - leftpad[b];
 *   - float8 descales are indexed by the query's request b;
 *   - float8 append: (value / descale) is formed in binary32 (the rotated k
 *     value rounded once to binary32 first) and rounded to the nearest e4m3fn
 *     code, ties to even; magnitudes beyond the largest finite 448 saturate to
 *     +-448 (the cache stays finite), NaN gives the NaN code 0x7f.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <time.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------- element decoding / encoding, from the IEEE-754 field layouts ---------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16 is the upper half of an IEEE binary32. */
double oracle_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* float8 e4m3fn (OCP): 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits;
 * no infinities, S.1111.111 is NaN, the largest finite is 448. */
double oracle_f8_to_f64(uint8_t x) {
    int s = x >> 7, e = (x >> 3) & 15, m = x & 7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9); /* subnormal: (m / 8) * 2^(1-7) */
    else
        v = ldexp((double)(m + 8), e - 10); /* (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

void oracle_decode_f8(const uint8_t *src, int64_t n, double *dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_f8_to_f64(src[i]);
}

/* The e4m3fn code nearest x: every finite magnitude code 0x00..0x7e is tried;
 * on a tie the even code (even last fraction bit) wins. Past 448 the nearest
 * finite code is 0x7e, so large magnitudes saturate. The sign bit is x's. */
uint8_t oracle_f32_to_f8(float x) {
    if (isnan(x)) return 0x7f;
    double a = fabs((double)x);
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7e; ++c) {
        double err = fabs(oracle_f8_to_f64((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0)) {
            best = c;
            best_err = err;
        }
    }
    return (uint8_t)(signbit(x) ? (best | 0x80) : best);
}

void oracle_encode_f8(const float *src, int64_t n, uint8_t *dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = oracle_f32_to_f8(src[i]);
}

/* Round a double once, to nearest with ties to even, onto a binary16. */
uint16_t oracle_f64_to_f16(double x) {
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x)) return 0x7e00;
    double a = fabs(x);
    if (a >= 65520.0) return sign | 0x7c00; /* rounds past the largest finite 65504 */
    double ulp;
    if (a < ldexp(1.0, -14)) {
        ulp = ldexp(1.0, -24);
    } else {
        int e;
        frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
        ulp = ldexp(1.0, e - 11);
    }
    double v = rint(a / ulp) * ulp; /* rint: current mode, round-half-even */
    if (v < ldexp(1.0, -14)) {
        /* subnormal (a field value of 1024 is exactly the smallest normal) */
        return sign | (uint16_t)(v / ldexp(1.0, -24));
    }
    int E;
    double f = frexp(v, &E);
    uint16_t exp_field = (uint16_t)(E - 1 + 15);
    uint16_t frac = (uint16_t)((f * 2.0 - 1.0) * 1024.0);
    return sign | (uint16_t)(exp_field << 10) | frac;
}

/* Round a double once, to nearest with ties to even, onto a bfloat16. */
uint16_t oracle_f64_to_bf16(double x) {
    if (isnan(x)) return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    /* largest finite is (2 - 2^-7) * 2^127; the halfway point to 2^128 overflows */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return sign | 0x7f80;
    double ulp;
    if (a < ldexp(1.0, -126)) {
        ulp = ldexp(1.0, -133);
    } else {
        int e;
        frexp(a, &e);
        ulp = ldexp(1.0, e - 8);
    }
    double v = rint(a / ulp) * ulp; /* exactly representable in binary32 */
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return sign | (uint16_t)(u >> 16);
}

void oracle_decode_elems(const uint16_t *src, int dtype, int64_t n, double *dst) {
    for (int64_t i = 0; i < n; ++i)
        dst[i] = dtype == 0 ? oracle_f16_to_f64(src[i]) : oracle_bf16_to_f64(src[i]);
}

void oracle_encode_elems(const double *src, int dtype, int64_t n, uint16_t *dst) {
    for (int64_t i = 0; i < n; ++i)
        dst[i] = dtype == 0 ? oracle_f64_to_f16(src[i]) : oracle_f64_to_bf16(src[i]);
}

/* ---------- the KV cache as the oracle sees it ---------- */

typedef struct {
    int B, Hq, Hkv, D;
    int dtype;             /* 0 = fp16, 1 = bf16, 2 = float8 e4m3fn */
    const void *k, *v;     /* raw element bits (2 bytes, or 1 for float8) */
    int page_size;         /* 0 = contiguous [B, capacity, Hkv, D] (by strides) */
    int capacity;          /* contiguous: rows per request */
    int64_t s_outer, s_token, s_head; /* element strides of (batch-or-page, token, head) */
    const int32_t *page_table;        /* [B, max_pages] */
    int max_pages;
    const int32_t *prefix_pages; /* cascade: shared prefix pages, or NULL */
    int prefix_len;              /* cascade: shared prefix tokens */
    const double *k_descale, *v_descale; /* float8: [B, Hkv] factors, or NULL for 1 */
    const int32_t *batch_idx; /* contiguous: cache row of request b, or NULL for b */
    const int32_t *leftpad;   /* first valid row of request b, or NULL for 0 */
} oracle_kv;

static int first_row(const oracle_kv *kv, int b) { return kv->leftpad ? kv->leftpad[b] : 0; }

/* Element offset of logical token j of request b for KV head g. */
static int64_t row_offset(const oracle_kv *kv, int b, int j, int g) {
    int64_t outer, slot;
    if (kv->page_size == 0) {
        outer = kv->batch_idx ? kv->batch_idx[b] : b;
        slot = j;
    } else if (kv->prefix_pages && j < kv->prefix_len) {
        outer = kv->prefix_pages[j / kv->page_size];
        slot = j % kv->page_size;
    } else {
        int jj = kv->prefix_pages ? j - kv->prefix_len : j;
        outer = kv->page_table[(int64_t)b * kv->max_pages + jj / kv->page_size];
        slot = jj % kv->page_size;
    }
    return outer * kv->s_outer + slot * kv->s_token + (int64_t)g * kv->s_head;
}

/* Value of one K or V element of request b, KV head g (descale applied for float8). */
static double elem(const oracle_kv *kv, const void *base, const double *descale, int b, int g, int64_t off) {
    if (kv->dtype == 2) {
        double f = descale ? descale[(int64_t)b * kv->Hkv + g] : 1.0;
        return oracle_f8_to_f64(((const uint8_t *)base)[off]) * f;
    }
    uint16_t u = ((const uint16_t *)base)[off];
    return kv->dtype == 0 ? oracle_f16_to_f64(u) : oracle_bf16_to_f64(u);
}

/* Score of token j for query vector q (already in double) against KV head g. */
static double score(const oracle_kv *kv, const double *q, int b, int j, int g, double scale) {
    int64_t off = row_offset(kv, b, j, g);
    double s = 0.0;
    for (int d = 0; d < kv->D; ++d) s += q[d] * elem(kv, kv->k, kv->k_descale, b, g, off + d);
    return scale * s;
}

/*
 * Attention of each (b, h) over tokens [lo, hi): writes the local max, the
 * local sum of exp(s_j - max) and the unnormalised sum of exp(s_j - max) V_j.
 * An empty range gives (0, -inf, 0).
 */
static void attend_range(const oracle_kv *kv, const double *q, int b, int h, int lo, int hi,
                         double scale, double *sbuf, double *o_tilde, double *m_out,
                         double *d_out) {
    int G = kv->Hq / kv->Hkv, g = h / G, D = kv->D;
    for (int d = 0; d < D; ++d) o_tilde[d] = 0.0;
    if (hi <= lo) {
        *m_out = -INFINITY;
        *d_out = 0.0;
        return;
    }
    double m = -INFINITY;
    for (int j = lo; j < hi; ++j) {
        sbuf[j - lo] = score(kv, q, b, j, g, scale);
        if (sbuf[j - lo] > m) m = sbuf[j - lo];
    }
    double dsum = 0.0;
    for (int j = lo; j < hi; ++j) {
        double p = exp(sbuf[j - lo] - m);
        dsum += p;
        int64_t off = row_offset(kv, b, j, g);
        for (int d = 0; d < D; ++d) o_tilde[d] += p * elem(kv, kv->v, kv->v_descale, b, g, off + d);
    }
    *m_out = m;
    *d_out = dsum;
}

static int max_len(const oracle_kv *kv, const int32_t *lens) {
    int mx = 0;
    for (int b = 0; b < kv->B; ++b) {
        int L = lens[b] + (kv->prefix_pages ? kv->prefix_len : 0);
        if (L > mx) mx = L;
    }
    return mx;
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    return nthreads;
#else
    (void)nthreads;
    return 1;
#endif
}

/*
 * out[b,h,:] = sum_j exp(s_j - m) V_j / sum_j exp(s_j - m),
 * lse[b,h]   = m + ln sum_j exp(s_j - m),
 * s_j = scale * q[b,h,:] . K_j, over the L_b tokens of request b.
 * L_b = lens[b] (cascade: prefix_len + lens[b]). q is [B, Hq, D] doubles.
 */
void oracle_decode(const oracle_kv *kv, const double *q, const int32_t *lens, double scale,
                   double *out, double *lse, int nthreads) {
    int B = kv->B, Hq = kv->Hq, D = kv->D;
    int mx = max_len(kv, lens);
    int nt = set_threads(nthreads);
    (void)nt;
#pragma omp parallel num_threads(nt)
    {
        double *sbuf = (double *)malloc(sizeof(double) * (size_t)(mx > 0 ? mx : 1));
#pragma omp for schedule(dynamic)
        for (int bh = 0; bh < B * Hq; ++bh) {
            int b = bh / Hq, h = bh % Hq;
            int L = lens[b] + (kv->prefix_pages ? kv->prefix_len : 0);
            int lo = first_row(kv, b);
            double m, dsum;
            double *o = out + (int64_t)bh * D;
            attend_range(kv, q + (int64_t)bh * D, b, h, lo, L, scale, sbuf, o, &m, &dsum);
            if (L <= lo) {
                lse[bh] = -INFINITY;
                continue;
            }
            for (int d = 0; d < D; ++d) o[d] /= dsum;
            lse[bh] = m + log(dsum);
        }
        free(sbuf);
    }
}

/*
 * Multi-token decode: q is [B, q_len, Hq, D] doubles; query token i of request
 * b attends to rows [leftpad[b], L_b - q_len + i] (L_b = lens[b], counted from
 * row 0). out [B, q_len, Hq, D]; lse [B, Hq, q_len]. A token with no rows gives
 * out = 0, lse = -inf.
 */
void oracle_decode_multi(const oracle_kv *kv, const double *q, const int32_t *lens, int q_len,
                         double scale, double *out, double *lse, int nthreads) {
    int B = kv->B, Hq = kv->Hq, D = kv->D;
    int mx = max_len(kv, lens);
    int nt = set_threads(nthreads);
    (void)nt;
#pragma omp parallel num_threads(nt)
    {
        double *sbuf = (double *)malloc(sizeof(double) * (size_t)(mx > 0 ? mx : 1));
#pragma omp for schedule(dynamic)
        for (int bih = 0; bih < B * q_len * Hq; ++bih) {
            int b = bih / (q_len * Hq), i = (bih / Hq) % q_len, h = bih % Hq;
            int lo = first_row(kv, b);
            int hi = lens[b] - q_len + i + 1; /* the token's own row is the last it sees */
            double m, dsum;
            double *o = out + (int64_t)bih * D;
            double *l = lse + ((int64_t)b * Hq + h) * q_len + i;
            attend_range(kv, q + (int64_t)bih * D, b, h, lo, hi, scale, sbuf, o, &m, &dsum);
            if (hi <= lo) {
                *l = -INFINITY;
                continue;
            }
            for (int d = 0; d < D; ++d) o[d] /= dsum;
            *l = m + log(dsum);
        }
        free(sbuf);
    }
}

/*
 * Map stage with explicit split boundaries: bounds is [B, S+1]; split i of
 * request b covers tokens [bounds[b][i], bounds[b][i+1]) (clipped to
 * [leftpad[b], L_b)).
 * po [B,Hq,S,D], pm/pd [B,Hq,S].
 */
void oracle_partials(const oracle_kv *kv, const double *q, const int32_t *lens, double scale,
                     int S, const int32_t *bounds, double *po, double *pm, double *pd,
                     int nthreads) {
    int B = kv->B, Hq = kv->Hq, D = kv->D;
    int mx = max_len(kv, lens);
    int nt = set_threads(nthreads);
    (void)nt;
#pragma omp parallel num_threads(nt)
    {
        double *sbuf = (double *)malloc(sizeof(double) * (size_t)(mx > 0 ? mx : 1));
#pragma omp for schedule(dynamic)
        for (int bh = 0; bh < B * Hq; ++bh) {
            int b = bh / Hq, h = bh % Hq;
            int L = lens[b] + (kv->prefix_pages ? kv->prefix_len : 0);
            for (int i = 0; i < S; ++i) {
                int lo = bounds[(int64_t)b * (S + 1) + i];
                int hi = bounds[(int64_t)b * (S + 1) + i + 1];
                if (hi > L) hi = L;
                if (lo < first_row(kv, b)) lo = first_row(kv, b);
                if (lo > hi) lo = hi;
                int64_t si = (int64_t)bh * S + i;
                attend_range(kv, q + (int64_t)bh * D, b, h, lo, hi, scale, sbuf, po + si * D,
                             pm + si, pd + si);
            }
        }
        free(sbuf);
    }
}

/*
 * Reduce stage over S states per (b,h):
 *   m = max_i m_i; alpha_i = exp(m_i - m) (0 when m_i = -inf);
 *   d = sum_i alpha_i d_i; out = sum_i alpha_i O~_i / d; lse = m + ln d.
 * All states empty: out = 0, lse = -inf.
 */
void oracle_merge(const double *po, const double *pm, const double *pd, int B, int Hq, int S,
                  int D, double *out, double *lse) {
    for (int64_t bh = 0; bh < (int64_t)B * Hq; ++bh) {
        double m = -INFINITY;
        for (int i = 0; i < S; ++i)
            if (pm[bh * S + i] > m) m = pm[bh * S + i];
        double *o = out + bh * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (m == -INFINITY) {
            lse[bh] = -INFINITY;
            continue;
        }
        double dsum = 0.0;
        for (int i = 0; i < S; ++i) {
            double mi = pm[bh * S + i];
            double alpha = (mi == -INFINITY) ? 0.0 : exp(mi - m);
            dsum += alpha * pd[bh * S + i];
            for (int d = 0; d < D; ++d) o[d] += alpha * po[(bh * S + i) * D + d];
        }
        for (int d = 0; d < D; ++d) o[d] /= dsum;
        lse[bh] = m + log(dsum);
    }
}

/*
 * GPT-NeoX rotary embedding (non-interleaved): for i < rd/2, the pair
 * (x_i, x_{i+rd/2}) is rotated by the angle pos * base^(-2i/rd); dims >= rd
 * are untouched. In place, in double.
 */
void oracle_rope_neox(double *x, int D, int rotary_dim, int pos, double base) {
    int half = rotary_dim / 2;
    (void)D;
    for (int i = 0; i < half; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)rotary_dim);
        double ang = (double)pos * theta;
        double c = cos(ang), s = sin(ang);
        double a = x[i], b = x[i + half];
        x[i] = a * c - b * s;
        x[i + half] = a * s + b * c;
    }
}

/*
 * KV append with fused rotary, for a contiguous or paged cache. For each
 * request b with c = cache_seqlens[b] and position p = c - leftpad[b]:
 *   k row c of every KV head  <- round_once(rope(k_new[b,g], p))   (rotary_dim > 0)
 *                                or k_new[b,g] bit-copied          (rotary_dim == 0)
 *   v row c of every KV head  <- v_new[b,g] bit-copied
 *   q_out[b,h]                <- rope(q[b,h], p) in double (or q unchanged)
 * k_cache/v_cache are modified in place (the caller passes copies).
 * cache_seqlens is not modified; attention then covers c + 1 tokens.
 */
void oracle_append(oracle_kv *kv, void *k_cache, void *v_cache, const uint16_t *k_new,
                   const uint16_t *v_new, const double *q, const int32_t *cache_seqlens,
                   int rotary_dim, double base, double *q_out) {
    int B = kv->B, Hq = kv->Hq, Hkv = kv->Hkv, D = kv->D;
    const int f8 = kv->dtype == 2;
    /* new rows arrive in the queries' dtype: the cache's own, bf16 for float8 */
    const int new_dtype = f8 ? 1 : kv->dtype;
    double *tmp = (double *)malloc(sizeof(double) * (size_t)D);
    for (int b = 0; b < B; ++b) {
        int c = cache_seqlens[b];
        int pos = c - first_row(kv, b);
        for (int g = 0; g < Hkv; ++g) {
            int64_t off = row_offset(kv, b, c, g);
            const uint16_t *kn = k_new + ((int64_t)b * Hkv + g) * D;
            const uint16_t *vn = v_new + ((int64_t)b * Hkv + g) * D;
            for (int d = 0; d < D; ++d) tmp[d] = new_dtype == 0 ? oracle_f16_to_f64(kn[d]) : oracle_bf16_to_f64(kn[d]);
            if (rotary_dim > 0) oracle_rope_neox(tmp, D, rotary_dim, pos, base);
            if (f8) {
                uint8_t *kc = (uint8_t *)k_cache, *vc = (uint8_t *)v_cache;
                const float kd = kv->k_descale ? (float)kv->k_descale[(int64_t)b * Hkv + g] : 1.0f;
                const float vd = kv->v_descale ? (float)kv->v_descale[(int64_t)b * Hkv + g] : 1.0f;
                for (int d = 0; d < D; ++d) {
                    volatile float x = (float)tmp[d]; /* binary32, then one binary32 division */
                    kc[off + d] = oracle_f32_to_f8(x / kd);
                    volatile float y = (float)oracle_bf16_to_f64(vn[d]);
                    vc[off + d] = oracle_f32_to_f8(y / vd);
                }
            } else {
                uint16_t *kc = (uint16_t *)k_cache, *vc = (uint16_t *)v_cache;
                for (int d = 0; d < D; ++d)
                    kc[off + d] = rotary_dim > 0 ? (kv->dtype == 0 ? oracle_f64_to_f16(tmp[d]) : oracle_f64_to_bf16(tmp[d]))
                                                 : kn[d];
                for (int d = 0; d < D; ++d) vc[off + d] = vn[d];
            }
        }
        for (int h = 0; h < Hq; ++h) {
            const double *qi = q + ((int64_t)b * Hq + h) * D;
            double *qo = q_out + ((int64_t)b * Hq + h) * D;
            for (int d = 0; d < D; ++d) qo[d] = qi[d];
            if (rotary_dim > 0) oracle_rope_neox(qo, D, rotary_dim, pos, base);
        }
    }
    free(tmp);
}

/* Wall-clock seconds, for the CPU-baseline timing. */
double oracle_now(void) {
    struct timespec ts;
    clock_gettime(CLOCK_MONOTONIC, &ts);
    return (double)ts.tv_sec + 1e-9 * (double)ts.tv_nsec;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
