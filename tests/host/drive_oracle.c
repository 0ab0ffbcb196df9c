/*
 * Drives the fp64 oracle (oracle/oracle.c, compiled into this program) over
 * seeded random cases, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py: every buffer is
 * sized exactly, so any read past a cache, page table, length or state array
 * is reported. Along the way it checks identities the oracle must satisfy
 * (each exact up to rounding):
 *   - merging its own partial states at random boundaries gives its decode;
 *   - multi-token decode with one token gives decode;
 *   - decode after an append (16-bit or float8 cache) gives finite outputs
 *     over the cache the append wrote.
 * Exits non-zero on a failed identity; the sanitizers abort on any report.
 */
#include "../../oracle/oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint64_t rnd(void) {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}
static int ri(int lo, int hi) { return lo + (int)(rnd() % (uint64_t)(hi - lo + 1)); } /* [lo, hi] */
static double rn(void) { return ((double)(rnd() >> 11) / 9007199254740992.0) * 4.0 - 2.0; }

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int fail_count = 0;
static void expect_close(const char *what, int c, const double *a, const double *b, int64_t n, double tol) {
    for (int64_t i = 0; i < n; ++i) {
        int both_inf = isinf(a[i]) && isinf(b[i]) && (a[i] < 0) == (b[i] < 0);
        if (!both_inf && !(fabs(a[i] - b[i]) <= tol * (1.0 + fabs(b[i])))) {
            fprintf(stderr, "case %d: %s differs at %lld: %.17g vs %.17g\n", c, what, (long long)i, a[i], b[i]);
            ++fail_count;
            return;
        }
    }
}

static void one_case(int c) {
    int B = ri(1, 4), Hkv = ri(1, 2), G = (int[]){1, 2, 4}[ri(0, 2)], Hq = G * Hkv;
    int D = (int[]){8, 16, 64, 128}[ri(0, 3)];
    int dtype = ri(0, 2), es = dtype == 2 ? 1 : 2;
    int paged = ri(0, 1), ps = paged ? (int[]){16, 32, 64}[ri(0, 2)] : 0;
    int cap = ri(1, 300);
    oracle_kv kv;
    memset(&kv, 0, sizeof kv);
    kv.B = B, kv.Hq = Hq, kv.Hkv = Hkv, kv.D = D, kv.dtype = dtype, kv.page_size = ps;
    int32_t *lens = xmalloc(sizeof(int32_t) * B);
    int32_t *lp = NULL, *bidx = NULL, *table = NULL, *prefix = NULL;
    int64_t elems;
    int rows = B + ri(0, 2), npages = 0, maxp = 0, prefix_len = 0;
    if (!paged) {
        kv.capacity = cap;
        kv.s_token = (int64_t)Hkv * D, kv.s_head = D, kv.s_outer = (int64_t)cap * Hkv * D;
        elems = (int64_t)rows * cap * Hkv * D;
        if (ri(0, 2) == 0) {
            bidx = xmalloc(sizeof(int32_t) * B);
            for (int b = 0; b < B; ++b) bidx[b] = (b + 1) % rows;
            kv.batch_idx = bidx;
        }
    } else {
        maxp = (cap + ps - 1) / ps;
        cap = maxp * ps;
        if (ri(0, 2) == 0) prefix_len = ri(1, 100);
        int prefix_pages = (prefix_len + ps - 1) / ps;
        npages = B * maxp + prefix_pages + ri(0, 3);
        kv.s_token = (int64_t)Hkv * D, kv.s_head = D, kv.s_outer = (int64_t)ps * Hkv * D;
        elems = (int64_t)npages * ps * Hkv * D;
        table = xmalloc(sizeof(int32_t) * B * maxp);
        int32_t *perm = xmalloc(sizeof(int32_t) * npages);
        for (int i = 0; i < npages; ++i) perm[i] = i;
        for (int i = npages - 1; i > 0; --i) {
            int j = ri(0, i), t = perm[i];
            perm[i] = perm[j], perm[j] = t;
        }
        for (int i = 0; i < B * maxp; ++i) table[i] = perm[i];
        if (prefix_len) {
            prefix = xmalloc(sizeof(int32_t) * prefix_pages);
            for (int i = 0; i < prefix_pages; ++i) prefix[i] = perm[B * maxp + i];
            kv.prefix_pages = prefix, kv.prefix_len = prefix_len;
        }
        free(perm);
        kv.page_table = table, kv.max_pages = maxp;
    }
    for (int b = 0; b < B; ++b) lens[b] = ri(0, cap - 1); /* room for one appended row */
    if (ri(0, 2) == 0 && !prefix_len) {
        lp = xmalloc(sizeof(int32_t) * B);
        for (int b = 0; b < B; ++b) lp[b] = ri(0, lens[b]);
        kv.leftpad = lp;
    }
    /* caches: random values encoded to the cache type (float8: random bytes, no NaN codes) */
    void *k = xmalloc((size_t)elems * es), *v = xmalloc((size_t)elems * es);
    double *tmp = xmalloc(sizeof(double) * (size_t)(elems ? elems : 1));
    double *kd = NULL, *vd = NULL;
    if (dtype == 2) {
        for (int64_t i = 0; i < elems; ++i) {
            uint8_t x = (uint8_t)rnd(), y = (uint8_t)rnd();
            ((uint8_t *)k)[i] = (x & 0x7f) == 0x7f ? 0 : x;
            ((uint8_t *)v)[i] = (y & 0x7f) == 0x7f ? 0 : y;
        }
        kd = xmalloc(sizeof(double) * B * Hkv), vd = xmalloc(sizeof(double) * B * Hkv);
        for (int i = 0; i < B * Hkv; ++i) kd[i] = 0.01 + 0.05 * fabs(rn()), vd[i] = 0.01 + 0.05 * fabs(rn());
        kv.k_descale = kd, kv.v_descale = vd;
    } else {
        for (int64_t i = 0; i < elems; ++i) tmp[i] = rn();
        oracle_encode_elems(tmp, dtype, elems, (uint16_t *)k);
        for (int64_t i = 0; i < elems; ++i) tmp[i] = rn();
        oracle_encode_elems(tmp, dtype, elems, (uint16_t *)v);
    }
    kv.k = k, kv.v = v;
    const int64_t nq = (int64_t)B * Hq * D;
    double *q = xmalloc(sizeof(double) * nq), *out = xmalloc(sizeof(double) * nq);
    double *out2 = xmalloc(sizeof(double) * nq), *lse = xmalloc(sizeof(double) * B * Hq);
    double *lse2 = xmalloc(sizeof(double) * B * Hq);
    for (int64_t i = 0; i < nq; ++i) q[i] = rn();
    const double scale = 1.0 / sqrt((double)D);
    oracle_decode(&kv, q, lens, scale, out, lse, 2);

    /* partials at random boundaries (empty and one-token splits included), merged */
    int S = ri(1, 7);
    int32_t *bounds = xmalloc(sizeof(int32_t) * B * (S + 1));
    for (int b = 0; b < B; ++b) {
        int L = lens[b] + prefix_len;
        bounds[b * (S + 1)] = 0;
        for (int i = 1; i < S; ++i) bounds[b * (S + 1) + i] = ri(bounds[b * (S + 1) + i - 1], L);
        bounds[b * (S + 1) + S] = L;
    }
    double *po = xmalloc(sizeof(double) * nq * S), *pm = xmalloc(sizeof(double) * B * Hq * S);
    double *pd = xmalloc(sizeof(double) * B * Hq * S);
    oracle_partials(&kv, q, lens, scale, S, bounds, po, pm, pd, 2);
    oracle_merge(po, pm, pd, B, Hq, S, D, out2, lse2);
    expect_close("merged partials (out)", c, out2, out, nq, 1e-12);
    expect_close("merged partials (lse)", c, lse2, lse, (int64_t)B * Hq, 1e-12);

    /* one query token: decode_multi == decode */
    if (!prefix_len) {
        oracle_decode_multi(&kv, q, lens, 1, scale, out2, lse2, 1);
        expect_close("multi q_len=1 (out)", c, out2, out, nq, 0.0);
        expect_close("multi q_len=1 (lse)", c, lse2, lse, (int64_t)B * Hq, 0.0);
        int ql = ri(1, 4);
        double *qm = xmalloc(sizeof(double) * nq * ql), *om = xmalloc(sizeof(double) * nq * ql);
        double *lm = xmalloc(sizeof(double) * B * Hq * ql);
        for (int64_t i = 0; i < nq * ql; ++i) qm[i] = rn();
        oracle_decode_multi(&kv, qm, lens, ql, scale, om, lm, 2);
        free(qm), free(om), free(lm);
    }

    /* append (new rows in the queries' dtype, bf16 for float8): decode of the
       written cache at length c + 1 */
    if (!prefix_len) {
        void *kc = xmalloc((size_t)elems * es), *vc = xmalloc((size_t)elems * es);
        memcpy(kc, k, (size_t)elems * es), memcpy(vc, v, (size_t)elems * es);
        uint16_t *kn = xmalloc(sizeof(uint16_t) * B * Hkv * D), *vn = xmalloc(sizeof(uint16_t) * B * Hkv * D);
        double *t2 = xmalloc(sizeof(double) * B * Hkv * D);
        const int new_dtype = dtype == 2 ? 1 : dtype;
        for (int i = 0; i < B * Hkv * D; ++i) t2[i] = rn();
        oracle_encode_elems(t2, new_dtype, (int64_t)B * Hkv * D, kn);
        for (int i = 0; i < B * Hkv * D; ++i) t2[i] = rn();
        oracle_encode_elems(t2, new_dtype, (int64_t)B * Hkv * D, vn);
        int rd = (int[]){0, D / 2, D}[ri(0, 2)] & ~1;
        double *qr = xmalloc(sizeof(double) * nq);
        oracle_append(&kv, kc, vc, kn, vn, q, lens, rd, 10000.0, qr);
        int32_t *l1 = xmalloc(sizeof(int32_t) * B);
        for (int b = 0; b < B; ++b) l1[b] = lens[b] + 1;
        oracle_kv after = kv;
        after.k = kc, after.v = vc;
        oracle_decode(&after, qr, l1, scale, out2, lse2, 2);
        for (int64_t i = 0; i < nq; ++i)
            if (!isfinite(out2[i])) {
                fprintf(stderr, "case %d: non-finite output after append\n", c);
                ++fail_count;
                break;
            }
        free(kc), free(vc), free(kn), free(vn), free(t2), free(qr), free(l1);
    }
    free(lens), free(lp), free(bidx), free(table), free(prefix), free(k), free(v), free(tmp), free(kd), free(vd);
    free(q), free(out), free(out2), free(lse), free(lse2), free(bounds), free(po), free(pm), free(pd);
}

int main(int argc, char **argv) {
    int n = argc > 1 ? atoi(argv[1]) : 300;
    /* conversions: every 16-bit pattern round-trips through double */
    for (int u = 0; u < 65536; ++u) {
        double h = oracle_f16_to_f64((uint16_t)u), bf = oracle_bf16_to_f64((uint16_t)u);
        if (!isnan(h) && oracle_f64_to_f16(h) != (uint16_t)u && !(h == 0.0)) ++fail_count;
        if (!isnan(bf) && oracle_f64_to_bf16(bf) != (uint16_t)u && !(bf == 0.0)) ++fail_count;
    }
    for (int c = 0; c < n; ++c) one_case(c);
    if (fail_count) {
        fprintf(stderr, "%d identity failures\n", fail_count);
        return 1;
    }
    printf("oracle sweep ok: %d cases\n", n);
    return 0;
}
