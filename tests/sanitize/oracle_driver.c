/*
 * Host sanitizer run of the oracle (test infrastructure): every exported
 * function on small seeded inputs, with the edge cases the parity tests use
 * (empty sequences, causal rows that see no key, splits past a sequence's
 * end, head_dim 1, several threads) and with arguments it must reject.
 * tests/test_sanitizers.py builds it with AddressSanitizer and
 * UndefinedBehaviorSanitizer (no recovery) and expects exit status 0.
 * Checks here are structural (finite outputs, -inf LSE for empty rows,
 * rejected arguments); values are pinned by the other oracle tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_paged_attention(int B, int qlen, int hq, int hkv, int d, int page_size, int max_pages,
                           int dtype, const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                           const int32_t *block_table, const int32_t *seqlens, double scale,
                           int causal, int nthreads, double *out, double *lse);
int oracle_dense_attention(int hq, int hkv, int qlen, int kvlen, int d, int dtype,
                           const uint16_t *q, const uint16_t *k, const uint16_t *v, double scale,
                           int causal, int nthreads, double *out, double *lse);
int oracle_paged_split_partials(int B, int qlen, int hq, int hkv, int d, int page_size,
                                int max_pages, int dtype, const uint16_t *q, const uint16_t *kc,
                                const uint16_t *vc, const int32_t *block_table,
                                const int32_t *seqlens, double scale, int causal, int num_splits,
                                int split_keys, int block, int nthreads, double *o_part,
                                double *lse_part);
int oracle_dense_split_partials(int hq, int hkv, int qlen, int kvlen, int d, int dtype,
                                const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                double scale, int causal, int num_splits, int split_keys,
                                int block, int nthreads, double *o_part, double *lse_part);
void oracle_combine(int num_splits, int nrows, int d, const double *o_part,
                    const double *lse_part, double *out, double *lse);
double oracle_decode_scalar(uint16_t x, int dtype);

static uint32_t state = 2463534242u;
static uint32_t next_u32(void) { /* xorshift32 */
    state ^= state << 13;
    state ^= state >> 17;
    state ^= state << 5;
    return state;
}
/* a finite 16-bit value of magnitude about 2^-4 .. 2^1 */
static uint16_t rnd16(int dtype) {
    uint32_t r = next_u32();
    uint16_t sign = (uint16_t)((r & 1u) << 15);
    if (dtype == 0) return sign | (uint16_t)((11u + (r >> 1) % 6u) << 10) | (uint16_t)((r >> 8) & 0x3FFu);
    return sign | (uint16_t)((123u + (r >> 1) % 6u) << 7) | (uint16_t)((r >> 8) & 0x7Fu);
}
static uint16_t *fill16(size_t n, int dtype) {
    uint16_t *p = (uint16_t *)malloc(sizeof(uint16_t) * (n ? n : 1));
    size_t i;
    for (i = 0; i < n; ++i) p[i] = rnd16(dtype);
    return p;
}

static int failures = 0;
#define CHECK(c, msg) do { if (!(c)) { fprintf(stderr, "FAIL: %s (%s:%d)\n", msg, __FILE__, __LINE__); ++failures; } } while (0)

static void check_rows(const double *o, const double *lse, int nrows, int d, const int *visible) {
    int n, e;
    for (n = 0; n < nrows; ++n) {
        if (visible[n] == 0) {
            CHECK(lse[n] == -INFINITY, "empty row LSE");
            for (e = 0; e < d; ++e) CHECK(o[(size_t)n * d + e] == 0.0, "empty row output");
        } else {
            CHECK(isfinite(lse[n]), "LSE finite");
            for (e = 0; e < d; ++e) CHECK(isfinite(o[(size_t)n * d + e]), "output finite");
        }
    }
}

static int visible_of(int L, int qlen, int i, int causal) {
    int v = causal ? L - qlen + 1 + i : L;
    return v < 0 ? 0 : (v > L ? L : v);
}

static void paged_case(int B, int qlen, int hq, int hkv, int d, int page, int dtype, int causal,
                       const int32_t *lens, int nthreads) {
    int b, i, h, maxp = 1, pages = 0, t, s;
    int nrows = B * qlen * hq;
    for (b = 0; b < B; ++b) {
        int np = (lens[b] + page - 1) / page;
        if (np > maxp) maxp = np;
        pages += np;
    }
    pages += 1; /* a spare page for table slots past a sequence's end */
    {
        uint16_t *q = fill16((size_t)nrows * d, dtype);
        uint16_t *kc = fill16((size_t)pages * page * hkv * d, dtype);
        uint16_t *vc = fill16((size_t)pages * page * hkv * d, dtype);
        int32_t *bt = (int32_t *)malloc(sizeof(int32_t) * (size_t)B * maxp);
        double *out = (double *)malloc(sizeof(double) * (size_t)nrows * d);
        double *lse = (double *)malloc(sizeof(double) * (size_t)nrows);
        double *lse_rows = (double *)malloc(sizeof(double) * (size_t)nrows);
        int *vis = (int *)malloc(sizeof(int) * (size_t)nrows);
        int next = 0, maxL = 0;
        for (b = 0; b < B; ++b) {
            int np = (lens[b] + page - 1) / page;
            for (t = 0; t < maxp; ++t) bt[(size_t)b * maxp + t] = t < np ? next++ : pages - 1;
            if (lens[b] > maxL) maxL = lens[b];
        }
        CHECK(oracle_paged_attention(B, qlen, hq, hkv, d, page, maxp, dtype, q, kc, vc, bt, lens,
                                     0.125, causal, nthreads, out, lse) == 0, "paged call");
        for (b = 0; b < B; ++b)
            for (i = 0; i < qlen; ++i)
                for (h = 0; h < hq; ++h) {
                    const int n = (b * qlen + i) * hq + h;
                    vis[n] = visible_of(lens[b], qlen, i, causal);
                    lse_rows[n] = lse[((size_t)b * hq + h) * qlen + i];
                }
        check_rows(out, lse_rows, nrows, d, vis);
        /* split partials and their combine, for several split counts */
        for (s = 1; s <= 7; s += 3) {
            const int C = maxL > 0 ? (maxL + s - 1) / s : 1;
            double *op = (double *)malloc(sizeof(double) * (size_t)s * nrows * d);
            double *lp = (double *)malloc(sizeof(double) * (size_t)s * nrows);
            double *o2 = (double *)malloc(sizeof(double) * (size_t)nrows * d);
            double *l2 = (double *)malloc(sizeof(double) * (size_t)nrows);
            int blk;
            for (blk = 1; blk <= 16; blk += 15) {
                CHECK(oracle_paged_split_partials(B, qlen, hq, hkv, d, page, maxp, dtype, q, kc, vc,
                                                  bt, lens, 0.125, causal, s, C, blk, nthreads,
                                                  op, lp) == 0, "paged partials");
                oracle_combine(s, nrows, d, op, lp, o2, l2);
                check_rows(o2, l2, nrows, d, vis);
            }
            /* splits that do not cover every key are rejected */
            if (maxL > 1)
                CHECK(oracle_paged_split_partials(B, qlen, hq, hkv, d, page, maxp, dtype, q, kc, vc,
                                                  bt, lens, 0.125, causal, 1, maxL - 1, 4, 1, op,
                                                  lp) != 0, "uncovered keys rejected");
            free(op); free(lp); free(o2); free(l2);
        }
        /* rejected shapes */
        CHECK(oracle_paged_attention(B, qlen, hq + 1, hkv, d, page, maxp, dtype, q, kc, vc, bt, lens,
                                     0.125, causal, 1, out, lse) != 0 || (hq + 1) % hkv == 0,
              "Hq % Hkv rejected");
        CHECK(oracle_paged_attention(B, qlen, hq, hkv, 0, page, maxp, dtype, q, kc, vc, bt, lens,
                                     0.125, causal, 1, out, lse) != 0, "d = 0 rejected");
        free(q); free(kc); free(vc); free(bt); free(out); free(lse); free(lse_rows); free(vis);
    }
}

static void dense_case(int hq, int hkv, int qlen, int kvlen, int d, int dtype, int causal,
                       int nthreads) {
    int nrows = hq * qlen, n, s;
    uint16_t *q = fill16((size_t)nrows * d, dtype);
    uint16_t *k = fill16((size_t)hkv * kvlen * d, dtype);
    uint16_t *v = fill16((size_t)hkv * kvlen * d, dtype);
    double *out = (double *)malloc(sizeof(double) * (size_t)nrows * d);
    double *lse = (double *)malloc(sizeof(double) * (size_t)nrows);
    int *vis = (int *)malloc(sizeof(int) * (size_t)nrows);
    for (n = 0; n < nrows; ++n) vis[n] = visible_of(kvlen, qlen, n % qlen, causal);
    CHECK(oracle_dense_attention(hq, hkv, qlen, kvlen, d, dtype, q, k, v, 0.25, causal, nthreads,
                                 out, lse) == 0, "dense call");
    check_rows(out, lse, nrows, d, vis);
    for (s = 1; s <= 5; s += 4) {
        const int C = kvlen > 0 ? (kvlen + s - 1) / s : 1;
        double *op = (double *)malloc(sizeof(double) * (size_t)s * nrows * d);
        double *lp = (double *)malloc(sizeof(double) * (size_t)s * nrows);
        CHECK(oracle_dense_split_partials(hq, hkv, qlen, kvlen, d, dtype, q, k, v, 0.25, causal, s,
                                          C, 3, nthreads, op, lp) == 0, "dense partials");
        oracle_combine(s, nrows, d, op, lp, out, lse);
        check_rows(out, lse, nrows, d, vis);
        free(op); free(lp);
    }
    CHECK(oracle_dense_attention(hq, hkv, qlen, -1, d, dtype, q, k, v, 0.25, causal, 1, out, lse)
          != 0, "negative kv_len rejected");
    free(q); free(k); free(v); free(out); free(lse); free(vis);
}

int main(void) {
    static const int32_t lens_a[3] = {0, 17, 40};
    static const int32_t lens_b[4] = {1, 16, 33, 0};
    static const int32_t lens_c[2] = {5, 70};
    int x, dtype, causal;
    for (x = 0; x < 65536; ++x) { /* every 16-bit pattern decodes without UB */
        (void)oracle_decode_scalar((uint16_t)x, 0);
        (void)oracle_decode_scalar((uint16_t)x, 1);
    }
    for (dtype = 0; dtype < 2; ++dtype)
        for (causal = 0; causal < 2; ++causal) {
            paged_case(3, 1, 4, 2, 8, 16, dtype, causal, lens_a, 1);
            paged_case(4, 3, 6, 3, 1, 16, dtype, causal, lens_b, 3);
            paged_case(2, 2, 2, 2, 64, 32, dtype, causal, lens_c, 2);
            dense_case(4, 2, 3, 37, 8, dtype, causal, 2);
            dense_case(2, 1, 1, 0, 5, dtype, causal, 1);
            dense_case(3, 3, 4, 2, 1, dtype, causal, 3);
        }
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run: ok\n");
    return 0;
}
