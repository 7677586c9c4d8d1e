/*
 * attn_oracle.c -- float64 CPU oracle for exact decode / small-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path may include, link,
 * load or call this file; only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark do.  It shares no code, header, table or
 * helper with the GPU library.
 *
 * What it computes (the plain definition, no blocking, fusion or reordering):
 *
 *   For every output row (batch b, query position i, query head hq) with
 *   kv head h = hq / G (G = Hq / Hkv), key/value rows k_j, v_j for j < L:
 *       s_j = scale * sum_d q[d] * k_j[d]
 *       m   = max_j s_j
 *       l   = sum_j exp(s_j - m)
 *       O   = sum_j exp(s_j - m) * v_j / l
 *       LSE = m + ln(l)
 *
 *   Sources:
 *   - "SmallQ FlashAttention (Vector)" README, section 接口 (interface):
 *     O = softmax(Q K^T / sqrt(headDim)) V over [heads, qLen, headDim].
 *   - ai6s.net FlashAttention / ops-transformer article, sections
 *     "标准 Attention 的问题" (standard attention) and
 *     "FlashAttention 的数学细节" (softmax with the max offset m).
 *   - lpnh.cn "pack_gqa 与 num_splits" article, section
 *     "两个开关在 kernel 层面各做了什么": the query heads of one KV head share
 *     that KV head (grouped-query attention), and each KV split yields a
 *     partial output plus its logsumexp, merged afterwards.
 *   - MXFlashAttn 1.4.0 page, section 能力矩阵 (capability matrix): paged KV
 *     cache; MixedQuantSparseFlashMlaMetadata article, section 参数说明:
 *     the PA_BBND cache layout (block, token-in-block, head, dim).
 *
 *   Inputs are the raw 16-bit patterns (IEEE binary16 or bfloat16); each is
 *   converted exactly to double.  All arithmetic is double; the outputs are
 *   not rounded to any 16-bit type.
 *
 *   Readings where the pages are silent (each also listed in the design
 *   notes): natural-log LSE in units of scaled scores; L = 0 gives O = 0 and
 *   LSE = -inf; head mapping h = hq / G; split s covers keys
 *   [s*C, (s+1)*C) clipped to [0, L), with one split length C for the whole
 *   batch (callers take C = 16*ceil(ceil(maxL/16)/S)); an empty split gives
 *   (O_s = 0, LSE_s = -inf); the combine is the max-shifted log-sum-exp merge.
 *
 *   Causal (the lpnh.cn article's flash_attn_with_kvcache(..., causal=True)
 *   example in section "num_splits 怎么选"; the pages do not define the
 *   alignment): the qlen new queries are the last qlen positions of the
 *   sequence, so query i of qlen sees keys j <= L - qlen + i, i.e. the first
 *   max(0, L - qlen + 1 + i) keys (bottom-right alignment).  A row that sees
 *   no key is an empty row (O = 0, LSE = -inf).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F16 0
#define ORC_BF16 1

/* ---- exact 16-bit -> double decoding (from the format definitions) ---- */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
static double decode_bf16(uint16_t b) {
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xff;
    int f = b & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133); /* f * 2^-126 * 2^-7 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134); /* (1 + f/128) * 2^(e-127) */
    return sign ? -v : v;
}

static double decode(uint16_t x, int dtype) {
    return dtype == ORC_BF16 ? decode_bf16(x) : decode_f16(x);
}

double oracle_decode_scalar(uint16_t x, int dtype) { return decode(x, dtype); }

/* ---- one problem instance, described by row-pointer tables ------------- */

typedef struct {
    int nrows;         /* output rows                                      */
    int d;             /* head dim                                         */
    int dtype;
    double scale;
    const uint16_t *const *qrow;  /* [nrows] -> d elements                 */
    const int *len;               /* [nrows] number of keys L              */
    const uint16_t *const *const *krow; /* [nrows] -> [L] -> d elements    */
    const uint16_t *const *const *vrow;
    double *out;                  /* [nrows][d]                            */
    double *lse;                  /* [nrows]                               */
    /* split model (optional) */
    int num_splits;
    int split_keys;    /* keys per split, C                                */
    int block;
    double *o_part;               /* [S][nrows][d]                         */
    double *lse_part;             /* [S][nrows]                            */
} problem_t;

/* Two-pass softmax attention over keys [j0, j1) of one row. */
static void attend_direct(const problem_t *P, int r, int j0, int j1, double *o, double *lse) {
    int d = P->d;
    double q[1024];
    double *s;
    double m = -INFINITY, l = 0.0;
    int j, e;
    for (e = 0; e < d; ++e) q[e] = decode(P->qrow[r][e], P->dtype);
    for (e = 0; e < d; ++e) o[e] = 0.0;
    if (j1 <= j0) {
        *lse = -INFINITY;
        return;
    }
    s = (double *)malloc(sizeof(double) * (size_t)(j1 - j0));
    for (j = j0; j < j1; ++j) {
        const uint16_t *k = P->krow[r][j];
        double acc = 0.0;
        for (e = 0; e < d; ++e) acc += q[e] * decode(k[e], P->dtype);
        s[j - j0] = P->scale * acc;
        if (s[j - j0] > m) m = s[j - j0];
    }
    for (j = j0; j < j1; ++j) l += exp(s[j - j0] - m);
    for (j = j0; j < j1; ++j) {
        const uint16_t *v = P->vrow[r][j];
        double p = exp(s[j - j0] - m);
        for (e = 0; e < d; ++e) o[e] += p * decode(v[e], P->dtype);
    }
    for (e = 0; e < d; ++e) o[e] /= l;
    *lse = m + log(l);
    free(s);
}

/*
 * Online softmax over keys [j0, j1) in blocks of `block` keys, in the order
 * of the ai6s.net article's FlashAttention pseudocode (section
 * "FlashAttention 的数学细节"): new running max from the block's max,
 * rescale the running output and running sum by exp(m_old - m_new), add the
 * block's exp(s - m_new)-weighted values and sums; divide by l at the end.
 */
static void attend_online(const problem_t *P, int r, int j0, int j1, double *o, double *lse) {
    int d = P->d, blk = P->block > 0 ? P->block : 1;
    double q[1024], s[4096];
    double m = -INFINITY, l = 0.0;
    int jb, j, e;
    for (e = 0; e < d; ++e) q[e] = decode(P->qrow[r][e], P->dtype);
    for (e = 0; e < d; ++e) o[e] = 0.0;
    if (blk > 4096) blk = 4096;
    for (jb = j0; jb < j1; jb += blk) {
        int je = jb + blk < j1 ? jb + blk : j1;
        double bmax = -INFINITY, m_new, alpha, bsum = 0.0;
        for (j = jb; j < je; ++j) {
            const uint16_t *k = P->krow[r][j];
            double acc = 0.0;
            for (e = 0; e < d; ++e) acc += q[e] * decode(k[e], P->dtype);
            s[j - jb] = P->scale * acc;
            if (s[j - jb] > bmax) bmax = s[j - jb];
        }
        m_new = m > bmax ? m : bmax;
        /* exp_old: the old sum carried to the new max (m = -inf on the
         * first block gives 0); exp_new: the block's own sum taken at its
         * own max, carried to the new max. */
        alpha = exp(m - m_new);
        for (j = jb; j < je; ++j) bsum += exp(s[j - jb] - bmax);
        for (e = 0; e < d; ++e) o[e] *= alpha;
        for (j = jb; j < je; ++j) {
            const uint16_t *v = P->vrow[r][j];
            double p = exp(s[j - jb] - m_new);
            for (e = 0; e < d; ++e) o[e] += p * decode(v[e], P->dtype);
        }
        l = alpha * l + exp(bmax - m_new) * bsum;
        m = m_new;
    }
    if (j1 <= j0) {
        *lse = -INFINITY;
        return;
    }
    for (e = 0; e < d; ++e) o[e] /= l;
    *lse = m + log(l);
}

/* Split s of a row with L keys covers [s*C, (s+1)*C) clipped to [0, L). */
static void split_range(int L, int C, int s, int *j0, int *j1) {
    long a = (long)s * C, b = (long)(s + 1) * C;
    if (a > L) a = L;
    if (b > L) b = L;
    *j0 = (int)a;
    *j1 = (int)b;
}

typedef struct {
    const problem_t *P;
    int r0, r1;
} work_t;

static void *run_rows(void *arg) {
    const work_t *w = (const work_t *)arg;
    const problem_t *P = w->P;
    int r;
    for (r = w->r0; r < w->r1; ++r) {
        if (P->num_splits <= 0) {
            attend_direct(P, r, 0, P->len[r], P->out + (size_t)r * P->d, P->lse + r);
        } else {
            int s;
            for (s = 0; s < P->num_splits; ++s) {
                int j0, j1;
                split_range(P->len[r], P->split_keys, s, &j0, &j1);
                attend_online(P, r, j0, j1, P->o_part + ((size_t)s * P->nrows + r) * P->d,
                              P->lse_part + (size_t)s * P->nrows + r);
            }
        }
    }
    return NULL;
}

static void run_problem(const problem_t *P, int nthreads) {
    int t;
    pthread_t th[256];
    work_t w[256];
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > P->nrows) nthreads = P->nrows > 0 ? P->nrows : 1;
    for (t = 0; t < nthreads; ++t) {
        w[t].P = P;
        w[t].r0 = (int)((long)P->nrows * t / nthreads);
        w[t].r1 = (int)((long)P->nrows * (t + 1) / nthreads);
    }
    if (nthreads == 1) {
        run_rows(&w[0]);
        return;
    }
    for (t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, run_rows, &w[t]);
    for (t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ---- tables for the two layouts ---------------------------------------- */

typedef struct {
    const uint16_t **qrow;
    int *len;
    const uint16_t ***krow;
    const uint16_t ***vrow;
    const uint16_t **kpool, **vpool; /* per-row key tables live here */
} tables_t;

static void free_tables(tables_t *T, int nrows) {
    (void)nrows;
    free(T->qrow);
    free(T->len);
    free(T->krow);
    free(T->vrow);
    free(T->kpool);
    free(T->vpool);
}

/* Keys query i of qlen sees in a sequence of L keys. */
static int visible_keys(int L, int qlen, int i, int causal) {
    int n;
    if (!causal) return L;
    n = L - qlen + 1 + i;
    if (n < 0) n = 0;
    return n < L ? n : L;
}

/*
 * Paged layout.  q, out: [B, qlen, Hq, d]; lse: [B, Hq, qlen];
 * k_cache, v_cache: [num_pages, page_size, Hkv, d];
 * block_table: [B, max_pages] (key j of sequence b sits in physical page
 * block_table[b][j / page_size], slot j % page_size); seqlens: [B].
 * Row n = (b * qlen + i) * Hq + hq.
 */
static int build_paged(tables_t *T, int B, int qlen, int hq, int hkv, int d, int page_size,
                       int max_pages, const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                       const int32_t *bt, const int32_t *seqlens, int causal) {
    int nrows = B * qlen * hq, G = hq / hkv;
    long total = 0;
    int b, i, h, j;
    T->qrow = (const uint16_t **)malloc(sizeof(void *) * (size_t)(nrows > 0 ? nrows : 1));
    T->len = (int *)malloc(sizeof(int) * (size_t)(nrows > 0 ? nrows : 1));
    T->krow = (const uint16_t ***)malloc(sizeof(void *) * (size_t)(nrows > 0 ? nrows : 1));
    T->vrow = (const uint16_t ***)malloc(sizeof(void *) * (size_t)(nrows > 0 ? nrows : 1));
    for (b = 0; b < B; ++b) total += (long)seqlens[b] * hkv;
    T->kpool = (const uint16_t **)malloc(sizeof(void *) * (size_t)(total > 0 ? total : 1));
    T->vpool = (const uint16_t **)malloc(sizeof(void *) * (size_t)(total > 0 ? total : 1));
    total = 0;
    for (b = 0; b < B; ++b) {
        int L = seqlens[b];
        if (L < 0 || L > max_pages * page_size) return -1;
        for (h = 0; h < hkv; ++h) {
            const uint16_t **kt = T->kpool + total, **vt = T->vpool + total;
            for (j = 0; j < L; ++j) {
                long page = bt[(long)b * max_pages + j / page_size];
                long off = ((page * page_size + j % page_size) * hkv + h) * (long)d;
                kt[j] = kc + off;
                vt[j] = vc + off;
            }
            for (i = 0; i < qlen; ++i) {
                int g;
                for (g = 0; g < G; ++g) {
                    int hh = h * G + g;
                    int n = (b * qlen + i) * hq + hh;
                    T->qrow[n] = q + (size_t)n * d;
                    T->len[n] = visible_keys(L, qlen, i, causal);
                    T->krow[n] = kt;
                    T->vrow[n] = vt;
                }
            }
            total += L;
        }
    }
    return 0;
}

/* Dense layout.  q, out: [Hq, qlen, d]; lse: [Hq, qlen]; k, v: [Hkv, kvlen, d].
 * Row n = hq * qlen + i. */
static void build_dense(tables_t *T, int hq, int hkv, int qlen, int kvlen, int d,
                        const uint16_t *q, const uint16_t *k, const uint16_t *v, int causal) {
    int nrows = hq * qlen, G = hq / hkv;
    int h, i, j, hh;
    T->qrow = (const uint16_t **)malloc(sizeof(void *) * (size_t)(nrows > 0 ? nrows : 1));
    T->len = (int *)malloc(sizeof(int) * (size_t)(nrows > 0 ? nrows : 1));
    T->krow = (const uint16_t ***)malloc(sizeof(void *) * (size_t)(nrows > 0 ? nrows : 1));
    T->vrow = (const uint16_t ***)malloc(sizeof(void *) * (size_t)(nrows > 0 ? nrows : 1));
    T->kpool = (const uint16_t **)malloc(sizeof(void *) * (size_t)((long)hkv * kvlen + 1));
    T->vpool = (const uint16_t **)malloc(sizeof(void *) * (size_t)((long)hkv * kvlen + 1));
    for (h = 0; h < hkv; ++h)
        for (j = 0; j < kvlen; ++j) {
            T->kpool[(long)h * kvlen + j] = k + ((long)h * kvlen + j) * d;
            T->vpool[(long)h * kvlen + j] = v + ((long)h * kvlen + j) * d;
        }
    for (hh = 0; hh < hq; ++hh)
        for (i = 0; i < qlen; ++i) {
            int n = hh * qlen + i;
            h = hh / G;
            T->qrow[n] = q + (size_t)n * d;
            T->len[n] = visible_keys(kvlen, qlen, i, causal);
            T->krow[n] = T->kpool + (long)h * kvlen;
            T->vrow[n] = T->vpool + (long)h * kvlen;
        }
}

static int check_common(int hq, int hkv, int d) {
    if (hq <= 0 || hkv <= 0 || hq % hkv != 0) return -1;
    if (d <= 0 || d > 1024) return -1;
    return 0;
}

/* Exact attention, paged KV cache.  out/lse in the [B,qlen,Hq,d] / [B,Hq,qlen] layouts. */
int oracle_paged_attention(int B, int qlen, int hq, int hkv, int d, int page_size, int max_pages,
                           int dtype, const uint16_t *q, const uint16_t *kc, const uint16_t *vc,
                           const int32_t *block_table, const int32_t *seqlens, double scale,
                           int causal, int nthreads, double *out, double *lse) {
    tables_t T;
    problem_t P;
    int nrows = B * qlen * hq, b, i, h;
    double *lse_rows;
    if (check_common(hq, hkv, d) || page_size <= 0) return -1;
    memset(&T, 0, sizeof(T));
    if (build_paged(&T, B, qlen, hq, hkv, d, page_size, max_pages, q, kc, vc, block_table, seqlens,
                    causal)) {
        free_tables(&T, nrows);
        return -1;
    }
    lse_rows = (double *)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1));
    memset(&P, 0, sizeof(P));
    P.nrows = nrows; P.d = d; P.dtype = dtype; P.scale = scale;
    P.qrow = T.qrow; P.len = T.len;
    P.krow = (const uint16_t *const *const *)T.krow;
    P.vrow = (const uint16_t *const *const *)T.vrow;
    P.out = out; P.lse = lse_rows;
    run_problem(&P, nthreads);
    for (b = 0; b < B; ++b)
        for (i = 0; i < qlen; ++i)
            for (h = 0; h < hq; ++h)
                lse[((long)b * hq + h) * qlen + i] = lse_rows[((long)b * qlen + i) * hq + h];
    free(lse_rows);
    free_tables(&T, nrows);
    return 0;
}

/* Exact attention, dense K/V.  out [Hq,qlen,d], lse [Hq,qlen]. */
int oracle_dense_attention(int hq, int hkv, int qlen, int kvlen, int d, int dtype,
                           const uint16_t *q, const uint16_t *k, const uint16_t *v, double scale,
                           int causal, int nthreads, double *out, double *lse) {
    tables_t T;
    problem_t P;
    if (check_common(hq, hkv, d) || kvlen < 0) return -1;
    memset(&T, 0, sizeof(T));
    build_dense(&T, hq, hkv, qlen, kvlen, d, q, k, v, causal);
    memset(&P, 0, sizeof(P));
    P.nrows = hq * qlen; P.d = d; P.dtype = dtype; P.scale = scale;
    P.qrow = T.qrow; P.len = T.len;
    P.krow = (const uint16_t *const *const *)T.krow;
    P.vrow = (const uint16_t *const *const *)T.vrow;
    P.out = out; P.lse = lse;
    run_problem(&P, nthreads);
    free_tables(&T, hq * qlen);
    return 0;
}

/*
 * Split partials with the online recurrence, paged layout.
 * o_part: [S][nrows][d], lse_part: [S][nrows], rows n = (b*qlen+i)*Hq+hq.
 */
int oracle_paged_split_partials(int B, int qlen, int hq, int hkv, int d, int page_size,
                                int max_pages, int dtype, const uint16_t *q, const uint16_t *kc,
                                const uint16_t *vc, const int32_t *block_table,
                                const int32_t *seqlens, double scale, int causal, int num_splits,
                                int split_keys, int block, int nthreads, double *o_part,
                                double *lse_part) {
    tables_t T;
    problem_t P;
    int nrows = B * qlen * hq;
    int b;
    if (check_common(hq, hkv, d) || page_size <= 0 || num_splits < 1 || split_keys < 1) return -1;
    for (b = 0; b < B; ++b) /* the splits must cover every key */
        if ((long)num_splits * split_keys < seqlens[b]) return -1;
    memset(&T, 0, sizeof(T));
    if (build_paged(&T, B, qlen, hq, hkv, d, page_size, max_pages, q, kc, vc, block_table, seqlens,
                    causal)) {
        free_tables(&T, nrows);
        return -1;
    }
    memset(&P, 0, sizeof(P));
    P.nrows = nrows; P.d = d; P.dtype = dtype; P.scale = scale;
    P.qrow = T.qrow; P.len = T.len;
    P.krow = (const uint16_t *const *const *)T.krow;
    P.vrow = (const uint16_t *const *const *)T.vrow;
    P.num_splits = num_splits; P.split_keys = split_keys; P.block = block;
    P.o_part = o_part; P.lse_part = lse_part;
    run_problem(&P, nthreads);
    free_tables(&T, nrows);
    return 0;
}

/* Split partials, dense layout.  Rows n = hq*qlen+i. */
int oracle_dense_split_partials(int hq, int hkv, int qlen, int kvlen, int d, int dtype,
                                const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                double scale, int causal, int num_splits, int split_keys,
                                int block, int nthreads, double *o_part, double *lse_part) {
    tables_t T;
    problem_t P;
    if (check_common(hq, hkv, d) || kvlen < 0 || num_splits < 1 || split_keys < 1) return -1;
    if ((long)num_splits * split_keys < kvlen) return -1; /* the splits must cover every key */
    memset(&T, 0, sizeof(T));
    build_dense(&T, hq, hkv, qlen, kvlen, d, q, k, v, causal);
    memset(&P, 0, sizeof(P));
    P.nrows = hq * qlen; P.d = d; P.dtype = dtype; P.scale = scale;
    P.qrow = T.qrow; P.len = T.len;
    P.krow = (const uint16_t *const *const *)T.krow;
    P.vrow = (const uint16_t *const *const *)T.vrow;
    P.num_splits = num_splits; P.split_keys = split_keys; P.block = block;
    P.o_part = o_part; P.lse_part = lse_part;
    run_problem(&P, nthreads);
    free_tables(&T, hq * qlen);
    return 0;
}

/*
 * Merge S partials per row (lpnh.cn article, section
 * "两个开关在 kernel 层面各做了什么": per-split partial attention and its
 * logsumexp, reduced at the end).  Max-shifted log-sum-exp weights:
 *   M = max_s LSE_s, w_s = exp(LSE_s - M),
 *   O = sum_s w_s O_s / sum_s w_s, LSE = M + ln(sum_s w_s).
 * Rows whose partials are all empty (LSE_s = -inf) give O = 0, LSE = -inf.
 */
void oracle_combine(int num_splits, int nrows, int d, const double *o_part,
                    const double *lse_part, double *out, double *lse) {
    int n, s, e;
    for (n = 0; n < nrows; ++n) {
        double M = -INFINITY, wsum = 0.0;
        double *o = out + (size_t)n * d;
        for (s = 0; s < num_splits; ++s)
            if (lse_part[(size_t)s * nrows + n] > M) M = lse_part[(size_t)s * nrows + n];
        for (e = 0; e < d; ++e) o[e] = 0.0;
        if (M == -INFINITY) {
            lse[n] = -INFINITY;
            continue;
        }
        for (s = 0; s < num_splits; ++s) {
            double w = exp(lse_part[(size_t)s * nrows + n] - M);
            const double *os = o_part + ((size_t)s * nrows + n) * d;
            wsum += w;
            for (e = 0; e < d; ++e) o[e] += w * os[e];
        }
        for (e = 0; e < d; ++e) o[e] /= wsum;
        lse[n] = M + log(wsum);
    }
}
