/*
 * CPU oracle for SAF3R head-wise dynamic sparse global attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library it checks.
 *
 * Plain, slow and meant to be read against the pages: every function below
 * follows one passage of "SAF3R: Dynamic Sparse Attention for Feed-Forward 3D
 * Reconstruction Transformers" (arXiv 2607.03612, HTML version) and works in
 * double precision on the exact input values (bfloat16 inputs are decoded
 * exactly).  Loops go over the definition's own indices; the only
 * parallelism is an OpenMP loop over independent queries / rows.
 *
 * Token layout (a reading of the pages, which name camera and register tokens
 * but not their order): frame f holds T = ns + P tokens, the ns special tokens
 * first, then the P patches row-major.  Token j lies in frame j / T at offset
 * t = j % T; it is special iff t < ns.  Patch number u = f * P + p is token
 * f * T + ns + p.
 *
 * Element type codes: 0 = float32, 1 = bfloat16 (raw 16-bit patterns).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* Threads the OpenMP loops below use (reported with CPU timings). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

static double load_elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[i];
    uint32_t bits = ((uint32_t)((const uint16_t *)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------
 * Static key sets (Sec. 4.1 "Static Kernel" and "Uniform Sampling Kernel";
 * Sec. 3 Observation #2 for the anchor frame and sink tokens).
 * ------------------------------------------------------------------------ */

/* Position heads: every special token, every token of the anchor frame and
 * every token of the query's own frame, as a set (no repeats), ascending.
 * Returns the set size; writes it to out when out != NULL. */
int64_t oracle_position_set(int32_t S, int32_t ns, int32_t P, int32_t anchor,
                            int32_t query_frame, int64_t *out)
{
    const int64_t T = (int64_t)ns + P, N = (int64_t)S * T;
    int64_t n = 0;
    for (int64_t j = 0; j < N; ++j) {
        const int64_t f = j / T, t = j % T;
        const int member = (t < ns) || (f == anchor) || (f == query_frame);
        if (member) {
            if (out)
                out[n] = j;
            ++n;
        }
    }
    return n;
}

/* Scanning heads: keys on a fixed stride s of the global token index (phase
 * 0), together with all special tokens, as a set, ascending. */
int64_t oracle_scan_set(int32_t S, int32_t ns, int32_t P, int32_t stride, int64_t *out)
{
    const int64_t T = (int64_t)ns + P, N = (int64_t)S * T;
    int64_t n = 0;
    for (int64_t j = 0; j < N; ++j) {
        const int member = (j % stride == 0) || (j % T < ns);
        if (member) {
            if (out)
                out[n] = j;
            ++n;
        }
    }
    return n;
}

/* ------------------------------------------------------------------------
 * Top-K with the ordering (score descending, id ascending).
 * ------------------------------------------------------------------------ */
typedef struct {
    double score;
    int64_t id;
} scored_t;

static int cmp_score_desc_id_asc(const void *a, const void *b)
{
    const scored_t *x = (const scored_t *)a, *y = (const scored_t *)b;
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
    return (x->id < y->id) ? -1 : (x->id > y->id);
}

static int cmp_i64(const void *a, const void *b)
{
    const int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x < y) ? -1 : (x > y);
}

/* Order the n candidates by (score desc, id asc), keep the first min(K, n),
 * write their ids ascending to out and return how many were kept.  kth (if
 * not NULL) receives the score of the last kept candidate and next (if not
 * NULL) the score of the first dropped one (-inf when none is dropped). */
int64_t oracle_topk(const double *score, const int64_t *ids, int64_t n, int64_t K,
                    int64_t *out, double *kth, double *next)
{
    if (n <= 0 || K <= 0)
        return 0;
    scored_t *tmp = (scored_t *)malloc((size_t)n * sizeof *tmp);
    if (!tmp)
        return -1;
    for (int64_t i = 0; i < n; ++i) {
        tmp[i].score = score[i];
        tmp[i].id = ids ? ids[i] : i;
    }
    qsort(tmp, (size_t)n, sizeof *tmp, cmp_score_desc_id_asc);
    const int64_t kept = K < n ? K : n;
    for (int64_t i = 0; i < kept; ++i)
        out[i] = tmp[i].id;
    if (kth)
        *kth = tmp[kept - 1].score;
    if (next)
        *next = kept < n ? tmp[kept].score : -INFINITY;
    free(tmp);
    qsort(out, (size_t)kept, sizeof *out, cmp_i64);
    return kept;
}

/* ------------------------------------------------------------------------
 * Query probe for vertical-line heads (Sec. 4.3, "Query-Probe Top-K Kernel"):
 * the column average of S = Q K^T / sqrt(D) equals qbar K^T / sqrt(D) with
 * qbar the mean of all N queries.
 * ------------------------------------------------------------------------ */
int oracle_mean_query(const void *q, int dtype, int64_t N, int32_t d, int64_t row_stride,
                      double *qbar)
{
    for (int32_t c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int64_t i = 0; i < N; ++i)
            acc += load_elem(q, dtype, i * row_stride + c);
        qbar[c] = acc / (double)N;
    }
    return 0;
}

int oracle_probe_scores(const void *k, int dtype, int64_t N, int32_t d, int64_t row_stride,
                        const double *qbar, double *r)
{
    const double scale = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j) {
        double acc = 0.0;
        for (int32_t c = 0; c < d; ++c)
            acc += qbar[c] * load_elem(k, dtype, j * row_stride + c);
        r[j] = acc * scale;
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * DINO correspondence index (Sec. 4.1 "DINO Top-K Kernel", Sec. 4.3): cosine
 * similarity between a patch's DINO feature and the patches of the other
 * frames.  Candidates exclude the query's own frame.  Scores of own-frame
 * patches are written as NaN.
 * ------------------------------------------------------------------------ */
static double feat_dot(const void *F, int dtype, int64_t row_stride, int32_t Df, int64_t a, int64_t b)
{
    double acc = 0.0;
    for (int32_t c = 0; c < Df; ++c)
        acc += load_elem(F, dtype, a * row_stride + c) * load_elem(F, dtype, b * row_stride + c);
    return acc;
}

int oracle_feature_norms(const void *F, int dtype, int64_t Np, int32_t Df, int64_t row_stride,
                         double *norms)
{
#pragma omp parallel for schedule(static)
    for (int64_t u = 0; u < Np; ++u)
        norms[u] = sqrt(feat_dot(F, dtype, row_stride, Df, u, u));
    return 0;
}

/* out: nrows x (S*P) cosines for the patches listed in rows (patch numbers). */
int oracle_corr_scores(const void *F, int dtype, int32_t S, int32_t P, int32_t Df,
                       int64_t row_stride, const double *norms, const int64_t *rows,
                       int64_t nrows, double *out)
{
    const int64_t Np = (int64_t)S * P;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t u = rows[r];
        double *row = out + r * Np;
        for (int64_t v = 0; v < Np; ++v) {
            if (v / P == u / P) {
                row[v] = NAN;
                continue;
            }
            const double nn = norms[u] * norms[v];
            row[v] = nn > 0.0 ? feat_dot(F, dtype, row_stride, Df, u, v) / nn : 0.0;
        }
    }
    return 0;
}

/* Index rows for the listed patches.  mode 0 ("total"): the first
 * min(K, (S-1)P) candidates by (cosine desc, token asc).  mode 1
 * ("per frame"): the first min(K, P) of every other frame.  Output: global
 * token indices, ascending, kc per row (kc = min(K,(S-1)P) or (S-1)min(K,P)).
 * tau[r] (may be NULL) receives the smallest kept score (total mode) and
 * next[r] the best dropped score.  Returns kc, or a negative value. */
int64_t oracle_corr_index(const void *F, int dtype, int32_t S, int32_t ns, int32_t P, int32_t Df,
                          int64_t row_stride, int32_t K, int32_t mode, const int64_t *rows,
                          int64_t nrows, int64_t *out, double *tau, double *next)
{
    const int64_t Np = (int64_t)S * P, T = (int64_t)ns + P;
    if (S < 2 || K <= 0)
        return -1;
    const int64_t kc = mode == 0 ? ((int64_t)K < (S - 1) * (int64_t)P ? K : (S - 1) * (int64_t)P)
                                 : (int64_t)(S - 1) * (K < P ? K : P);
    double *norms = (double *)malloc((size_t)Np * sizeof(double));
    if (!norms)
        return -2;
    oracle_feature_norms(F, dtype, Np, Df, row_stride, norms);
    int failed = 0;
#pragma omp parallel
    {
        double *sc = (double *)malloc((size_t)Np * sizeof(double));
        int64_t *id = (int64_t *)malloc((size_t)Np * sizeof(int64_t));
        if (!sc || !id) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!sc || !id)
                continue;
            const int64_t u = rows[r], fu = u / P;
            int64_t *dst = out + r * kc;
            if (mode == 0) {
                int64_t n = 0;
                for (int64_t v = 0; v < Np; ++v) {
                    if (v / P == fu)
                        continue;
                    const double nn = norms[u] * norms[v];
                    sc[n] = nn > 0.0 ? feat_dot(F, dtype, row_stride, Df, u, v) / nn : 0.0;
                    id[n] = (v / P) * T + ns + (v % P);
                    ++n;
                }
                oracle_topk(sc, id, n, K, dst, tau ? &tau[r] : NULL, next ? &next[r] : NULL);
            } else {
                int64_t w = 0;
                for (int64_t g = 0; g < S; ++g) {
                    if (g == fu)
                        continue;
                    for (int64_t p = 0; p < P; ++p) {
                        const int64_t v = g * P + p;
                        const double nn = norms[u] * norms[v];
                        sc[p] = nn > 0.0 ? feat_dot(F, dtype, row_stride, Df, u, v) / nn : 0.0;
                        id[p] = g * T + ns + p;
                    }
                    w += oracle_topk(sc, id, P, K, dst + w, NULL, NULL);
                }
                qsort(dst, (size_t)w, sizeof *dst, cmp_i64);
                if (tau)
                    tau[r] = NAN;
                if (next)
                    next[r] = NAN;
            }
        }
        free(sc);
        free(id);
    }
    free(norms);
    return failed ? -2 : kc;
}

/* ------------------------------------------------------------------------
 * Attention over a key set (softmax with excluded logits at -inf; scale
 * 1/sqrt(D) as in Sec. 4.3):
 *   l_j = q . k_j / sqrt(d),  m = max_j l_j,  w_j = exp(l_j - m),
 *   o = sum_j w_j v_j / sum_j w_j.
 * Rows sharing a key set point to one set: row r uses
 * set_keys[set_ptr[s] .. set_ptr[s+1]) with s = row_set[r].  q, k, v point at
 * one head's [N, d] block with the given row strides (in elements).
 * ------------------------------------------------------------------------ */
int oracle_attention(const void *q, const void *k, const void *v, int dtype, int32_t d,
                     int64_t q_stride, int64_t kv_stride, int64_t nrows, const int64_t *rows,
                     const int64_t *row_set, const int64_t *set_ptr, const int64_t *set_keys,
                     double *out)
{
    const double scale = 1.0 / sqrt((double)d);
    int bad = 0;
#pragma omp parallel
    {
        int64_t cap = 0;
        double *logit = NULL;
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t s = row_set[r];
            const int64_t *keys = set_keys + set_ptr[s];
            const int64_t n = set_ptr[s + 1] - set_ptr[s];
            double *o = out + r * d;
            if (n <= 0) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            if (n > cap) {
                free(logit);
                cap = n;
                logit = (double *)malloc((size_t)cap * sizeof(double));
            }
            const int64_t qi = rows[r];
            double m = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                double acc = 0.0;
                for (int32_t c = 0; c < d; ++c)
                    acc += load_elem(q, dtype, qi * q_stride + c) *
                           load_elem(k, dtype, keys[j] * kv_stride + c);
                logit[j] = acc * scale;
                if (logit[j] > m)
                    m = logit[j];
            }
            double denom = 0.0;
            for (int32_t c = 0; c < d; ++c)
                o[c] = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                const double w = exp(logit[j] - m);
                denom += w;
                for (int32_t c = 0; c < d; ++c)
                    o[c] += w * load_elem(v, dtype, keys[j] * kv_stride + c);
            }
            for (int32_t c = 0; c < d; ++c)
                o[c] /= denom;
        }
        free(logit);
    }
    return bad ? -1 : 0;
}
