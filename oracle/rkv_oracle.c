/*
 * rkv_oracle.c -- plain, slow CPU oracle for the RocketKV decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * Sources (three web pages on RocketKV, cited by title and section):
 *   [P1] "RocketKV: Accelerating Long-Context LLM Inference via Two-Stage KV
 *        Cache Compression" (atlas.scime.ai summary), sections "Approach" and
 *        "Key results".
 *   [P2] The paper's abstract (papers.pytorch.kr/papers/2502.14051).
 *   [P3] "RocketKV-adapted -- Two-Stage Compression" (veloxquant-mlx docs),
 *        sections "Where it sits -- the mechanism gap", "The one setting worth
 *        tuning", "Adaptation notes" and "Evidence".
 *
 * Every function works on one (sequence, KV head) unit with logical,
 * contiguous rows; element type is given by `dt` (0 = fp32, 1 = bf16 bits).
 * Floating-point arithmetic follows the order written in each comment; the
 * file is compiled with -ffp-contract=off so no multiply-add is fused.
 *
 * Parity status: every function below is pinned by tests/test_oracle_*.py
 * (closed forms, the pages' worked example, invariants, library special
 * cases, brute force on small inputs).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define RKVO_OK 0
#define RKVO_EINVAL (-1)
#define RKVO_ENOMEM (-2)

/* ---- element access --------------------------------------------------- */

static float bf16_bits_to_float(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Element i of an array of type dt, as fp32 (bf16 widens exactly). */
static float elem(const void *p, int dt, int64_t i) {
    if (dt == 0) return ((const float *)p)[i];
    return bf16_bits_to_float(((const uint16_t *)p)[i]);
}

/* Copy element (no rounding: max/min pick an existing element). */
static void copy_elem(void *dst, int64_t di, const void *src, int64_t si, int dt) {
    if (dt == 0) ((float *)dst)[di] = ((const float *)src)[si];
    else ((uint16_t *)dst)[di] = ((const uint16_t *)src)[si];
}

/* ---- O1: adaptive split of the compression ratio ----------------------- */
/*
 * [P3] "The one setting worth tuning": r = clip(0.2 + 0.06*log2(c), 0.2, 0.8);
 * stage 1 (eviction) compresses by c^r, stage 2 (HSA) by c^(1-r).
 * [P1] "Approach": an adaptive formula splits the ratio between the stages.
 * keep = floor(L / c^r), never below the observation window w, never above L.
 */
int rkvo_split_ratio(double c, int64_t L, int64_t w, double *r, double *c1,
                     double *c2, int64_t *keep) {
    if (!(c >= 1.0) || !isfinite(c) || L < 0 || w < 0) return RKVO_EINVAL;
    double rr = 0.2 + 0.06 * log2(c);
    if (rr < 0.2) rr = 0.2;
    if (rr > 0.8) rr = 0.8;
    double a = pow(c, rr);
    double b = pow(c, 1.0 - rr);
    if (r) *r = rr;
    if (c1) *c1 = a;
    if (c2) *c2 = b;
    if (keep) {
        int64_t k = (int64_t)floor((double)L / a);
        if (k < w) k = w;
        if (k > L) k = L;
        *keep = k;
    }
    return RKVO_OK;
}

/* ---- O3: per-page element-wise key max/min summaries ------------------- */
/*
 * [P3] "Where it sits": Quest-style paged element-wise max/min along the
 * sequence dimension.  Page p covers rows [p*P, min(p*P+P, n)).  Within a page
 * rows are visited in ascending order and a later row replaces the running
 * extreme only when strictly larger (max) / smaller (min), so among equal
 * values the first one's bits are kept.
 * Output layout: smax[p*d + c], smin[p*d + c], same element type as k.
 */
void rkvo_summaries_rebuild(const void *k, int dt, int64_t n, int d, int P,
                            void *smax, void *smin) {
    int64_t np = (n + P - 1) / P;
    for (int64_t p = 0; p < np; ++p) {
        int64_t r0 = p * P, r1 = r0 + P < n ? r0 + P : n;
        for (int c = 0; c < d; ++c) {
            int64_t imax = r0 * d + c, imin = r0 * d + c;
            for (int64_t t = r0 + 1; t < r1; ++t) {
                float x = elem(k, dt, t * d + c);
                if (x > elem(k, dt, imax)) imax = t * d + c;
                if (x < elem(k, dt, imin)) imin = t * d + c;
            }
            copy_elem(smax, p * d + c, k, imax, dt);
            copy_elem(smin, p * d + c, k, imin, dt);
        }
    }
}

/*
 * [P3] "Evidence": the incremental update used during decode must give the
 * same bits as a rebuild.  Rows [n_old, n_new) are folded, in ascending order,
 * into the page they fall in; a page that starts at or after n_old starts
 * from its first new row.
 */
void rkvo_summaries_append(const void *k, int dt, int64_t n_old, int64_t n_new,
                           int d, int P, void *smax, void *smin) {
    for (int64_t t = n_old; t < n_new; ++t) {
        int64_t p = t / P;
        for (int c = 0; c < d; ++c) {
            if (t % P == 0) {
                copy_elem(smax, p * d + c, k, t * d + c, dt);
                copy_elem(smin, p * d + c, k, t * d + c, dt);
            } else {
                float x = elem(k, dt, t * d + c);
                if (x > elem(smax, dt, p * d + c)) copy_elem(smax, p * d + c, k, t * d + c, dt);
                if (x < elem(smin, dt, p * d + c)) copy_elem(smin, p * d + c, k, t * d + c, dt);
            }
        }
    }
}

/* ---- shared selection helper: top-K by (score desc, index asc) --------- */

typedef struct { float s; int64_t i; } scored;

static int cmp_desc_then_index(const void *a, const void *b) {
    const scored *x = (const scored *)a, *y = (const scored *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i < y->i) ? -1 : (x->i > y->i);
}

static int cmp_i64(const void *a, const void *b) {
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x < y) ? -1 : (x > y);
}

/* Indices of the K best of s[0..n) (higher score first, lower index on
 * ties), written in ascending index order into out[0..K). */
static int topk_ascending(const float *s, int64_t n, int64_t K, int64_t *out) {
    scored *v = (scored *)malloc((size_t)(n > 0 ? n : 1) * sizeof *v);
    if (!v) return RKVO_ENOMEM;
    for (int64_t i = 0; i < n; ++i) { v[i].s = s[i]; v[i].i = i; }
    qsort(v, (size_t)n, sizeof *v, cmp_desc_then_index);
    for (int64_t i = 0; i < K; ++i) out[i] = v[i].i;
    qsort(out, (size_t)K, sizeof *out, cmp_i64);
    free(v);
    return RKVO_OK;
}

/* ---- O2: SnapKV++ stage-1 eviction for one KV head group --------------- */
/*
 * [P2] abstract: SnapKV++ adds adaptive pooling size and full GQA
 * compatibility to SnapKV.  [P1] "Approach": SnapKV with a large pooling
 * kernel and selection at the GQA-group level.  [P3] "The problem this
 * solves": stage 1 reuses SnapKV's observation-window scoring.
 *
 * q_win : [G][w][d]  the last w prompt queries of the G query heads that share
 *                    this KV head (query i sits at position L-w+i).
 * k     : [L][d]     prompt keys of this KV head.
 * Steps, for window query i of query head j:
 *   z[t]  = fl(sum_{c ascending} fl(q[c]*k_t[c])) * scale,  t <= L-w+i
 *   m     = max_t z[t];   e[t] = expf(z[t] - m)
 *   ell   = (float) sum_{t ascending} (double) e[t]      (fp64 accumulator)
 *   p[t]  = e[t] / ell
 * A_j[t] = sum_{i ascending} p_{j,i}[t] and A[t] = sum_{j ascending} A_j[t]
 * for the prefix t < L-w (fp32, from +0).
 * Pooled[t] = max{A[u] : |u-t| <= pool_kernel/2, 0 <= u < L-w}.
 * Keep the (keep-w) best prefix positions by (Pooled desc, t asc), sorted
 * ascending, followed by the w window positions.  keep >= L keeps all rows.
 * A and pooled (length L-w) are optional outputs.
 */
int rkvo_snapkv_group(const void *q_win, const void *k, int dt, int64_t L, int d,
                      int G, int w, int pool_kernel, int64_t keep, float scale,
                      float *A_out, float *pooled_out, int32_t *kept) {
    if (L < 0 || d < 1 || G < 1 || w < 1 || pool_kernel < 1 || (pool_kernel % 2) == 0)
        return RKVO_EINVAL;
    if (keep >= L) {
        for (int64_t t = 0; t < L; ++t) kept[t] = (int32_t)t;
        return RKVO_OK;
    }
    if (keep < w || L < w) return RKVO_EINVAL;
    int64_t npre = L - w;
    float *z = (float *)malloc((size_t)L * sizeof(float));
    float *Aj = (float *)malloc((size_t)(npre > 0 ? npre : 1) * sizeof(float));
    float *A = (float *)malloc((size_t)(npre > 0 ? npre : 1) * sizeof(float));
    float *pl = (float *)malloc((size_t)(npre > 0 ? npre : 1) * sizeof(float));
    int64_t *sel = (int64_t *)malloc((size_t)(keep > 0 ? keep : 1) * sizeof(int64_t));
    if (!z || !Aj || !A || !pl || !sel) {
        free(z); free(Aj); free(A); free(pl); free(sel);
        return RKVO_ENOMEM;
    }
    for (int64_t t = 0; t < npre; ++t) A[t] = 0.0f;
    for (int j = 0; j < G; ++j) {
        for (int64_t t = 0; t < npre; ++t) Aj[t] = 0.0f;
        for (int i = 0; i < w; ++i) {
            int64_t qoff = ((int64_t)j * w + i) * d;
            int64_t last = L - w + i; /* causal: keys 0..last */
            float m = -INFINITY;
            for (int64_t t = 0; t <= last; ++t) {
                float dot = 0.0f;
                for (int c = 0; c < d; ++c) {
                    float prod = elem(q_win, dt, qoff + c) * elem(k, dt, t * d + c);
                    dot = dot + prod;
                }
                z[t] = dot * scale;
                if (z[t] > m) m = z[t];
            }
            double acc = 0.0;
            for (int64_t t = 0; t <= last; ++t) acc += (double)expf(z[t] - m);
            float ell = (float)acc;
            for (int64_t t = 0; t < npre; ++t) {
                float p = expf(z[t] - m) / ell;
                Aj[t] = Aj[t] + p;
            }
        }
        for (int64_t t = 0; t < npre; ++t) A[t] = A[t] + Aj[t];
    }
    int64_t half = pool_kernel / 2;
    for (int64_t t = 0; t < npre; ++t) {
        int64_t u0 = t - half < 0 ? 0 : t - half;
        int64_t u1 = t + half > npre - 1 ? npre - 1 : t + half;
        float best = A[u0];
        for (int64_t u = u0 + 1; u <= u1; ++u)
            if (A[u] > best) best = A[u];
        pl[t] = best;
    }
    int rc = topk_ascending(pl, npre, keep - w, sel);
    if (rc == RKVO_OK) {
        for (int64_t q = 0; q < keep - w; ++q) kept[q] = (int32_t)sel[q];
        for (int i = 0; i < w; ++i) kept[keep - w + i] = (int32_t)(L - w + i);
        if (A_out) memcpy(A_out, A, (size_t)npre * sizeof(float));
        if (pooled_out) memcpy(pooled_out, pl, (size_t)npre * sizeof(float));
    }
    free(z); free(Aj); free(A); free(pl); free(sel);
    return rc;
}

/* ---- O4: Hybrid Sparse Attention decode for one KV head group ---------- */
/*
 * [P3] "Where it sits": scores are approximated by a two-dimensional
 * reduction -- SparQ-style top-magnitude channel selection along the head
 * dimension and Quest-style paged max/min summaries along the sequence --
 * giving a per-page bound.  [P3] "Adaptation notes": whole pages are selected
 * (k2 of them).  [P3] "Evidence": the page score bounds every in-page dot
 * product.  [P1]/[P2]: exact attention over the selected tokens.
 *
 * q          : [G][d]    decode queries of the G heads sharing this KV head.
 * k, v       : [n][d]    the (pruned) cache rows.
 * smax, smin : [NP][d]   page summaries (NP = ceil(n/P)), same type as k.
 * Steps:
 *   a[c]   = sum_{j ascending} |q_j[c]|                  (fp32, from +0)
 *   I1     = the k1 best channels by (a desc, c asc), ascending
 *   s_j(p) = sum_{c in I1 ascending} max(fl(q_j[c]*smax[p][c]),
 *                                         fl(q_j[c]*smin[p][c]))   (fp32)
 *   S(p)   = sum_{j ascending} s_j(p)                    (fp32, from +0)
 *   I2     = the min(k2, NP) best pages by (S desc, p asc), ascending
 *   out_j  = softmax_t(scale * q_j . k_t) v_t over the valid rows t of the
 *            pages in I2, evaluated in fp64.
 * chan[k1], pages[k2] (padded with -1), S[NP] (optional), out[G][d] (fp64).
 * n = 0 gives no pages and a zero output.
 */
int rkvo_hsa_group(const void *q, const void *k, const void *v, int dt,
                   const void *smax, const void *smin, int64_t n, int d, int G,
                   int P, int k1, int k2, double scale, int32_t *chan,
                   int32_t *pages, float *S_out, double *out) {
    if (n < 0 || d < 1 || G < 1 || P < 1 || k1 < 1 || k1 > d || k2 < 1) return RKVO_EINVAL;
    int64_t np = (n + P - 1) / P;
    float *a = (float *)malloc((size_t)d * sizeof(float));
    int64_t *ci = (int64_t *)malloc((size_t)k1 * sizeof(int64_t));
    float *S = (float *)malloc((size_t)(np > 0 ? np : 1) * sizeof(float));
    int64_t nsel = np < k2 ? np : k2;
    int64_t *pi = (int64_t *)malloc((size_t)(nsel > 0 ? nsel : 1) * sizeof(int64_t));
    double *sc = (double *)malloc((size_t)(nsel * P > 0 ? nsel * P : 1) * sizeof(double));
    if (!a || !ci || !S || !pi || !sc) {
        free(a); free(ci); free(S); free(pi); free(sc);
        return RKVO_ENOMEM;
    }
    int rc = RKVO_OK;
    /* channels */
    for (int c = 0; c < d; ++c) {
        float acc = 0.0f;
        for (int j = 0; j < G; ++j) acc = acc + fabsf(elem(q, dt, (int64_t)j * d + c));
        a[c] = acc;
    }
    rc = topk_ascending(a, d, k1, ci);
    if (rc != RKVO_OK) goto done;
    for (int i = 0; i < k1; ++i) chan[i] = (int32_t)ci[i];
    /* page scores */
    for (int64_t p = 0; p < np; ++p) {
        float tot = 0.0f;
        for (int j = 0; j < G; ++j) {
            float s = 0.0f;
            for (int i = 0; i < k1; ++i) {
                int64_t c = ci[i];
                float qc = elem(q, dt, (int64_t)j * d + c);
                float hi = qc * elem(smax, dt, p * d + c);
                float lo = qc * elem(smin, dt, p * d + c);
                s = s + (hi > lo ? hi : lo);
            }
            tot = tot + s;
        }
        S[p] = tot;
    }
    if (S_out) memcpy(S_out, S, (size_t)np * sizeof(float));
    /* pages */
    rc = topk_ascending(S, np, nsel, pi);
    if (rc != RKVO_OK) goto done;
    for (int i = 0; i < k2; ++i) pages[i] = i < nsel ? (int32_t)pi[i] : -1;
    /* exact attention over the rows of the selected pages */
    for (int j = 0; j < G; ++j) {
        int64_t nt = 0;
        double m = -INFINITY;
        for (int64_t s = 0; s < nsel; ++s) {
            int64_t r0 = pi[s] * P, r1 = r0 + P < n ? r0 + P : n;
            for (int64_t t = r0; t < r1; ++t) {
                double dot = 0.0;
                for (int c = 0; c < d; ++c)
                    dot += (double)elem(q, dt, (int64_t)j * d + c) * (double)elem(k, dt, t * d + c);
                sc[nt] = dot * scale;
                if (sc[nt] > m) m = sc[nt];
                ++nt;
            }
        }
        double den = 0.0;
        for (int64_t u = 0; u < nt; ++u) den += exp(sc[u] - m);
        for (int c = 0; c < d; ++c) out[(int64_t)j * d + c] = 0.0;
        nt = 0;
        for (int64_t s = 0; s < nsel; ++s) {
            int64_t r0 = pi[s] * P, r1 = r0 + P < n ? r0 + P : n;
            for (int64_t t = r0; t < r1; ++t) {
                double pw = exp(sc[nt] - m) / den;
                for (int c = 0; c < d; ++c)
                    out[(int64_t)j * d + c] += pw * (double)elem(v, dt, t * d + c);
                ++nt;
            }
        }
    }
done:
    free(a); free(ci); free(S); free(pi); free(sc);
    return rc;
}
