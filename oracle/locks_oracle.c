/*
 * Oracle for the decode-step hot path of page-local key summaries.
 * TEST INFRASTRUCTURE ONLY (see locks_oracle.h): plain, slow, double precision.
 *
 * Written from the pages, in their notation:
 *   P_j   tokens of page j, mu_j its centroid, V_j its rank-r basis,
 *   c_i   coefficients of token i, d the head dimension, q the query.
 */
#include "locks_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

#define NTHREADS(n) ((n) > 0 ? (n) : omp_get_max_threads())

/* ------------------------------------------------------------------------ */
/* Log-sum-exp.  The LSE of the reconstructed logits is the page-mass
 * estimate (gist.science technical summary, section 2, subsection
 * Reconstructie en Selectie). */
double orc_lse(int n, const double* x) {
    double m = -INFINITY;
    for (int i = 0; i < n; ++i)
        if (x[i] > m) m = x[i];
    if (m == -INFINITY) return -INFINITY;
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += exp(x[i] - m);
    return m + log(s);
}

static double dot(int n, const double* a, const double* b) {
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += a[i] * b[i];
    return s;
}

/* ------------------------------------------------------------------------ */
/* Step 1: the page-local spectral summary.
 * Section 2, "Pagina-lokale Spectrale Decompositie": when a page is final,
 * a small eigendecomposition of its centred keys (key deviations) is taken;
 * the summary keeps the top-r eigenvectors (the basis) and each token's
 * coefficients.  The centroid mu_j appears in the estimator of the same
 * section.  The eigenvectors of the centred scatter matrix
 * Kc^T Kc are the right singular vectors of Kc, found here by one-sided
 * (Hestenes) Jacobi: pairs of rows of Kc are rotated until all rows are
 * mutually orthogonal; row k then equals sigma_k v_k^T. */
int orc_page_summary(int P, int d, int r, const double* keys, double* mu, double* basis,
                     double* coef, double* sigma) {
    const int nsv = P < d ? P : d;
    if (r < 0 || r > nsv || P <= 0 || d <= 0) return -1;

    /* centroid mu = (1/P) sum_i k_i */
    for (int e = 0; e < d; ++e) {
        double s = 0.0;
        for (int i = 0; i < P; ++i) s += keys[(size_t)i * d + e];
        mu[e] = s / P;
    }
    /* centred keys Kc = K - 1 mu^T, rows w_i */
    double* w = (double*)malloc(sizeof(double) * (size_t)P * d);
    double* kc = (double*)malloc(sizeof(double) * (size_t)P * d);
    int* order = (int*)malloc(sizeof(int) * (size_t)P);
    double* norms = (double*)malloc(sizeof(double) * (size_t)P);
    for (int i = 0; i < P; ++i)
        for (int e = 0; e < d; ++e)
            kc[(size_t)i * d + e] = w[(size_t)i * d + e] = keys[(size_t)i * d + e] - mu[e];

    /* A pair is orthogonal when |w_p . w_q| <= 1e-15 |w_p| |w_q|, or when the
     * coupling is negligible against the block's energy (rows that are
     * numerically null, e.g. beyond rank d when P > d). */
    double fro2 = 0.0;
    for (size_t e = 0; e < (size_t)P * d; ++e) fro2 += w[e] * w[e];
    int sweeps = 0;
    for (; sweeps < 100; ++sweeps) {
        int rotated = 0;
        for (int p = 0; p < P - 1; ++p) {
            for (int q = p + 1; q < P; ++q) {
                double* wp = w + (size_t)p * d;
                double* wq = w + (size_t)q * d;
                const double alpha = dot(d, wp, wp), beta = dot(d, wq, wq);
                const double gamma = dot(d, wp, wq);
                if (gamma == 0.0 || fabs(gamma) <= 1e-15 * sqrt(alpha * beta) ||
                    fabs(gamma) <= 1e-30 * fro2)
                    continue;
                rotated = 1;
                const double zeta = (beta - alpha) / (2.0 * gamma);
                const double t = (zeta >= 0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
                const double c = 1.0 / sqrt(1.0 + t * t), s = c * t;
                for (int e = 0; e < d; ++e) {
                    const double a = wp[e], b = wq[e];
                    wp[e] = c * a - s * b;
                    wq[e] = s * a + c * b;
                }
            }
        }
        if (!rotated) break;
    }

    /* sort rows by norm (the singular values), descending; ties by index */
    for (int i = 0; i < P; ++i) {
        norms[i] = sqrt(dot(d, w + (size_t)i * d, w + (size_t)i * d));
        order[i] = i;
    }
    for (int i = 1; i < P; ++i) {
        const int oi = order[i];
        int k = i;
        while (k > 0 && norms[order[k - 1]] < norms[oi]) {
            order[k] = order[k - 1];
            --k;
        }
        order[k] = oi;
    }
    for (int k = 0; k < nsv; ++k) sigma[k] = norms[order[k]];

    /* basis row k = v_k = w_(k) / sigma_k; coefficient c_i[k] = v_k . (k_i - mu) */
    const double tiny = 1e-13 * (nsv > 0 ? sigma[0] : 0.0);
    for (int k = 0; k < r; ++k) {
        double* vk = basis + (size_t)k * d;
        const double s = sigma[k];
        const int null_dir = !(s > tiny);
        for (int e = 0; e < d; ++e) vk[e] = null_dir ? 0.0 : w[(size_t)order[k] * d + e] / s;
        for (int i = 0; i < P; ++i)
            coef[(size_t)i * r + k] = null_dir ? 0.0 : dot(d, vk, kc + (size_t)i * d);
    }
    free(w);
    free(kc);
    free(order);
    free(norms);
    return sweeps;
}

/* ------------------------------------------------------------------------ */
/* Step 2: reconstructed within-page logits and their LSE,
 *   s_j(q) = log sum_{i in P_j} exp((q^T mu_j + (V_j^T q)^T c_i) / sqrt(d))
 * (section 2, "Reconstructie en Selectie", displayed equation).  No key or
 * value of the page is read: only mu_j, V_j and the c_i. */
double orc_page_estimate(int P, int d, int r, const double* q, const double* mu,
                         const double* basis, const double* coef) {
    double* t = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
    double* logit = (double*)malloc(sizeof(double) * (size_t)P);
    for (int k = 0; k < r; ++k) t[k] = dot(d, basis + (size_t)k * d, q); /* V_j^T q */
    const double qmu = dot(d, q, mu);
    const double scale = 1.0 / sqrt((double)d);
    for (int i = 0; i < P; ++i) logit[i] = (qmu + dot(r, t, coef + (size_t)i * r)) * scale;
    const double s = orc_lse(P, logit);
    free(t);
    free(logit);
    return s;
}

/* The quantity the estimate stands in for: the exact LSE of the page's
 * true logits, as used by the exact-LSE selection that reads every key
 * (abstract; section 3, subsection Retrieval en QA). */
double orc_page_exact_lse(int n, int d, const double* q, const double* keys) {
    double* logit = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    const double scale = 1.0 / sqrt((double)d);
    for (int i = 0; i < n; ++i) logit[i] = dot(d, q, keys + (size_t)i * d) * scale;
    const double s = orc_lse(n, logit);
    free(logit);
    return s;
}

/* ------------------------------------------------------------------------ */
/* Step 3a: rank pages by estimated mass and keep the top ones (section 2,
 * subsection Reconstructie en Selectie; abstract).
 * Readings: larger mass first; equal fp32 values go to the lower page index;
 * the k winners are reported in ascending page order. */
typedef struct {
    float mass;
    int32_t page;
} ranked_t;

static int cmp_rank(const void* a, const void* b) {
    const ranked_t* x = (const ranked_t*)a;
    const ranked_t* y = (const ranked_t*)b;
    if (x->mass > y->mass) return -1;
    if (x->mass < y->mass) return 1;
    return (x->page > y->page) - (x->page < y->page);
}

static int cmp_page(const void* a, const void* b) {
    const ranked_t* x = (const ranked_t*)a;
    const ranked_t* y = (const ranked_t*)b;
    return (x->page > y->page) - (x->page < y->page);
}

int orc_select_topk(int n, const float* mass, int k, int width, int32_t* sel, float* sel_mass) {
    if (k < 0) k = 0;
    if (k > n) k = n;
    if (k > width) k = width;
    ranked_t* all = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)(n > 0 ? n : 1));
    for (int j = 0; j < n; ++j) {
        all[j].mass = mass[j];
        all[j].page = j;
    }
    qsort(all, (size_t)n, sizeof(ranked_t), cmp_rank);
    qsort(all, (size_t)k, sizeof(ranked_t), cmp_page);
    for (int s = 0; s < width; ++s) {
        sel[s] = s < k ? all[s].page : -1;
        if (sel_mass) sel_mass[s] = s < k ? all[s].mass : -INFINITY;
    }
    free(all);
    return k;
}

/* ------------------------------------------------------------------------ */
/* Step 3b: softmax attention over the attended tokens only (abstract).
 * Reading: the softmax is renormalised over the attended set. */
void orc_attend_tokens(int n, int d, const double* q, const double* keys, const double* vals,
                       double* out, double* lse) {
    for (int e = 0; e < d; ++e) out[e] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }
    double* s = (double*)calloc((size_t)n, sizeof(double));
    const double scale = 1.0 / sqrt((double)d);
    for (int i = 0; i < n; ++i) s[i] = dot(d, q, keys + (size_t)i * d) * scale;
    const double L = orc_lse(n, s);
    for (int i = 0; i < n; ++i) {
        const double p = exp(s[i] - L);
        for (int e = 0; e < d; ++e) out[e] += p * vals[(size_t)i * d + e];
    }
    *lse = L;
    free(s);
}

/* ------------------------------------------------------------------------ */
/* Paged-cache drivers. */

static int layout_ok(const orc_layout* L) {
    return L && L->batch > 0 && L->num_q_heads > 0 && L->num_kv_heads > 0 &&
           L->num_q_heads % L->num_kv_heads == 0 && L->head_dim > 0 && L->page_size > 0 &&
           L->max_pages >= 0 && L->block_table && L->seq_lens;
}

static int full_pages(const orc_layout* L, int b) { return L->seq_lens[b] / L->page_size; }

/* Pages of sequence b that compete for the budget: the full pages whose
 * summaries exist (all full pages when no count is given). */
static int candidate_pages(const orc_layout* L, int b) {
    const int full = full_pages(L, b);
    if (!L->summarized) return full;
    const int s = L->summarized[b] < 0 ? 0 : L->summarized[b];
    return s < full ? s : full;
}

static int all_pages(const orc_layout* L, int b) {
    return (L->seq_lens[b] + L->page_size - 1) / L->page_size;
}

/* Widen n floats at src into dst (double). */
static void widen(size_t n, const float* src, double* dst) {
    for (size_t i = 0; i < n; ++i) dst[i] = (double)src[i];
}

/* Keys of logical page j of (b, g), widened. */
static const float* page_ptr(const orc_layout* L, const float* pool, int b, int g, int j) {
    const int32_t phys = L->block_table[(size_t)b * L->max_pages + j];
    return pool + ((size_t)phys * L->num_kv_heads + g) * (size_t)L->page_size * L->head_dim;
}

int orc_build_units(const orc_layout* L, int r, const float* k_pool, int n, const int32_t* ub,
                    const int32_t* ug, const int32_t* uj, double* mu, double* basis, double* coef,
                    double* sigma, int nthreads) {
    if (!layout_ok(L)) return -1;
    const int P = L->page_size, d = L->head_dim, nsv = P < d ? P : d;
    if (r < 0 || r > nsv) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(NTHREADS(nthreads))
    for (int u = 0; u < n; ++u) {
        if (ub[u] < 0 || ub[u] >= L->batch || ug[u] < 0 || ug[u] >= L->num_kv_heads ||
            uj[u] < 0 || uj[u] >= full_pages(L, ub[u])) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        double* keys = (double*)malloc(sizeof(double) * (size_t)P * d);
        widen((size_t)P * d, page_ptr(L, k_pool, ub[u], ug[u], uj[u]), keys);
        orc_page_summary(P, d, r, keys, mu + (size_t)u * d, basis + (size_t)u * r * d,
                         coef + (size_t)u * P * r, sigma + (size_t)u * nsv);
        free(keys);
    }
    return bad ? -1 : 0;
}

int orc_build_pool(const orc_layout* L, int r, const float* k_pool, float* mu, float* basis,
                   float* coef, double* sigma_out, int nthreads) {
    if (!layout_ok(L)) return -1;
    const int P = L->page_size, d = L->head_dim, H = L->num_kv_heads, nsv = P < d ? P : d;
    if (r < 0 || r > nsv) return -1;
    /* flatten (b, j, g) over full pages */
    int64_t total = 0;
    for (int b = 0; b < L->batch; ++b) total += (int64_t)full_pages(L, b) * H;
#pragma omp parallel num_threads(NTHREADS(nthreads))
    {
        double* keys = (double*)malloc(sizeof(double) * (size_t)P * d);
        double* m = (double*)malloc(sizeof(double) * (size_t)d);
        double* v = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1) * d);
        double* c = (double*)malloc(sizeof(double) * (size_t)P * (r > 0 ? r : 1));
        double* s = (double*)malloc(sizeof(double) * (size_t)nsv);
#pragma omp for schedule(dynamic, 4)
        for (int64_t u = 0; u < total; ++u) {
            int64_t rem = u / H;
            const int g = (int)(u % H);
            int b = 0;
            while (rem >= full_pages(L, b)) rem -= full_pages(L, b++);
            const int j = (int)rem;
            widen((size_t)P * d, page_ptr(L, k_pool, b, g, j), keys);
            orc_page_summary(P, d, r, keys, m, v, c, s);
            const size_t unit = (size_t)L->block_table[(size_t)b * L->max_pages + j] * H + g;
            for (int e = 0; e < d; ++e) mu[unit * d + e] = (float)m[e];
            for (int e = 0; e < r * d; ++e) basis[unit * r * d + e] = (float)v[e];
            for (int e = 0; e < P * r; ++e) coef[unit * P * r + e] = (float)c[e];
            if (sigma_out)
                for (int e = 0; e < nsv; ++e) sigma_out[unit * nsv + e] = s[e];
        }
        free(keys);
        free(m);
        free(v);
        free(c);
        free(s);
    }
    return 0;
}

/* Estimates of one unit for every head of the group, and their aggregate.
 * Reading for Group-Shared Selection (section 2, "Group-Shared Selection"):
 * the group's shared score is the LSE over its heads of the per-head
 * estimates (the summed unnormalised mass); head h is in group h / G. */
static double scan_unit(const orc_layout* L, int r, const float* q, const float* mu,
                        const float* basis, const float* coef, int b, int g, int j,
                        double* head_out) {
    const int P = L->page_size, d = L->head_dim, H = L->num_kv_heads;
    const int G = L->num_q_heads / H;
    const size_t unit = (size_t)L->block_table[(size_t)b * L->max_pages + j] * H + g;
    double* m = (double*)malloc(sizeof(double) * (size_t)d);
    double* v = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1) * d);
    double* c = (double*)malloc(sizeof(double) * (size_t)P * (r > 0 ? r : 1));
    double* qh = (double*)malloc(sizeof(double) * (size_t)d);
    double* est = (double*)malloc(sizeof(double) * (size_t)G);
    widen((size_t)d, mu + unit * d, m);
    widen((size_t)r * d, basis + unit * r * d, v);
    widen((size_t)P * r, coef + unit * P * r, c);
    for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        widen((size_t)d, q + ((size_t)b * L->num_q_heads + h) * d, qh);
        est[hh] = orc_page_estimate(P, d, r, qh, m, v, c);
        if (head_out) head_out[hh] = est[hh];
    }
    const double a = orc_lse(G, est);
    free(m);
    free(v);
    free(c);
    free(qh);
    free(est);
    return a;
}

int orc_scan_units(const orc_layout* L, int r, const float* q, const float* mu,
                   const float* basis, const float* coef, int n, const int32_t* ub,
                   const int32_t* ug, const int32_t* uj, double* head_mass, double* page_mass) {
    if (!layout_ok(L)) return -1;
    const int G = L->num_q_heads / L->num_kv_heads;
    for (int u = 0; u < n; ++u) {
        if (ub[u] < 0 || ub[u] >= L->batch || ug[u] < 0 || ug[u] >= L->num_kv_heads ||
            uj[u] < 0 || uj[u] >= candidate_pages(L, ub[u]))
            return -1;
        const double a = scan_unit(L, r, q, mu, basis, coef, ub[u], ug[u], uj[u],
                                   head_mass ? head_mass + (size_t)u * G : NULL);
        if (page_mass) page_mass[u] = a;
    }
    return 0;
}

int orc_scan_pool(const orc_layout* L, int r, const float* q, const float* mu,
                  const float* basis, const float* coef, double* head_mass, double* page_mass,
                  int nthreads) {
    if (!layout_ok(L)) return -1;
    const int H = L->num_kv_heads, G = L->num_q_heads / H, MP = L->max_pages;
    const int64_t units = (int64_t)L->batch * H * MP;
#pragma omp parallel for schedule(dynamic, 64) num_threads(NTHREADS(nthreads))
    for (int64_t u = 0; u < units; ++u) {
        const int j = (int)(u % MP), g = (int)((u / MP) % H), b = (int)(u / ((int64_t)MP * H));
        double est[1024];
        double a = -INFINITY;
        if (j < candidate_pages(L, b)) {
            a = scan_unit(L, r, q, mu, basis, coef, b, g, j, est);
        } else {
            for (int hh = 0; hh < G; ++hh) est[hh] = -INFINITY;
        }
        if (page_mass) page_mass[u] = a;
        if (head_mass)
            for (int hh = 0; hh < G; ++hh)
                head_mass[((size_t)b * L->num_q_heads + g * G + hh) * MP + j] = est[hh];
    }
    return 0;
}

int orc_share_pool(const orc_layout* L, const double* head_mass, double* page_share) {
    if (!layout_ok(L)) return -1;
    const int H = L->num_kv_heads, Hq = L->num_q_heads, G = Hq / H, MP = L->max_pages;
    double* z = (double*)malloc(sizeof(double) * (size_t)Hq);
    double* terms = (double*)malloc(sizeof(double) * (size_t)G);
    if (!z || !terms) {
        free(z);
        free(terms);
        return -1;
    }
    for (int b = 0; b < L->batch; ++b) {
        const int full = candidate_pages(L, b);
        /* each head's total estimated mass over the sequence's candidate pages */
        for (int h = 0; h < Hq; ++h) z[h] = orc_lse(full, head_mass + ((size_t)b * Hq + h) * MP);
        for (int g = 0; g < H; ++g)
            for (int j = 0; j < MP; ++j) {
                double v = -INFINITY;
                if (j < full) {
                    for (int hh = 0; hh < G; ++hh) {
                        const int h = g * G + hh;
                        terms[hh] = head_mass[((size_t)b * Hq + h) * MP + j] - z[h];
                    }
                    v = orc_lse(G, terms) - log((double)G); /* log of the mean share */
                }
                page_share[((size_t)b * H + g) * MP + j] = v;
            }
    }
    free(z);
    free(terms);
    return 0;
}

int orc_exact_pool(const orc_layout* L, const float* q, const float* k_pool, double* head_lse,
                   double* page_lse, int nthreads) {
    if (!layout_ok(L)) return -1;
    const int P = L->page_size, d = L->head_dim, H = L->num_kv_heads;
    const int G = L->num_q_heads / H, MP = L->max_pages;
    const int64_t units = (int64_t)L->batch * H * MP;
#pragma omp parallel for schedule(dynamic, 64) num_threads(NTHREADS(nthreads))
    for (int64_t u = 0; u < units; ++u) {
        const int j = (int)(u % MP), g = (int)((u / MP) % H), b = (int)(u / ((int64_t)MP * H));
        double est[1024];
        const int n_tok = j < all_pages(L, b)
                              ? (L->seq_lens[b] - j * P < P ? L->seq_lens[b] - j * P : P)
                              : 0;
        double* keys = (double*)malloc(sizeof(double) * (size_t)P * d);
        double* qh = (double*)malloc(sizeof(double) * (size_t)d);
        if (n_tok > 0) widen((size_t)n_tok * d, page_ptr(L, k_pool, b, g, j), keys);
        for (int hh = 0; hh < G; ++hh) {
            const int h = g * G + hh;
            widen((size_t)d, q + ((size_t)b * L->num_q_heads + h) * d, qh);
            est[hh] = orc_page_exact_lse(n_tok, d, qh, keys);
            if (head_lse) head_lse[((size_t)b * L->num_q_heads + h) * MP + j] = est[hh];
        }
        if (page_lse) page_lse[u] = orc_lse(G, est);
        free(keys);
        free(qh);
    }
    return 0;
}

/* Reading for the token budget: k = floor(budget / P) pages, never more than
 * the sequence's full pages; a budget below one page selects nothing. */
int orc_select_pool(const orc_layout* L, int budget_tokens, const float* page_mass, int width,
                    int32_t* sel_pages, float* sel_mass) {
    if (!layout_ok(L) || budget_tokens < 0 || width < 0) return -1;
    const int H = L->num_kv_heads, MP = L->max_pages;
    const int k = budget_tokens / L->page_size;
    for (int b = 0; b < L->batch; ++b)
        for (int g = 0; g < H; ++g) {
            const size_t row = (size_t)b * H + g;
            orc_select_topk(candidate_pages(L, b), page_mass + row * MP, k, width,
                            sel_pages + row * width, sel_mass ? sel_mass + row * width : NULL);
        }
    return 0;
}

/* Reading for the partial last page: it has no summary yet (summaries are
 * made when a page is final, section 2), so it is never a candidate and is
 * always attended; so is every full page whose summary does not exist yet
 * (pages from candidate_pages(b) on). */
int orc_attend_pool(const orc_layout* L, const float* q, const float* k_pool,
                    const float* v_pool, const int32_t* sel_pages, int width, double* out,
                    double* lse, int nthreads) {
    if (!layout_ok(L)) return -1;
    const int P = L->page_size, d = L->head_dim, H = L->num_kv_heads;
    const int Hq = L->num_q_heads, G = Hq / H;
    const int64_t rows = (int64_t)L->batch * Hq;
#pragma omp parallel for schedule(dynamic, 1) num_threads(NTHREADS(nthreads))
    for (int64_t bh = 0; bh < rows; ++bh) {
        const int b = (int)(bh / Hq), h = (int)(bh % Hq), g = h / G;
        const int cand = candidate_pages(L, b), np = all_pages(L, b);
        /* the attended pages: the listed candidates, then every page without a
         * summary (unsummarised full pages and the partial last page) */
        int32_t* pages = (int32_t*)malloc(sizeof(int32_t) * (size_t)(np + width > 0 ? np + width : 1));
        int n_pages = 0;
        if (sel_pages) {
            const int32_t* s = sel_pages + ((size_t)b * H + g) * width;
            for (int t = 0; t < width; ++t)
                if (s[t] >= 0 && s[t] < cand) pages[n_pages++] = s[t];
            for (int j = cand; j < np; ++j) pages[n_pages++] = j;
        } else {
            for (int j = 0; j < np; ++j) pages[n_pages++] = j;
        }
        double* qh = (double*)malloc(sizeof(double) * (size_t)d);
        widen((size_t)d, q + (size_t)bh * d, qh);
        /* pass 1: logits of every attended token, and their LSE */
        int n_tok = 0;
        for (int t = 0; t < n_pages; ++t) {
            const int j = pages[t];
            n_tok += L->seq_lens[b] - j * P < P ? L->seq_lens[b] - j * P : P;
        }
        double* logit = (double*)malloc(sizeof(double) * (size_t)(n_tok > 0 ? n_tok : 1));
        const double scale = 1.0 / sqrt((double)d);
        int idx = 0;
        for (int t = 0; t < n_pages; ++t) {
            const int j = pages[t];
            const int valid = L->seq_lens[b] - j * P < P ? L->seq_lens[b] - j * P : P;
            const float* kp = page_ptr(L, k_pool, b, g, j);
            for (int i = 0; i < valid; ++i) {
                double sdot = 0.0;
                for (int e = 0; e < d; ++e) sdot += qh[e] * (double)kp[(size_t)i * d + e];
                logit[idx++] = sdot * scale;
            }
        }
        const double Lse = orc_lse(n_tok, logit);
        /* pass 2: out = sum_i exp(logit_i - LSE) v_i */
        double* o = out + (size_t)bh * d;
        for (int e = 0; e < d; ++e) o[e] = 0.0;
        idx = 0;
        for (int t = 0; t < n_pages; ++t) {
            const int j = pages[t];
            const int valid = L->seq_lens[b] - j * P < P ? L->seq_lens[b] - j * P : P;
            const float* vp = page_ptr(L, v_pool, b, g, j);
            for (int i = 0; i < valid; ++i) {
                const double p = exp(logit[idx++] - Lse);
                for (int e = 0; e < d; ++e) o[e] += p * (double)vp[(size_t)i * d + e];
            }
        }
        if (lse) lse[bh] = n_tok > 0 ? Lse : -INFINITY;
        free(pages);
        free(qh);
        free(logit);
    }
    return 0;
}

/* ---------------- shared-basis sketch (ablation baseline) ---------------- */

int orc_pooled_covariance(const orc_layout* L, const float* k_pool, double* cov, int nthreads) {
    if (!layout_ok(L)) return -1;
    const int P = L->page_size, d = L->head_dim, H = L->num_kv_heads;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    for (int g = 0; g < H; ++g) {
        double* C = cov + (size_t)g * d * d;
        memset(C, 0, sizeof(double) * (size_t)d * d);
        for (int b = 0; b < L->batch; ++b) {
            const int nf = full_pages(L, b) < L->max_pages ? full_pages(L, b) : L->max_pages;
            #pragma omp parallel
            {
                double* part = (double*)calloc((size_t)d * d, sizeof(double));
                double* kc = (double*)malloc(sizeof(double) * (size_t)P * d);
                double* mu = (double*)malloc(sizeof(double) * (size_t)d);
                #pragma omp for schedule(static)
                for (int j = 0; j < nf; ++j) {
                    const float* k = page_ptr(L, k_pool, b, g, j);
                    for (int e = 0; e < d; ++e) {
                        double acc = 0.0;
                        for (int i = 0; i < P; ++i) acc += k[(size_t)i * d + e];
                        mu[e] = acc / P;
                    }
                    for (int i = 0; i < P; ++i)
                        for (int e = 0; e < d; ++e) kc[(size_t)i * d + e] = k[(size_t)i * d + e] - mu[e];
                    for (int i = 0; i < P; ++i)
                        for (int x = 0; x < d; ++x) {
                            const double a = kc[(size_t)i * d + x];
                            for (int y = 0; y < d; ++y) part[(size_t)x * d + y] += a * kc[(size_t)i * d + y];
                        }
                }
                #pragma omp critical
                for (size_t e = 0; e < (size_t)d * d; ++e) C[e] += part[e];
                free(part);
                free(kc);
                free(mu);
            }
        }
    }
    return 0;
}

int orc_sketch_pool(const orc_layout* L, int rho, const float* k_pool, const double* basis,
                    float* mu_out, float* coef_out, int nthreads) {
    if (!layout_ok(L) || rho <= 0 || L->head_dim > 1024) return -1;
    const int P = L->page_size, d = L->head_dim, H = L->num_kv_heads;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    for (int b = 0; b < L->batch; ++b) {
        const int nf = full_pages(L, b) < L->max_pages ? full_pages(L, b) : L->max_pages;
        #pragma omp parallel for collapse(2) schedule(static)
        for (int j = 0; j < nf; ++j)
            for (int g = 0; g < H; ++g) {
                const float* k = page_ptr(L, k_pool, b, g, j);
                const size_t unit = (size_t)L->block_table[(size_t)b * L->max_pages + j] * H + g;
                double mu[1024];
                for (int e = 0; e < d; ++e) {
                    double acc = 0.0;
                    for (int i = 0; i < P; ++i) acc += k[(size_t)i * d + e];
                    mu[e] = acc / P;
                    mu_out[unit * d + e] = (float)mu[e];
                }
                const double* V = basis + (size_t)g * rho * d;
                for (int i = 0; i < P; ++i)
                    for (int t = 0; t < rho; ++t) {
                        double acc = 0.0;
                        for (int e = 0; e < d; ++e) acc += (k[(size_t)i * d + e] - mu[e]) * V[(size_t)t * d + e];
                        coef_out[(unit * P + i) * rho + t] = (float)acc;
                    }
            }
    }
    return 0;
}

/* ---------------- quantised summaries (section 2, "Kwantisatie") ---------------- */

void orc_quantize_vec(int n, int stride, const float* x, int qmax, float* scale, int8_t* code) {
    float m = 0.0f;
    for (int i = 0; i < n; ++i) {
        const float a = fabsf(x[(size_t)i * stride]);
        if (a > m) m = a;
    }
    const float s = m / (float)qmax;
    *scale = s;
    for (int i = 0; i < n; ++i) {
        int c = 0;
        if (s > 0.0f) {
            const float y = rintf(x[(size_t)i * stride] / s);  /* ties to even */
            c = (int)y;
            if (c > qmax) c = qmax;
            if (c < -qmax) c = -qmax;
        }
        code[(size_t)i * stride] = (int8_t)c;
    }
}

int orc_quantize_pool(int num_blocks, int num_kv_heads, int P, int d, int r, const float* mu,
                      const float* basis, const float* coef, int8_t* mu_q, uint8_t* basis_q,
                      int8_t* coef_q, float* scales) {
    if (num_blocks < 0 || num_kv_heads <= 0 || P <= 0 || d <= 0 || d % 2 || r <= 0) return -1;
    int8_t* row = (int8_t*)malloc((size_t)d);
    if (!row) return -1;
    const size_t units = (size_t)num_blocks * num_kv_heads;
    for (size_t u = 0; u < units; ++u) {
        float* sc = scales + u * (size_t)(1 + 2 * r);
        orc_quantize_vec(d, 1, mu + u * d, 127, &sc[0], mu_q + u * d);
        for (int k = 0; k < r; ++k) {
            orc_quantize_vec(d, 1, basis + (u * r + k) * d, 7, &sc[1 + k], row);
            uint8_t* out = basis_q + (u * r + k) * (size_t)(d / 2);
            for (int t = 0; t < d / 2; ++t)
                out[t] = (uint8_t)(((uint8_t)row[2 * t] & 0x0F) | (((uint8_t)row[2 * t + 1] & 0x0F) << 4));
        }
        for (int k = 0; k < r; ++k)
            orc_quantize_vec(P, r, coef + u * (size_t)P * r + k, 127, &sc[1 + r + k],
                             coef_q + u * (size_t)P * r + k);
    }
    free(row);
    return 0;
}

static int nibble(uint8_t byte, int hi) {
    const int v = hi ? (byte >> 4) : (byte & 0x0F);
    return v >= 8 ? v - 16 : v;
}

int orc_dequantize_pool(int num_blocks, int num_kv_heads, int P, int d, int r,
                        const int8_t* mu_q, const uint8_t* basis_q, const int8_t* coef_q,
                        const float* scales, float* mu, float* basis, float* coef) {
    if (num_blocks < 0 || num_kv_heads <= 0 || P <= 0 || d <= 0 || d % 2 || r <= 0) return -1;
    const size_t units = (size_t)num_blocks * num_kv_heads;
    for (size_t u = 0; u < units; ++u) {
        const float* sc = scales + u * (size_t)(1 + 2 * r);
        for (int i = 0; i < d; ++i) mu[u * d + i] = (float)((double)sc[0] * mu_q[u * d + i]);
        for (int k = 0; k < r; ++k)
            for (int i = 0; i < d; ++i)
                basis[(u * r + k) * d + i] = (float)((double)sc[1 + k] *
                    nibble(basis_q[(u * r + k) * (size_t)(d / 2) + i / 2], i & 1));
        for (int t = 0; t < P; ++t)
            for (int k = 0; k < r; ++k)
                coef[(u * P + t) * r + k] =
                    (float)((double)sc[1 + r + k] * coef_q[(u * P + t) * r + k]);
    }
    return 0;
}
