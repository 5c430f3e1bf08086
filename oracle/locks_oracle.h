/*
 * Oracle for the decode-step hot path of page-local key summaries ("LOCKS:
 * Page-Local Compact Key Summaries for Efficient Long-Context Decoding",
 * arXiv 2607.24555).
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, double-precision CPU
 * implementation used to check the GPU library.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the GPU
 * library never does, and the two share no code.
 *
 * Passages followed (page = the gist.science technical summary unless noted):
 *   centred keys, centroid, top-r eigenvectors, per-token coefficients:
 *       section 2, "Pagina-lokale Spectrale Decompositie";
 *   reconstructed within-page logit estimate s_j(q): section 2,
 *       "Reconstructie en Selectie", the displayed equation;
 *   LSE page mass, ranking, no candidate K/V read: same subsection, and the
 *       English abstract (insight.aitobox.com page, "Abstract");
 *   exact-LSE selection that reads every key: abstract, and section 3
 *       "Retrieval en QA";
 *   attention over the top pages only: abstract;
 *   stored summary precision (int4 basis, int8 coefficients and centroid):
 *       section 2, "Kwantisatie".
 * Readings where the pages are silent (all stated again at each function):
 *   GQA aggregation is the LSE over the group's heads; head h belongs to
 *   KV group h / G; k = min(floor(budget / P), full pages); ties go to the
 *   lowest page index; output in ascending page order; the partial last page
 *   of a sequence has no summary, is never a candidate and is always
 *   attended; attention renormalises over the attended tokens.
 *
 * Parity pins: every function here is checked against closed forms, special
 * cases and library routines in tests/test_oracle_pins.py.
 */
#ifndef LOCKS_ORACLE_H
#define LOCKS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------- single-page / single-vector primitives ---------------- */

/* log(sum_i exp(x_i)), max-shifted; -inf for n == 0 or all -inf. */
double orc_lse(int n, const double* x);

/*
 * Summary of one page (P tokens x d): centroid mu (d), basis (r x d, row k =
 * k-th eigenvector of the centred keys' scatter matrix, largest first),
 * coef (P x r, coef[i][k] = basis_k . (key_i - mu)), sigma (min(P, d)
 * singular values of the centred key block, descending).  The eigenvectors
 * come from a one-sided (Hestenes) Jacobi SVD of the centred block.
 * Directions with sigma <= 1e-13 * sigma_0 are numerically null: their basis
 * row and coefficient column are written as zero.
 * Returns the number of Jacobi sweeps, or -1 for r < 0 or r > min(P, d).
 * (r = 0 is accepted: the summary is the centroid alone.)
 */
int orc_page_summary(int P, int d, int r, const double* keys, double* mu, double* basis,
                     double* coef, double* sigma);

/* Reconstructed within-page estimate
 *   s_j(q) = log sum_i exp((q.mu + (V^T q).c_i) / sqrt(d))
 * (section 2 "Reconstructie en Selectie", displayed equation). */
double orc_page_estimate(int P, int d, int r, const double* q, const double* mu,
                         const double* basis, const double* coef);

/* Exact page LSE: log sum_{i < n} exp(q.k_i / sqrt(d)). */
double orc_page_exact_lse(int n, int d, const double* q, const double* keys);

/*
 * Top-k page choice for one (sequence, KV group) from fp32 masses a[0..n):
 * the k largest values, equal values ordered by ascending index; returned in
 * ascending page order in sel[0..k), with their masses.  Slots k..width-1
 * are padded with -1 / -inf.  k is clamped to [0, n].  Returns k.
 */
int orc_select_topk(int n, const float* mass, int k, int width, int32_t* sel, float* sel_mass);

/* Softmax attention of one query over n tokens (scale 1/sqrt(d)):
 * out = sum_i softmax_i v_i, lse = log sum_i exp(q.k_i / sqrt(d)).
 * n == 0: out = 0, lse = -inf. */
void orc_attend_tokens(int n, int d, const double* q, const double* keys, const double* vals,
                       double* out, double* lse);

/* ---------------- paged-cache drivers ---------------- */

/* The paged layout shared with the GPU library (plain arrays, host memory):
 *   q            [B][Hq][d] float
 *   k/v pools    [NB][Hkv][P][d] float (bf16 inputs widened exactly)
 *   block_table  [B][max_pages] int32, logical page -> physical block
 *   seq_lens     [B] int32
 *   summaries    mu [NB][Hkv][d], basis [NB][Hkv][r][d], coef [NB][Hkv][P][r]
 * Full pages of sequence b: j < seq_lens[b] / P. */
typedef struct {
    int32_t batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages;
    const int32_t* block_table;
    const int32_t* seq_lens;
    /* Nullable [B]: the leading pages of each sequence whose summaries exist.
     * Reading (technical summary, section 2: a page's summary is made once
     * the page is final, off the attention's critical path): only pages
     * j < min(summarized[b], seq_lens[b] / P) are candidates for selection;
     * full pages from there on have no summary yet and are attended like
     * the partial last page, outside the budget.  NULL: every full page. */
    const int32_t* summarized;
} orc_layout;

/* Summaries of every full page, written (rounded to float) at its physical
 * block; blocks of partial pages are left untouched.  sigma_out (nullable,
 * [NB][Hkv][min(P,d)] double) receives each unit's singular values of the
 * centred keys, descending.  Returns 0 or -1. */
int orc_build_pool(const orc_layout* L, int r, const float* k_pool, float* mu, float* basis,
                   float* coef, double* sigma_out, int nthreads);

/* Double-precision summaries of n listed units (b, g, j) into dense arrays
 * mu [n][d], basis [n][r][d], coef [n][P][r], sigma [n][min(P,d)]. */
int orc_build_units(const orc_layout* L, int r, const float* k_pool, int n, const int32_t* ub,
                    const int32_t* ug, const int32_t* uj, double* mu, double* basis, double* coef,
                    double* sigma, int nthreads);

/* Summary scan: per-head estimates head_mass [B][Hq][max_pages] and the
 * group masses page_mass [B][Hkv][max_pages] = LSE over the group's heads.
 * Entries of non-full pages are -inf.  Either output may be NULL. */
int orc_scan_pool(const orc_layout* L, int r, const float* q, const float* mu,
                  const float* basis, const float* coef, double* head_mass, double* page_mass,
                  int nthreads);

/* The same for n listed units (b, g, j): head_mass [n][G], page_mass [n]. */
int orc_scan_units(const orc_layout* L, int r, const float* q, const float* mu,
                   const float* basis, const float* coef, int n, const int32_t* ub,
                   const int32_t* ug, const int32_t* uj, double* head_mass, double* page_mass);

/* Mean-of-share group score (technical summary, section 2, Group-Shared
 * Selection: the heads' estimated mass shares are averaged over the group
 * into one table).  For every (b, g) and full page j:
 *   share_{j,h} = exp(s_{j,h} - Z_h),  Z_h = LSE over the full pages j' of s_{j',h},
 *   page_share[b][g][j] = log( (1/G) sum_{h in g} share_{j,h} ),
 * from per-head estimates head_mass [B][Hq][max_pages] (as orc_scan_pool
 * writes them).  Entries of pages that are not full are -inf. */
int orc_share_pool(const orc_layout* L, const double* head_mass, double* page_share);

/* Exact ("read every key") page masses: head_lse [B][Hq][max_pages] over every
 * page including a partial last one, page_lse [B][Hkv][max_pages] = LSE over
 * the group's heads; -inf past the last page.  Either output may be NULL. */
int orc_exact_pool(const orc_layout* L, const float* q, const float* k_pool, double* head_lse,
                   double* page_lse, int nthreads);

/* Selection for every (b, g) from fp32 group masses [B][Hkv][max_pages]:
 * k_b = min(floor(budget_tokens / P), full pages of b) winners in ascending
 * order in sel_pages [B][Hkv][width], padded with -1 / -inf. */
int orc_select_pool(const orc_layout* L, int budget_tokens, const float* page_mass, int width,
                    int32_t* sel_pages, float* sel_mass);

/* Attention per (b, h) over the tokens of the listed logical pages of its
 * group (sel_pages [B][Hkv][width], -1 = unused) plus the partial last page,
 * or over every token when sel_pages is NULL (dense).
 * out [B][Hq][d], lse [B][Hq] (lse may be NULL). */
int orc_attend_pool(const orc_layout* L, const float* q, const float* k_pool,
                    const float* v_pool, const int32_t* sel_pages, int width, double* out,
                    double* lse, int nthreads);

/* ---------------- shared-basis sketch (ablation baseline) ----------------
 * The pages argue that a query-independent projection shared by every page
 * is blind to page-specific directions (technical summary, section 3, the
 * proposition on a shared rank-rho projection; the abstract's contrast with
 * fixed sketches).  The baseline built to measure that: one rank-rho basis
 * per KV head, the top rho eigenvectors of the pooled within-page covariance
 * sum_j Kc_j^T Kc_j over every full page j (Kc_j = the page's keys minus its
 * centroid); every page keeps its centroid and its tokens' coordinates in the
 * shared basis, and is scored with the same estimator.  At rho =
 * r (1 + d / P) it stores as many values per page as a rank-r page summary. */

/* Pooled within-page covariance cov [Hkv][d][d] over every full page. */
int orc_pooled_covariance(const orc_layout* L, const float* k_pool, double* cov, int nthreads);

/* Centroids and shared-basis coordinates of every full page: mu [NB][Hkv][d],
 * coef [NB][Hkv][P][rho] = (k_i - mu) . basis_k, basis [Hkv][rho][d]. */
int orc_sketch_pool(const orc_layout* L, int rho, const float* k_pool, const double* basis,
                    float* mu, float* coef, int nthreads);

/* ---------------- quantised summaries ----------------
 * Stored precision (technical summary, section 2, "Kwantisatie": the basis
 * in int4, coefficients and centroid in int8).  The pages fix the widths
 * only; the reading used here: symmetric absmax scaling of one vector at a
 * time, in float arithmetic,
 *   scale = max_i |x_i| / Q          (IEEE float division),
 *   code_i = round-half-even(x_i / scale), clamped to [-Q, Q],
 * Q = 127 (int8) or 7 (int4), scale 0 and codes 0 for a zero vector; one
 * vector per centroid, per basis row and per coefficient column (a column
 * holds one basis direction's coordinates over the page's tokens).
 * Dequantised value: scale * code.
 *
 * Layout per unit (block, KV head): mu_q [d] int8; basis_q [r][d/2] bytes,
 * element 2t in the low nibble of byte t and 2t+1 in the high nibble, each a
 * 4-bit two's complement code; coef_q [P][r] int8; scales [1 + 2r] float:
 * the centroid's, then the r basis rows', then the r coefficient columns'. */

/* Quantise n values x[i * stride] (Q = qmax). */
void orc_quantize_vec(int n, int stride, const float* x, int qmax, float* scale, int8_t* code);

/* Quantise every unit of fp32 summary arrays of num_blocks blocks. */
int orc_quantize_pool(int num_blocks, int num_kv_heads, int P, int d, int r, const float* mu,
                      const float* basis, const float* coef, int8_t* mu_q, uint8_t* basis_q,
                      int8_t* coef_q, float* scales);

/* Dequantise into fp32 arrays (scale * code, rounded to float). */
int orc_dequantize_pool(int num_blocks, int num_kv_heads, int P, int d, int r,
                        const int8_t* mu_q, const uint8_t* basis_q, const int8_t* coef_q,
                        const float* scales, float* mu, float* basis, float* coef);

#ifdef __cplusplus
}
#endif
#endif
