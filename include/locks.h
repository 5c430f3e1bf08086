/*
 * locks.h - C ABI of the MI355X (gfx950) library for the decode-step hot
 * path of page-local key summaries (LOCKS, "Page-Local Compact Key Summaries
 * for Efficient Long-Context Decoding", arXiv 2607.24555).
 *
 * The decode step has three parts, each an entry point here:
 *   1. locks_build_summaries - a rank-r spectral summary per finished page:
 *      centroid, top-r eigenvectors of the centred keys, per-token
 *      coefficients (gist.science technical summary, section 2, subsection
 *      Pagina-lokale Spectrale Decompositie);
 *   2. locks_select - scan every summary, reconstruct within-page logits and
 *      take their log-sum-exp as the page's estimated attention mass, share
 *      one page table per GQA group, keep the top pages within a token
 *      budget; it reads no key or value (same section, subsections
 *      Reconstructie en Selectie and Group-Shared Selection; English
 *      abstract on the insight.aitobox.com page);
 *   3. locks_sparse_attend - attention over the selected pages only
 *      (abstract), against the locks_dense_attend baseline (abstract:
 *      latency compared with dense attention).
 * The whole step (2 + 3) can be captured once and replayed as a HIP graph
 * (technical summary, section 2, subsection Implementatie: the decode step
 * runs inside full graphs).
 *
 * Conventions
 *  - All tensor pointers are DEVICE pointers owned by the caller; sizes are
 *    element counts.  The library allocates nothing on the step path and
 *    keeps no state between calls except caller-owned graph handles.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).  Calls
 *    are asynchronous on it and do no host synchronisation, so they can be
 *    captured into a graph.
 *  - Validation happens on the host before any launch; a failed check
 *    returns a status and launches nothing.  Device-side contents (block
 *    table entries, sequence lengths) cannot be checked on the host: kernels
 *    clamp page counts to max_pages and skip block ids outside
 *    [0, num_blocks), so bad contents give wrong values, never a fault.
 *  - Launch failures return LOCKS_ERR_HIP; locks_last_hip_error() gives the
 *    hipError_t of the last failure on the calling thread.
 *  - Page indices returned by selection are LOGICAL page numbers j within a
 *    sequence (page j holds tokens [jP, jP + P)); the block table maps them
 *    to physical blocks.
 *  - Only full pages (j < seq_len / P) whose summaries exist compete for the
 *    budget: all of them, or the first summarized[b] when the page table
 *    carries that count.  The partial last page, and any full page whose
 *    summary is still being built, is always attended, outside the budget
 *    (technical summary, section 2: summaries are made once a page is final,
 *    off the attention's critical path).
 *
 * Layouts (row-major, innermost last)
 *   q            [B][H_q][d]             float32, one decode query per head
 *   K pool       [NB][H_kv][P][d]        bf16 or float32 (keys of a page contiguous)
 *   V pool       [NB][H_kv][d][P]        bf16 or float32 (each page stored transposed)
 *   block_table  [B][max_pages]          int32, logical page -> physical block
 *   seq_lens     [B]                     int32 tokens per sequence
 *   mu           [NB][H_kv][d]           float32 page centroid
 *   basis        [NB][H_kv][r][d]        float32, row k = k-th eigenvector
 *   coef         [NB][H_kv][P][r]        float32, coef[i][k] = basis_k . (k_i - mu)
 *   page_logmass [B][H_kv][max_pages]    float32 group log-mass, -inf if not a full page
 *   sel_pages    [B][H_kv][width]        int32 ascending logical pages, -1 padded
 *   sel_logmass  [B][H_kv][width]        float32 their log-masses, -inf padded
 *   out          [B][H_q][d]             cache dtype (bf16 rounded to nearest even)
 *   out_lse      [B][H_q]                float32 natural-log LSE of the attended logits
 * Query head h reads KV head g = h / (H_q / H_kv).  Logits are q.k / sqrt(d).
 *
 * Supported shapes (others return LOCKS_ERR_UNSUPPORTED):
 *   P in {16, 64}; d in {64, 128}; 1 <= r <= min(P, d, 16);
 *   G = H_q / H_kv in 1..16; max_pages <= 32768;
 *   bf16 caches need P = 64; float32 caches any supported P.
 */
#ifndef LOCKS_H
#define LOCKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LOCKS_OK = 0,
    LOCKS_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shapes */
    LOCKS_ERR_UNSUPPORTED = 2, /* valid but not instantiated (see supported shapes) */
    LOCKS_ERR_WORKSPACE = 3,   /* workspace missing or smaller than locks_workspace_bytes() */
    LOCKS_ERR_HIP = 4          /* a HIP call failed; see locks_last_hip_error() */
} locks_status;

/* Element types.  LOCKS_Q8Q4 is for summaries only (see locks_summaries). */
typedef enum { LOCKS_F32 = 0, LOCKS_BF16 = 1, LOCKS_Q8Q4 = 2 } locks_dtype;

/* How the heads of a GQA group are combined into one page score
 * (technical summary, section 2, Group-Shared Selection).  LSE: the log of
 * the sum of the heads' estimated masses.  MEAN_SHARE: the log of the mean
 * over the heads of each head's share of its own total estimated mass. */
typedef enum { LOCKS_AGG_LSE = 0, LOCKS_AGG_MEAN_SHARE = 1 } locks_agg;

/* Operations for locks_workspace_bytes(). */
typedef enum {
    LOCKS_OP_BUILD = 0,
    LOCKS_OP_SELECT = 1,
    LOCKS_OP_SPARSE_ATTEND = 2,
    LOCKS_OP_DENSE_ATTEND = 3,
    LOCKS_OP_STEP = 4 /* select + sparse attend, as captured by locks_step_graph_create */
} locks_op;

/* Paged K/V cache of one layer.  v may be NULL for locks_build_summaries. */
typedef struct {
    int32_t dtype; /* locks_dtype of both pools */
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t page_size;
    int32_t head_dim;
    const void* k; /* [NB][H_kv][P][d] */
    const void* v; /* [NB][H_kv][d][P] */
} locks_kv_cache;

/* Resident summaries of one layer, stored by physical block (technical
 * summary, section 2, Kwantisatie: the pages keep the summary at reduced
 * precision, the basis in int4 and coefficients and centroid in int8).
 *   LOCKS_F32   fp32 values; scales unused (may be NULL).
 *   LOCKS_BF16  each value is the fp32 summary rounded to the nearest bf16
 *               (ties to even); scales unused.
 *   LOCKS_Q8Q4  integer codes with fp32 scales, per unit (block, KV head):
 *               mu int8 [d]; basis int4 [r][d/2] bytes, element 2t in the
 *               low nibble of byte t and 2t+1 in the high nibble (4-bit two's
 *               complement); coef int8 [P][r]; scales fp32 [1 + 2r] = the
 *               centroid's, the r basis rows', the r coefficient columns'.
 *               A vector's scale is max|x| / Q (IEEE float division, Q = 127
 *               for int8, 7 for int4), its codes round-half-even(x / scale)
 *               clamped to [-Q, Q] (scale 0 and codes 0 for a zero vector);
 *               the value a code stands for is scale * code.  1220 bytes per
 *               unit at P 64, d 128, r 8 (fp32: 6656).
 * Arrays of any size the device holds are accepted: the scan addresses
 * them with 32-bit byte offsets while every array spans less than 4 GiB and
 * with 64-bit offsets beyond. */
typedef struct {
    int32_t dtype; /* locks_dtype of mu, basis and coef */
    int32_t num_blocks;
    int32_t num_kv_heads;
    int32_t page_size;
    int32_t head_dim;
    int32_t rank;
    void* mu;     /* [NB][H_kv][d] (int8 codes for LOCKS_Q8Q4) */
    void* basis;  /* [NB][H_kv][r][d] (LOCKS_Q8Q4: [NB][H_kv][r][d/2] bytes) */
    void* coef;   /* [NB][H_kv][P][r] */
    float* scales; /* LOCKS_Q8Q4: [NB][H_kv][1 + 2r]; otherwise unused */
} locks_summaries;

/* Block table of a batch of sequences.  summarized (nullable, device [B]):
 * how many leading pages of each sequence have their summaries built; pages
 * j < min(summarized[b], seq_lens[b] / P) compete for the budget, pages from
 * there to the end are attended outside it.  NULL: every full page has its
 * summary.  locks_refresh_summaries advances it. */
typedef struct {
    int32_t batch;
    int32_t max_pages;
    const int32_t* block_table; /* [B][max_pages] */
    const int32_t* seq_lens;    /* [B] */
    int32_t* summarized;        /* [B] or NULL */
} locks_page_table;

/* Bytes of workspace an operation needs for these shapes (0 if none).
 * k_pages is the selection width floor(budget_tokens / page_size). */
size_t locks_workspace_bytes(int32_t op, int32_t batch, int32_t max_pages, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t page_size, int32_t head_dim,
                             int32_t rank, int32_t k_pages);

/*
 * Step 1 - build the summary of every full page j with
 * page_begin[b] <= j < seq_lens[b] / P, for every KV head
 * (technical summary, section 2, Pagina-lokale Spectrale Decompositie: a
 * small eigendecomposition of the page's centred keys when the page is
 * final; the summary keeps the top-r eigenvectors and each token's
 * coefficients).  Per (page, KV head): mu = mean key; Kc = K - 1 mu^T;
 * the top-r eigenpairs (lambda_k, u_k) of the P x P Gram Kc Kc^T;
 * basis_k = Kc^T u_k / sqrt(lambda_k); coef[i][k] = sqrt(lambda_k) u_k[i].
 * Eigenvalues below 3e-6 * lambda_max give zero basis/coef (numerically null).
 * The top-r rows are then refined by two steps of subspace iteration applied
 * through Kc (V^T <- Kc^T (Kc V^T), re-orthonormalised), which brings the
 * rank-r subspace close to the accuracy of an SVD of Kc in fp32.
 * page_begin: device [B] or NULL (= all full pages).  Summaries of other
 * blocks are left untouched.  summaries->rank is r.  Computed in fp32 and
 * stored in out->dtype (bf16: rounded to nearest even; Q8Q4: the fp32
 * summary's codes and scales, exactly as locks_quantize_summaries makes
 * them).  Needs no workspace (ws may be NULL).
 */
locks_status locks_build_summaries(const locks_kv_cache* cache, const locks_page_table* pages,
                                   const int32_t* page_begin, const locks_summaries* out,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * Step 1 for pages that became final since the last step (technical summary,
 * section 2: a page's summary is made when the page is final, off the
 * attention's critical path): the same summaries as locks_build_summaries,
 * for the pages page_begin[b] <= j < min(page_begin[b] + max_new_pages,
 * seq_lens[b] / P) only, with a launch sized by max_new_pages (not by
 * max_pages).  page_begin: device [B], required.  When pages->summarized is
 * set, a second launch on the same stream then advances summarized[b] to the
 * end of that range (when summarized[b] >= page_begin[b], i.e. no gap).
 * Intended use: run it on a side stream once a step's token completes a
 * page, with page_begin[b] = summarized[b]; steps launched meanwhile attend
 * the new page outside the budget, and later steps see it as a candidate.
 * A step that reads summarized[b] while this call runs sees the old or the
 * new count; either is a valid state (the count advances only after the
 * summaries are written).
 */
locks_status locks_refresh_summaries(const locks_kv_cache* cache, const locks_page_table* pages,
                                     const int32_t* page_begin, int32_t max_new_pages,
                                     const locks_summaries* out, void* stream);

/*
 * Ablation baseline, not the method: the shared-basis sketch (technical
 * summary, section 3, the proposition that a query-independent projection
 * shared by every page is blind to page-specific directions; the abstract
 * contrasts page-local summaries with fixed sketches).  Given one rank-rho
 * basis per KV head, shared_basis [H_kv][rho][d] fp32 device (orthonormal
 * rows; how it is chosen is the caller's: the ablation uses the top
 * eigenvectors of the pooled within-page key covariance), every full page j
 * >= page_begin[b] (NULL: all) gets mu = its mean key and coef[i][k] =
 * (k_i - mu) . shared_basis[g][k]; out (LOCKS_F32, rank = rho) receives mu,
 * coef and the shared basis copied to each block, so locks_select scores it
 * with the same estimator.  At rho = r (1 + d / P) a page stores as many
 * values (mu + P rho) as a rank-r page summary.
 */
locks_status locks_build_sketch_summaries(const locks_kv_cache* cache,
                                          const locks_page_table* pages,
                                          const int32_t* page_begin, const float* shared_basis,
                                          const locks_summaries* out, void* stream);

/*
 * Quantise fp32 summaries into LOCKS_Q8Q4 codes and scales (technical
 * summary, section 2, Kwantisatie; the quantiser is the one described at
 * locks_summaries), for every unit (block, KV head) of the pools.
 * src: dtype LOCKS_F32; dst: dtype LOCKS_Q8Q4 with the same num_blocks,
 * num_kv_heads, page_size, head_dim and rank.  Device pointers; the caller
 * owns both.  LOCKS_ERR_INVALID_ARG on mismatched shapes or dtypes.
 */
locks_status locks_quantize_summaries(const locks_summaries* src, const locks_summaries* dst,
                                      void* stream);

/*
 * Step 2 - score every full page from its summary alone and select the top
 * pages per (sequence, KV group).  For each head h of group g:
 *   t = V_j^T q_h, beta = q_h . mu_j,
 *   s_hat_{j,h} = log sum_i exp((beta + t . c_i) / sqrt(d))
 * (technical summary, section 2, Reconstructie en Selectie, the displayed
 * estimator; the LSE of the reconstructed logits is the page's mass).
 * Group score, one shared selection per GQA group (section 2, Group-Shared
 * Selection), by agg: LOCKS_AGG_LSE a_{j,g} = log sum_{h in g} exp(s_hat_{j,h})
 * (the sum of the heads' unnormalised masses); LOCKS_AGG_MEAN_SHARE
 * a_{j,g} = log (1/G) sum_{h in g} exp(s_hat_{j,h} - Z_h), Z_h = log sum over
 * the full pages j' of exp(s_hat_{j',h}) (the heads' mean mass share).
 * Selection: k_b = min(floor(budget_tokens / P), full pages of b) pages
 * with the largest a (equal fp32 values: lowest j first), written in
 * ascending j to sel_pages / sel_logmass rows of width floor(budget/P),
 * padded with -1 / -inf.  No K or V pointer is taken: selection reads no
 * candidate key or value (abstract).
 * page_logmass: optional device [B][H_kv][max_pages] output (NULL: the
 * workspace holds it).  Workspace: locks_workspace_bytes(LOCKS_OP_SELECT,..);
 * it also receives the run maxima (see locks_scan) that let the top-k read
 * only the runs able to hold a winner.  A workspace is required unless
 * page_logmass is given (then, without one, the top-k reads every mass).
 */
locks_status locks_select(const float* q, int32_t num_q_heads, const locks_summaries* summaries,
                          const locks_page_table* pages, int32_t budget_tokens, int32_t agg,
                          int32_t* sel_pages, float* sel_logmass, float* page_logmass, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * locks_select without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and rules as
 * locks_select; the selection workspace (page masses unless page_logmass is
 * given, run maxima, per-head estimates and totals) lives in a static device
 * array of 16 MiB that the library holds on each device it runs on until the
 * process ends.  Shapes whose workspace,
 * locks_workspace_bytes(LOCKS_OP_SELECT, ...), exceeds 16 MiB return
 * LOCKS_ERR_WORKSPACE and launch nothing (for example B * max_pages *
 * (H_kv + H_q) floats above ~4M).  Allocates nothing: no hipMalloc, no
 * hipFree.  The first call on a device looks up that device's array
 * (hipGetSymbolAddress); make it before any stream capture.  Every call on
 * one device shares that device's array, which keeps the last call's
 * contents: calls that overlap on one device (concurrent streams, or
 * threads) race and give undefined results.
 */
locks_status locks_select_noalloc(const float* q, int32_t num_q_heads,
                                  const locks_summaries* summaries, const locks_page_table* pages,
                                  int32_t budget_tokens, int32_t agg, int32_t* sel_pages,
                                  float* sel_logmass, float* page_logmass, void* stream);

/*
 * Step 2 alone: the page masses without selection (same definitions as
 * locks_select).  page_logmass [B][H_kv][max_pages] is required;
 * head_logmass [B][H_q][max_pages] (per-head s_hat) is optional.
 * Entries of pages that are not full, or past max_pages' valid range, are -inf.
 * run_max (optional) [B][H_kv][ceil(max_pages / LOCKS_RUN_PAGES)]: entry r is
 * the largest page_logmass value of pages r*LOCKS_RUN_PAGES ..
 * (r+1)*LOCKS_RUN_PAGES - 1 (exactly one of those fp32 values; -inf when
 * none is a full page).  An index for locks_topk, not part of the method.
 */
#define LOCKS_RUN_PAGES 16
locks_status locks_scan(const float* q, int32_t num_q_heads, const locks_summaries* summaries,
                        const locks_page_table* pages, float* page_logmass, float* head_logmass,
                        float* run_max, void* stream);

/*
 * Step 2's selection alone, from given group masses page_logmass
 * [B][H_kv][max_pages] (only entries j < seq_lens[b] / P are read), with the
 * rule of locks_select.  width = row width of sel_pages / sel_logmass.
 * run_max (optional): the run maxima of these masses as locks_scan writes
 * them; with them the kernel reads only the runs whose maximum reaches a
 * lower bound of the k-th largest mass.  Maxima that do not match the
 * masses give an unspecified selection.
 */
locks_status locks_topk(const float* page_logmass, const locks_page_table* pages,
                        int32_t num_kv_heads, int32_t page_size, int32_t budget_tokens,
                        int32_t width, int32_t* sel_pages, float* sel_logmass,
                        const float* run_max, void* stream);

/*
 * The LOCKS_AGG_MEAN_SHARE group score alone, from per-head estimates
 * head_logmass [B][H_q][max_pages] (as locks_scan writes them; entries of
 * pages that are not full are ignored): page_logmass [B][H_kv][max_pages]
 * gets a_{j,g} of locks_select's MEAN_SHARE rule (-inf for pages that are
 * not full); run_max (optional) the run maxima of those scores as
 * locks_scan defines them.  Workspace: B * H_q floats (the totals Z_h),
 * locks_workspace_bytes(LOCKS_OP_SELECT, ...) suffices.
 */
locks_status locks_mean_share(const float* head_logmass, int32_t num_q_heads,
                              int32_t num_kv_heads, const locks_page_table* pages,
                              int32_t page_size, float* page_logmass, float* run_max, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * Step 3 - attention of every query head over the tokens of its group's
 * selected pages plus the sequence's partial last page (abstract: only the
 * top pages are attended).  The softmax is renormalised over exactly these
 * tokens.  sel_pages [B][H_kv][k_pages] as written by locks_select (-1 and
 * indices that are not full pages are ignored).  Split-K: one partial
 * (max, sum, output) per selected page (few pages) or per run of selected
 * pages (many), merged by log-sum-exp in page-list order (the two differ
 * only by rounding).  out: cache dtype; out_lse optional.  A sequence with
 * no token to attend (length 0) gets a zero output and out_lse -inf.
 * Workspace: locks_workspace_bytes(LOCKS_OP_SPARSE_ATTEND, ...).
 */
locks_status locks_sparse_attend(const float* q, int32_t num_q_heads, const locks_kv_cache* cache,
                                 const locks_page_table* pages, const int32_t* sel_pages,
                                 int32_t k_pages, void* out, float* out_lse, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * Baseline - the same attention over every token of every sequence (the
 * dense attention the pages compare decode latency against; abstract).
 * A length-0 sequence gets a zero output and out_lse -inf.
 * Workspace: locks_workspace_bytes(LOCKS_OP_DENSE_ATTEND, ...).
 */
locks_status locks_dense_attend(const float* q, int32_t num_q_heads, const locks_kv_cache* cache,
                                const locks_page_table* pages, void* out, float* out_lse,
                                void* ws, size_t ws_bytes, void* stream);

/* Everything one decode step needs (select + sparse attend). */
typedef struct {
    const float* q;
    int32_t num_q_heads;
    int32_t budget_tokens;
    int32_t agg;          /* locks_agg */
    locks_summaries summaries;
    locks_kv_cache cache;
    locks_page_table pages;
    int32_t* sel_pages;   /* [B][H_kv][floor(budget/P)] */
    float* sel_logmass;   /* same shape */
    float* page_logmass;  /* optional [B][H_kv][max_pages] */
    void* out;            /* [B][H_q][d] cache dtype */
    float* out_lse;       /* optional [B][H_q] */
    void* ws;             /* locks_workspace_bytes(LOCKS_OP_STEP, ...) */
    size_t ws_bytes;
} locks_step_args;

typedef struct locks_step_graph locks_step_graph;

/*
 * Capture one decode step (locks_select and locks_sparse_attend, with the
 * argument pointers given; summaries of newly final pages are built outside
 * it, see locks_refresh_summaries) into an instantiated HIP graph (technical
 * summary, section 2, Implementatie: scoring, selection and sparse attention
 * run inside full graphs).  The pointers are baked in: replay reads the
 * current contents of the same buffers.  The executable graph is uploaded to
 * the device before the call returns (the call synchronises with its own
 * capture stream), so its first launch costs what later ones do.  *graph
 * receives a handle owned by the caller.
 */
locks_status locks_step_graph_create(const locks_step_args* args, locks_step_graph** graph);
locks_status locks_step_graph_launch(locks_step_graph* graph, void* stream);
void locks_step_graph_destroy(locks_step_graph* graph);

/*
 * Measurement probes, not part of the decode step.  They give the summary
 * scan's HBM roofline two ceilings measured on the same device with the
 * same build: what a plain streaming read reaches, and what reading exactly
 * the scan's bytes in the scan's access pattern reaches.
 *
 * locks_probe_stream_read: reads the device buffer buf (bytes, a multiple of
 * 16) once, contiguously, with sink_floats / 4 workgroups of 256 threads
 * (sink_floats a multiple of 4, 4 .. 262144); writes sink_floats floats of
 * checksum to the device array sink.
 *
 * locks_probe_summary_read: reads what locks_scan reads for fp32 summaries at
 * P 64, d 128, r 8 (every full page's centroid, basis and coefficients, the
 * queries, the block table and sequence lengths), with the scan's mapping of
 * waves to runs of 16 pages of one (b, g) and its load widths and order,
 * but does none of the scan's arithmetic; writes one float per page to
 * page_out [B][H_kv][max_pages] (-inf for runs with no full page).  Pages of
 * a partly full run that are not full read block 0 instead.  Other dtypes or
 * shapes: LOCKS_ERR_UNSUPPORTED.
 */
locks_status locks_probe_stream_read(const void* buf, size_t bytes, float* sink,
                                     int32_t sink_floats, void* stream);
locks_status locks_probe_summary_read(const float* q, int32_t num_q_heads,
                                      const locks_summaries* summaries,
                                      const locks_page_table* pages, float* page_out,
                                      void* stream);

const char* locks_status_string(int32_t status);
int32_t locks_last_hip_error(void);
/* Library version as major * 10000 + minor * 100 + patch. */
int32_t locks_version(void);

#ifdef __cplusplus
}
#endif
#endif
